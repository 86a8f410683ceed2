"""The no-allocation entry point (prenorm_dconv1d_fwd_noalloc) against the regular one,
through the C ABI: two calls in a row on one device (the second with a smaller input, so
it reuses the fixed scratch array the first call filled), each bitwise equal to
prenorm_dconv1d_fwd on the same inputs (the same kernels run) and within the float32 bar
of the oracle. Also: C above the limit is rejected before anything is queued."""
import numpy as np
import pytest
import torch

import normalisation_dilated_conv1d_amd as dc
import oracle
from normalisation_dilated_conv1d_amd.inputs import prenorm_inputs

from test_gpu_parity import TOL_F32, announce, maxrel, to_dev

pytestmark = pytest.mark.gpu


def _args(q):
    return (q["x"], q["running_mean"], q["running_var"], q["gamma"], q["beta"], q["eps"],
            q["W"], q["b"])


def test_noalloc_matches_regular_entry_point_twice():
    cases = [(8, 512, 4096, 128, 60_001),   # the largest C the fixed scratch holds
             (2, 48, 1000, 3, 60_002)]      # smaller: reuses the array the first call left
    for N, C, L, d, seed in cases:
        announce("prenorm_dconv1d_fwd_noalloc", (N, C, L, d), "seed", seed)
        p = prenorm_inputs(N, C, L, seed)
        q = to_dev(p)
        out_na = torch.empty_like(q["x"])
        dc.prenorm_dconv1d_fwd_noalloc(*_args(q), d, out=out_na)
        torch.cuda.synchronize()
        out_reg = dc.prenorm_dconv1d_fwd(*_args(q), d)
        torch.cuda.synchronize()
        err_pair = maxrel(out_na.cpu().numpy(), out_reg.cpu().numpy().astype(np.float64))
        assert err_pair <= TOL_F32, err_pair
        assert torch.equal(out_na, out_reg)
        ref = oracle.prenorm_block(p["x"], p["running_mean"], p["running_var"], p["gamma"],
                                   p["beta"], p["eps"], p["W"], p["b"], d)
        err = maxrel(out_na.cpu().numpy(), ref)
        assert err <= TOL_F32, err


def test_noalloc_rejects_channels_above_limit():
    q = to_dev(prenorm_inputs(1, 513, 64, 60_003))
    out = torch.full_like(q["x"], 7.0)
    with pytest.raises(dc.Dconv1dError) as e:
        dc.prenorm_dconv1d_fwd_noalloc(*_args(q), 2, out=out)
    assert e.value.code == dc.DCONV1D_EINVAL
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)
