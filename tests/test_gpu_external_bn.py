"""Block with caller-supplied normalisation (relu_dconv1d_residual_fwd / _bf16) against
the float64 oracle (oracle.relu_conv_residual), through the C ABI.

Bars as for the block: float32 storage 2e-4, bfloat16 storage 2e-2, relative to
1 + |ref|."""
import numpy as np
import pytest
import torch

import normalisation_dilated_conv1d_amd as dc
import oracle
from normalisation_dilated_conv1d_amd.inputs import WORKLOADS, prenorm_inputs, seed_for

from test_gpu_parity import TOL_BF16, TOL_F32, announce, maxrel

pytestmark = pytest.mark.gpu


def ext_inputs(N, C, L, seed, bf16=False):
    """xn: a normalised-looking activation (mean ~0.1, std ~1); residual: the block input;
    W, b as in the block's inputs."""
    p = prenorm_inputs(N, C, L, seed, bf16=bf16)
    g = torch.Generator().manual_seed(seed + 1)
    xn = torch.randn((N, C, L), generator=g) + 0.1
    if bf16:
        xn = xn.to(torch.bfloat16)
    return dict(xn=xn, residual=p["x"], W=p["W"], b=p["b"])


def run_ext(p, d, bf16=False, inplace=False):
    q = {k: v.cuda() for k, v in p.items()}
    fn = dc.relu_dconv1d_residual_fwd_bf16 if bf16 else dc.relu_dconv1d_residual_fwd
    out = q["residual"] if inplace else None
    o = fn(q["xn"], q["W"], q["b"], q["residual"], d, out=out)
    torch.cuda.synchronize()
    return o.float().cpu().numpy()


def oracle_ext(p, d):
    return oracle.relu_conv_residual(p["xn"], p["W"], p["b"], p["residual"], d)


EXT_CASES = [
    # (N, C, L, d)
    (1, 1, 1, 1),
    (1, 3, 7, 2),
    (2, 16, 512, 128),
    (3, 48, 1000, 3),
    (2, 48, 1000, 1000),
    (2, 300, 700, 64),
    (8, 64, 8200, 128),
    (2, 33, 257, 31),
]


@pytest.mark.parametrize("N,C,L,d", EXT_CASES)
def test_external_bn_f32_matches_oracle(N, C, L, d):
    seed = 50_000 + N * 7 + C * 13 + L + d
    announce("relu_dconv1d_residual_fwd", (N, C, L, d), "seed", seed)
    p = ext_inputs(N, C, L, seed)
    err = maxrel(run_ext(p, d), oracle_ext(p, d))
    assert err <= TOL_F32, err


# (4, 512, 8190, 7) and (2, 384, 16384, 64) run the 512-channel (8-wave) bf16 tile, on the
# 2-byte-load and the paired-load path
@pytest.mark.parametrize("N,C,L,d", [(1, 3, 7, 2), (2, 96, 777, 50), (8, 64, 8200, 128),
                                     (4, 512, 8190, 7), (2, 384, 16384, 64)])
def test_external_bn_bf16_matches_oracle(N, C, L, d):
    seed = 60_000 + N + C + L + d
    announce("relu_dconv1d_residual_fwd_bf16", (N, C, L, d), "seed", seed)
    p = ext_inputs(N, C, L, seed, bf16=True)
    err = maxrel(run_ext(p, d, bf16=True), oracle_ext(p, d))
    assert err <= TOL_BF16, err


@pytest.mark.parametrize("bf16,N,C,L,d", [(False, 4, 80, 3000, 40), (True, 4, 80, 3000, 40),
                                          (True, 2, 384, 16384, 64)])
def test_external_bn_inplace_residual(bf16, N, C, L, d):
    """out = residual (the same buffer) gives the out-of-place result (the last case runs
    the 8-wave bf16 tile)."""
    announce("relu_dconv1d_residual in place", (N, C, L, d), "bf16", bf16)
    p = ext_inputs(N, C, L, 50_900 + bf16, bf16=bf16)
    ref = run_ext(p, d, bf16=bf16)
    got = run_ext(p, d, bf16=bf16, inplace=True)
    assert np.array_equal(got, ref)
    err = maxrel(got, oracle_ext(p, d))
    assert err <= (TOL_BF16 if bf16 else TOL_F32), err


def test_external_bn_residual_is_input():
    """residual and xn may be the same tensor."""
    N, C, L, d = 2, 40, 600, 5
    announce("relu_dconv1d_residual residual == xn", (N, C, L, d))
    p = ext_inputs(N, C, L, 50_950)
    xn = p["xn"].cuda()
    o = dc.relu_dconv1d_residual_fwd(xn, p["W"].cuda(), p["b"].cuda(), xn, d)
    torch.cuda.synchronize()
    err = maxrel(o.cpu().numpy(), oracle.relu_conv_residual(p["xn"], p["W"], p["b"], p["xn"], d))
    assert err <= TOL_F32, err


def test_external_bn_after_torch_training_batchnorm():
    """The fallback as used: torch's training-mode BatchNorm on the device, then this call
    with the block input as residual, equals the training-mode block of the oracle."""
    N, C, L, d = 4, 64, 2048, 128
    announce("torch BN(train) + relu_dconv1d_residual", (N, C, L, d))
    p = prenorm_inputs(N, C, L, 50_990)
    x = p["x"].cuda()
    xn = torch.nn.functional.batch_norm(x, p["running_mean"].cuda().clone(),
                                        p["running_var"].cuda().clone(), p["gamma"].cuda(),
                                        p["beta"].cuda(), training=True, momentum=0.1,
                                        eps=p["eps"])
    o = dc.relu_dconv1d_residual_fwd(xn.contiguous(), p["W"].cuda(), p["b"].cuda(), x, d)
    torch.cuda.synchronize()
    ref = oracle.prenorm_block_train(p["x"], p["running_mean"], p["running_var"], p["gamma"],
                                     p["beta"], p["eps"], 0.1, p["W"], p["b"], d)[0]
    err = maxrel(o.cpu().numpy(), ref)
    assert err <= TOL_F32, err


def test_external_bn_workload1_shape_full():
    """N=32, C=256, L=4096, d=128: every output against the oracle."""
    w = WORKLOADS[1].dims
    announce("relu_dconv1d_residual workload-1 shape", w)
    p = ext_inputs(w["N"], w["C"], w["L"], seed_for(1, 7))
    err = maxrel(run_ext(p, w["d"]), oracle_ext(p, w["d"]))
    assert err <= TOL_F32, err
