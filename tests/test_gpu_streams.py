"""Calls on different streams of one device share the library's per-device workspace
(repacked weights, folded BN vectors, partial statistics). The library orders them: a
call on another stream than the workspace's previous user waits for that call on the
device. Here two calls with different weights and inputs are queued on two streams
back to back, without any ordering by the caller, and both must match the oracle."""
import pytest
import torch

import normalisation_dilated_conv1d_amd as dc
import oracle
from normalisation_dilated_conv1d_amd.inputs import groupnorm_inputs, prenorm_inputs

from test_gpu_parity import TOL_BF16, TOL_F32, announce, maxrel, to_dev

pytestmark = pytest.mark.gpu


def _block(q, d, bf16=False):
    fn = dc.prenorm_dconv1d_fwd_bf16 if bf16 else dc.prenorm_dconv1d_fwd
    return fn(q["x"], q["running_mean"], q["running_var"], q["gamma"], q["beta"], q["eps"],
              q["W"], q["b"], d)


def _ref(p, d):
    return oracle.prenorm_block(p["x"], p["running_mean"], p["running_var"], p["gamma"],
                                p["beta"], p["eps"], p["W"], p["b"], d)


@pytest.mark.parametrize("second", ["f32", "bf16", "gn"])
def test_two_streams_unordered(second):
    """A long call (N=32, C=256, L=4096, about half a millisecond on the GPU) on one
    stream, then a short call with other weights on a second stream right away: without
    the library's ordering the second call's weight repack would overwrite the first
    call's weights while its conv kernel still reads them."""
    announce("two streams", "first f32 (32, 256, 4096, 128), second", second)
    pa = prenorm_inputs(32, 256, 4096, 50_001)
    qa = to_dev(pa)
    if second == "gn":
        pb = groupnorm_inputs(4, 64, 128, 2048, 50_002, with_bias=True)   # two-launch path
    else:
        pb = prenorm_inputs(2, 256, 4096, 50_002, bf16=(second == "bf16"))
    qb = to_dev(pb)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        out_a = _block(qa, 128)
    with torch.cuda.stream(s2):
        if second == "gn":
            out_b = dc.conv1d_groupnorm_fwd(qb["x"], qb["W"], qb["bias"], qb["gamma"],
                                            qb["beta"], qb["eps"], 16, 1, 1)
        else:
            out_b = _block(qb, 5, bf16=(second == "bf16"))
    torch.cuda.synchronize()
    err_a = maxrel(out_a.cpu().numpy(), _ref(pa, 128))
    if second == "gn":
        ref_b = oracle.conv_groupnorm(pb["x"], pb["W"], pb["bias"], pb["gamma"], pb["beta"],
                                      pb["eps"], 16, 1, 1)
        err_b, tol_b = maxrel(out_b.cpu().numpy(), ref_b), TOL_F32
    else:
        err_b = maxrel(out_b.float().cpu().numpy(), _ref(pb, 5))
        tol_b = TOL_BF16 if second == "bf16" else TOL_F32
    assert err_a <= TOL_F32, ("first call", err_a)
    assert err_b <= tol_b, ("second call", err_b)


def test_alternating_streams_many_calls():
    """Six calls with three different weight sets, alternating over three streams and
    queued without waiting: every output matches its own oracle result."""
    announce("alternating streams, 6 calls")
    ps = [prenorm_inputs(8, 128, 2048, 50_100 + i) for i in range(3)]
    qs = [to_dev(p) for p in ps]
    refs = [_ref(p, 64) for p in ps]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(3)]
    outs = []
    for i in range(6):
        with torch.cuda.stream(streams[i % 3]):
            outs.append((i % 3, _block(qs[(i * 2) % 3], 64)))
    torch.cuda.synchronize()
    for i, (_, o) in enumerate(outs):
        err = maxrel(o.cpu().numpy(), refs[(i * 2) % 3])
        assert err <= TOL_F32, (i, err)
