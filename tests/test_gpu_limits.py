"""Edge sizes through the C ABI against the float64 oracle: the largest per-sample size
the ABI accepts (C*L just under 2^31 elements, C = 16384 channels), very many tiny
samples, length 1, and GroupNorm with 16384 output channels.

The largest shapes are checked on sampled outputs that include every boundary region
(first/last time steps, the edges of the padding, first/last channels); their inputs are
drawn with torch's seeded generator directly in device memory (8.6 GB for x), and the
oracle reads the columns and weight rows it needs from there."""
import numpy as np
import pytest
import torch

import normalisation_dilated_conv1d_amd as dc
import oracle
from normalisation_dilated_conv1d_amd.inputs import groupnorm_inputs, prenorm_inputs

from test_gpu_parity import TOL_BF16, TOL_F32, announce, maxrel

pytestmark = pytest.mark.gpu

C_MAX = 16384


def _device_block_inputs(C, L, seed, bf16):
    g = torch.Generator(device="cuda").manual_seed(seed)
    x = torch.randn((1, C, L), device="cuda", generator=g)
    if bf16:
        x = x.to(torch.bfloat16)
    p = dict(x=x,
             running_mean=torch.rand(C, device="cuda", generator=g) - 0.5,
             running_var=torch.rand(C, device="cuda", generator=g) + 0.5,
             gamma=torch.rand(C, device="cuda", generator=g) + 0.5,
             beta=torch.randn(C, device="cuda", generator=g) * 0.1,
             W=torch.randn((C, C, 3), device="cuda", generator=g) / float(np.sqrt(3 * C)),
             b=torch.randn(C, device="cuda", generator=g) * 0.01,
             eps=1e-5)
    return p


def _boundary_points(C, L, d, count, seed):
    rng = np.random.default_rng(seed)
    ts = sorted({0, 1, d - 1, d, d + 1, L - d - 2, L - d - 1, L - d, L - 2, L - 1, 127, 128,
                 L // 2} & set(range(L)))
    cs = [0, 1, 255, 256, C // 2, C - 2, C - 1]
    pts = [(0, c, t) for t in ts for c in cs[:3]] + [(0, c, int(rng.integers(L))) for c in cs]
    while len(pts) < count:
        pts.append((0, int(rng.integers(C)), int(rng.integers(L))))
    return pts


@pytest.mark.parametrize("bf16,L,d", [(False, 131071, 5), (True, 131070, 6)],
                         ids=["f32_C16384_L131071", "bf16_C16384_L131070"])
def test_block_largest_sample(bf16, L, d):
    """C*L = 2^31 - 16384 (float32) / 2^31 - 32768 (bf16, even L and d: paired loads):
    every per-sample index is as large as the ABI allows."""
    C = C_MAX
    assert C * L < 2 ** 31
    announce("largest sample", "bf16" if bf16 else "f32", (1, C, L, d))
    p = _device_block_inputs(C, L, 70_000 + bf16, bf16)
    fn = dc.prenorm_dconv1d_fwd_bf16 if bf16 else dc.prenorm_dconv1d_fwd
    out = fn(p["x"], p["running_mean"], p["running_var"], p["gamma"], p["beta"], p["eps"],
             p["W"], p["b"], d)
    torch.cuda.synchronize()
    pts = _boundary_points(C, L, d, 96, 7)
    ref = oracle.prenorm_block_points(p["x"], p["running_mean"], p["running_var"], p["gamma"],
                                      p["beta"], p["eps"], p["W"], p["b"], d, pts)
    got = np.array([float(out[n, c, t].float()) for (n, c, t) in pts])
    del out, p
    torch.cuda.empty_cache()
    dc.release()
    err = maxrel(got, ref)
    assert err <= (TOL_BF16 if bf16 else TOL_F32), err


@pytest.mark.parametrize("bf16,L,d", [(False, 2 ** 30 - 1, 2 ** 30 - 4),
                                       (False, 2 ** 30 - 1, 2 ** 30 + 5),
                                       (True, 2 ** 30 - 2, 2 ** 30 - 6)],
                         ids=["f32_d_below_L", "f32_d_above_L", "bf16_d_below_L"])
def test_block_longest_length(bf16, L, d):
    """C = 1 at the longest length the ABI takes (L < 2^30). Tile start + column + tap
    offset then reaches about 2L = 2^31, past the int range, so this checks that the tap
    index is formed without overflow; with d just below L both padded and in-range outer
    taps occur at each end of the sequence (d >= L leaves the centre tap only)."""
    C = 1
    announce("longest length", "bf16" if bf16 else "f32", (1, C, L, d))
    p = _device_block_inputs(C, L, 70_400 + bf16 + (d > L), bf16)
    fn = dc.prenorm_dconv1d_fwd_bf16 if bf16 else dc.prenorm_dconv1d_fwd
    out = fn(p["x"], p["running_mean"], p["running_var"], p["gamma"], p["beta"], p["eps"],
             p["W"], p["b"], d)
    torch.cuda.synchronize()
    rng = np.random.default_rng(9)
    de = min(d, L)
    ts = sorted({0, 1, 2, 3, 4, 5, 127, 128, L // 2, L - de - 1, L - de, L - de + 1,
                 de - 1, de, de + 1, L - 129, L - 128, L - 6, L - 5, L - 4, L - 3, L - 2,
                 L - 1} & set(range(L)))
    pts = [(0, 0, t) for t in ts] + [(0, 0, int(rng.integers(L))) for _ in range(40)]
    ref = oracle.prenorm_block_points(p["x"], p["running_mean"], p["running_var"], p["gamma"],
                                      p["beta"], p["eps"], p["W"], p["b"], d, pts)
    got = np.array([float(out[n, c, t].float()) for (n, c, t) in pts])
    del out, p
    torch.cuda.empty_cache()
    dc.release()
    err = maxrel(got, ref)
    assert err <= (TOL_BF16 if bf16 else TOL_F32), err


def test_block_many_tiny_samples():
    """N = 20000 samples of (3, 5): one workgroup per sample, mostly padding."""
    N, C, L, d = 20000, 3, 5, 2
    announce("many tiny samples", (N, C, L, d))
    p = prenorm_inputs(N, C, L, 70_100)
    q = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    out = dc.prenorm_dconv1d_fwd(q["x"], q["running_mean"], q["running_var"], q["gamma"],
                                 q["beta"], q["eps"], q["W"], q["b"], d)
    torch.cuda.synchronize()
    ref = oracle.prenorm_block(p["x"], p["running_mean"], p["running_var"], p["gamma"],
                               p["beta"], p["eps"], p["W"], p["b"], d)
    err = maxrel(out.cpu().numpy(), ref)
    assert err <= TOL_F32, err


@pytest.mark.parametrize("bf16", [False, True])
def test_block_length_one(bf16):
    """L = 1: both outer taps are padding for any d."""
    N, C, L, d = 7, 300, 1, 3
    announce("length one", (N, C, L, d), "bf16", bf16)
    p = prenorm_inputs(N, C, L, 70_200 + bf16, bf16=bf16)
    q = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    fn = dc.prenorm_dconv1d_fwd_bf16 if bf16 else dc.prenorm_dconv1d_fwd
    out = fn(q["x"], q["running_mean"], q["running_var"], q["gamma"], q["beta"], q["eps"],
             q["W"], q["b"], d)
    torch.cuda.synchronize()
    ref = oracle.prenorm_block(p["x"], p["running_mean"], p["running_var"], p["gamma"],
                               p["beta"], p["eps"], p["W"], p["b"], d)
    err = maxrel(out.float().cpu().numpy(), ref)
    assert err <= (TOL_BF16 if bf16 else TOL_F32), err


def test_groupnorm_max_channels():
    """C_out = 16384 in 8 groups of 2048 channels x 2048 steps: 4M values per group merged
    from 32 time tiles x 2048 channels of partials."""
    N, C_in, C_out, T, G = 1, 64, C_MAX, 2048, 8
    announce("groupnorm max channels", (N, C_in, C_out, T, G))
    p = groupnorm_inputs(N, C_in, C_out, T, 70_300, with_bias=True)
    q = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    out = dc.conv1d_groupnorm_fwd(q["x"], q["W"], q["bias"], q["gamma"], q["beta"], q["eps"], G,
                                  1, 1)
    torch.cuda.synchronize()
    ref = oracle.conv_groupnorm(p["x"], p["W"], p["bias"], p["gamma"], p["beta"], p["eps"], G, 1, 1)
    err = maxrel(out.cpu().numpy(), ref)
    assert err <= TOL_F32, err
