"""The float32 block's two conv forms against the float64 oracle: the Winograd F(2,3)
kernel (DCONV1D_WINOGRAD=1: these shapes are too small for the automatic choice to take
it) and, with DCONV1D_WINOGRAD=0, the direct three-tap kernel on the same shapes.
Shapes cover both regular pair-tile layouts (d dividing 32: 64 contiguous outputs per
tile; d a multiple of 32: two 32-step runs d apart), dilations with tiles that cross
super-blocks, ragged super-blocks, L % 4 != 0 (per-element epilogue), odd chunk counts,
two output-channel tiles, d near L, and every entry point that computes the float32
block. The Conv1d + GroupNorm kernel's Winograd form (dilations 1, 2 and 4 with per-wave
windows) is checked the same way at the end."""
import numpy as np
import pytest
import torch

import normalisation_dilated_conv1d_amd as dc
import oracle
from normalisation_dilated_conv1d_amd.inputs import groupnorm_inputs, prenorm_inputs

from test_gpu_parity import TOL_F32, announce, maxrel, oracle_block, oracle_gn, run_block, to_dev

pytestmark = pytest.mark.gpu

WINO_CASES = [
    # (N, C, L, d)
    (1, 1, 6, 1),
    (2, 16, 62, 1),          # L % 4 != 0: per-element epilogue; ragged last tile
    (2, 40, 301, 2),
    (3, 48, 1000, 4),
    (2, 33, 257, 16),
    (2, 64, 128, 32),        # two super-blocks
    (2, 48, 1000, 96),       # a multiple of 32 that is not a power of two (3 tiles/block)
    (2, 48, 1280, 160),
    (2, 300, 700, 64),       # two output-channel tiles, C not a multiple of 32
    (4, 96, 2048, 8),        # 3 K-chunks: the loop ends without a barrier
    (3, 288, 4100, 128),     # 9 K-chunks, two channel tiles, ragged length
    (2, 32, 4096, 2048),     # d = L/2: one super-block
    # dilations neither dividing 32 nor multiples of it: tiles cross super-blocks, and the
    # epilogue is per element
    (2, 40, 300, 17),
    (3, 48, 1000, 100),
    (2, 33, 257, 24),
    (2, 64, 1000, 127),
    (3, 288, 4100, 77),
    (2, 32, 4096, 683),      # three super-blocks
    (1, 16, 1000, 250),      # two super-blocks
]


@pytest.mark.parametrize("N,C,L,d", WINO_CASES)
def test_winograd_matches_oracle_and_direct(N, C, L, d, monkeypatch):
    monkeypatch.setenv("DCONV1D_WINOGRAD", "1")
    assert dc.dconv1d_block_method(N, C, L, d) == dc.DCONV1D_METHOD_WINOGRAD
    seed = 50_000 + N * 7 + C * 13 + L + d
    announce("prenorm_dconv1d_fwd winograd", (N, C, L, d), "seed", seed)
    p = prenorm_inputs(N, C, L, seed)
    ref = oracle_block(p, d)
    wino = run_block(p, d).cpu().numpy()
    err_w = maxrel(wino, ref)
    monkeypatch.setenv("DCONV1D_WINOGRAD", "0")
    assert dc.dconv1d_block_method(N, C, L, d) == dc.DCONV1D_METHOD_DIRECT
    direct = run_block(p, d).cpu().numpy()
    err_d = maxrel(direct, ref)
    announce(f"   max rel err winograd {err_w:.2e}, direct {err_d:.2e}")
    assert err_w <= TOL_F32, err_w
    assert err_d <= TOL_F32, err_d


def test_winograd_deterministic_and_grid_invariant(monkeypatch):
    """Two calls give the same bits, and a sample computed alone gives the same bits as
    inside a batch (the per-output accumulation order does not depend on the grid)."""
    monkeypatch.setenv("DCONV1D_WINOGRAD", "1")
    N, C, L, d = 6, 96, 1024, 64
    announce("prenorm_dconv1d_fwd winograd bits", (N, C, L, d))
    p = prenorm_inputs(N, C, L, 61)
    a = run_block(p, d).cpu()
    b = run_block(p, d).cpu()
    assert torch.equal(a, b)
    one = {k: (v[2:3].contiguous() if k == "x" else v) for k, v in p.items()}
    alone = run_block(one, d).cpu()
    assert torch.equal(alone[0], a[2])


def test_winograd_negative_infinity_in_last_channel(monkeypatch):
    """-inf at some steps of the last input channel (C not a multiple of 32, so the padded
    channels read that row): ReLU(BN(-inf)) is 0 with a positive scale, so only the
    residual itself is non-finite, as in the direct kernel."""
    monkeypatch.setenv("DCONV1D_WINOGRAD", "1")
    N, C, L, d = 2, 40, 300, 4
    announce("prenorm block winograd -inf in last channel", (N, C, L, d))
    p = prenorm_inputs(N, C, L, 63)
    p["gamma"][C - 1] = p["gamma"][C - 1].abs() + 0.5
    p["x"][:, C - 1, 10:40:3] = float("-inf")
    got = run_block(p, d).cpu().numpy().astype(np.float64)
    ref = oracle_block(p, d)
    bad = ~np.isfinite(ref)
    assert bad.sum() == N * len(range(10, 40, 3))
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    assert np.all(np.isfinite(got[~bad]))
    assert maxrel(got[~bad], ref[~bad]) <= TOL_F32


def test_winograd_training_mode_and_caller_normalised(monkeypatch):
    """The training-mode and the caller-normalised entry points take the Winograd form
    too; both against the oracle."""
    monkeypatch.setenv("DCONV1D_WINOGRAD", "1")
    N, C, L, d = 3, 72, 1536, 16
    announce("prenorm_dconv1d_fwd_train / relu_dconv1d_residual_fwd winograd", (N, C, L, d))
    p = prenorm_inputs(N, C, L, 64)
    q = to_dev(p)
    rm, rv = q["running_mean"].clone(), q["running_var"].clone()
    got = dc.prenorm_dconv1d_fwd_train(q["x"], rm, rv, q["gamma"], q["beta"], q["eps"], 0.1,
                                       q["W"], q["b"], d)
    torch.cuda.synchronize()
    mean, var = oracle.batch_stats(p["x"])
    ref = oracle.prenorm_block(p["x"], mean, var, p["gamma"], p["beta"], p["eps"], p["W"],
                               p["b"], d)
    assert maxrel(got.cpu().numpy(), ref) <= TOL_F32
    xn = torch.relu(torch.randn(N, C, L, generator=torch.Generator().manual_seed(65)))
    res = torch.randn(N, C, L, generator=torch.Generator().manual_seed(66))
    got = dc.relu_dconv1d_residual_fwd(xn.cuda(), q["W"], q["b"], res.cuda(), d)
    torch.cuda.synchronize()
    ref = oracle.relu_conv_residual(xn, p["W"], p["b"], res, d)
    assert maxrel(got.cpu().numpy(), ref) <= TOL_F32


def test_automatic_choice(monkeypatch):
    """Without the override, a regular dilation takes the Winograd form on a full grid and
    on a one-sample grid (64-channel tiles), a dilation near L the direct form; all against
    the oracle."""
    monkeypatch.delenv("DCONV1D_WINOGRAD", raising=False)
    for N, C, L, d, method in ((4, 256, 4096, 128, dc.DCONV1D_METHOD_WINOGRAD),
                               (1, 256, 4096, 128, dc.DCONV1D_METHOD_WINOGRAD),
                               (1, 256, 4096, 1500, dc.DCONV1D_METHOD_DIRECT)):
        assert dc.dconv1d_block_method(N, C, L, d) == method
        announce("prenorm_dconv1d_fwd automatic", (N, C, L, d), "method", method)
        p = prenorm_inputs(N, C, L, 67 + N)
        assert maxrel(run_block(p, d).cpu().numpy(), oracle_block(p, d)) <= TOL_F32


GN_WINO_CASES = [
    # (N, C_in, C_out, T, G, padding, dilation)
    (16, 128, 256, 1024, 32, 1, 1),   # the GN workload's layer
    (2, 32, 64, 512, 8, 2, 2),        # dilation 2, window shift 2
    (2, 16, 32, 1008, 4, 4, 4),       # dilation 4, the widest per-wave window
    (2, 16, 32, 1008, 4, 0, 1),       # no padding: T_out = 1006, a pair across the end
    (1, 48, 16, 130, 16, 2, 1),       # two waves, the second with 2 steps; 16 groups
    (3, 64, 128, 255, 8, 1, 1),       # T_out = 255: a pair whose second output is past it
]


@pytest.mark.parametrize("N,C_in,C_out,T,G,pad,dil", GN_WINO_CASES)
def test_groupnorm_winograd_matches_oracle_and_three_tap(N, C_in, C_out, T, G, pad, dil,
                                                         monkeypatch):
    monkeypatch.delenv("DCONV1D_WINOGRAD", raising=False)
    seed = 52_000 + N * 7 + C_in + C_out * 3 + T + dil
    announce("conv1d_groupnorm_fwd winograd", (N, C_in, C_out, T, G, pad, dil), "seed", seed)
    p = groupnorm_inputs(N, C_in, C_out, T, seed, with_bias=True)
    q = to_dev(p)
    ref = oracle_gn(p, G, pad, dil)

    def run():
        o = dc.conv1d_groupnorm_fwd(q["x"], q["W"], q["bias"], q["gamma"], q["beta"], q["eps"],
                                    G, pad, dil)
        torch.cuda.synchronize()
        return o.cpu().numpy()

    assert dc.dconv1d_groupnorm_method(N, C_in, C_out, T, G, pad, dil, x=q["x"], W=q["W"]) == \
        dc.DCONV1D_METHOD_WINOGRAD
    err_w = maxrel(run(), ref)
    monkeypatch.setenv("DCONV1D_WINOGRAD", "0")
    assert dc.dconv1d_groupnorm_method(N, C_in, C_out, T, G, pad, dil, x=q["x"], W=q["W"]) == \
        dc.DCONV1D_METHOD_DIRECT
    err_d = maxrel(run(), ref)
    announce(f"   max rel err winograd {err_w:.2e}, three-tap {err_d:.2e}")
    assert err_w <= TOL_F32, err_w
    assert err_d <= TOL_F32, err_d


def test_groupnorm_w_not_16_byte_aligned_takes_three_taps(monkeypatch):
    """The Winograd form loads a lane's twelve weights as three 16-byte loads; W only
    8-byte aligned (a view two floats into a buffer) keeps the single-kernel path with
    the three-tap form."""
    monkeypatch.delenv("DCONV1D_WINOGRAD", raising=False)
    N, C_in, C_out, T, G, pad, dil = 2, 32, 64, 512, 8, 1, 1
    announce("conv1d_groupnorm_fwd W 8-byte aligned", (N, C_in, C_out, T, G, pad, dil))
    p = groupnorm_inputs(N, C_in, C_out, T, 52_999, with_bias=True)
    q = to_dev(p)
    buf = torch.empty(q["W"].numel() + 2, device="cuda")
    W = buf[2:].view_as(q["W"])
    W.copy_(q["W"])
    assert W.data_ptr() % 16 == 8
    assert dc.dconv1d_groupnorm_method(N, C_in, C_out, T, G, pad, dil, x=q["x"], W=W) == \
        dc.DCONV1D_METHOD_DIRECT
    out = dc.conv1d_groupnorm_fwd(q["x"], W, q["bias"], q["gamma"], q["beta"], q["eps"], G, pad,
                                  dil)
    torch.cuda.synchronize()
    assert maxrel(out.cpu().numpy(), oracle_gn(p, G, pad, dil)) <= TOL_F32


SMALL_C_CASES = [
    # (N, C, L, d): channel counts below 256 and between multiples of it take 64- and
    # 128-channel tiles in both kernels (a workgroup per CU or more)
    (32, 64, 4096, 128),      # direct 128-step x 64-channel tiles; Winograd 64-channel tiles
    (16, 128, 4096, 128),     # direct 128 x 128; Winograd 128-channel tiles
    (8, 192, 4096, 8),        # three 64-channel tiles
    (4, 320, 2048, 100),      # five 64-channel tiles; per-element Winograd epilogue
]


@pytest.mark.parametrize("N,C,L,d", SMALL_C_CASES)
@pytest.mark.parametrize("form", ["0", "1"])
def test_small_channel_tiles_match_oracle(N, C, L, d, form, monkeypatch):
    monkeypatch.setenv("DCONV1D_WINOGRAD", form)
    seed = 54_000 + N + C + L + d
    announce("prenorm_dconv1d_fwd channel tiles", form, (N, C, L, d), "seed", seed)
    p = prenorm_inputs(N, C, L, seed)
    err = maxrel(run_block(p, d).cpu().numpy(), oracle_block(p, d))
    announce(f"   max rel err {err:.2e}")
    assert err <= TOL_F32, err


GN_TWO_KERNEL_CASES = [
    # (N, C_in, C_out, T, G, padding = dilation): shapes the single kernel does not take
    (4, 64, 128, 2048, 16, 1),        # T_out > 1024
    (2, 40, 96, 333, 12, 1),          # C_in not a multiple of 16, ragged pair tile
    (2, 128, 256, 1024, 8, 1),        # 32 channels per group
    (2, 16, 48, 400, 4, 100),         # 12 channels per group, pairs 100 apart
    (1, 48, 300, 3001, 3, 5),         # C_out 300 (64-channel tiles), irregular dilation
    (2, 32, 64, 2500, 4, 64),         # regular dilation, two 32-step runs per tile
]


@pytest.mark.parametrize("N,C_in,C_out,T,G,d", GN_TWO_KERNEL_CASES)
def test_groupnorm_two_kernel_winograd(N, C_in, C_out, T, G, d, monkeypatch):
    """The two-kernel path's Winograd conv (GroupNorm statistics per pair tile) against
    the oracle and against its three-tap conv."""
    monkeypatch.delenv("DCONV1D_WINOGRAD", raising=False)
    seed = 56_000 + N + C_in + C_out + T + d
    announce("conv1d_groupnorm_fwd two kernels winograd", (N, C_in, C_out, T, G, d), "seed",
             seed)
    p = groupnorm_inputs(N, C_in, C_out, T, seed, with_bias=True)
    q = to_dev(p)
    ref = oracle_gn(p, G, d, d)

    def run():
        o = dc.conv1d_groupnorm_fwd(q["x"], q["W"], q["bias"], q["gamma"], q["beta"], q["eps"],
                                    G, d, d)
        torch.cuda.synchronize()
        return o.cpu().numpy()

    assert dc.dconv1d_groupnorm_method(N, C_in, C_out, T, G, d, d, x=q["x"], W=q["W"]) == \
        dc.DCONV1D_METHOD_WINOGRAD
    err_w = maxrel(run(), ref)
    monkeypatch.setenv("DCONV1D_WINOGRAD", "0")
    err_d = maxrel(run(), ref)
    announce(f"   max rel err winograd {err_w:.2e}, three-tap {err_d:.2e}")
    assert err_w <= TOL_F32, err_w
    assert err_d <= TOL_F32, err_d


STAGING_CASES = [
    # (N, C, L, d): d a multiple of 4 that divides 32 or is a multiple of 32, L % 4 == 0:
    # one 16-byte load per lattice step of four pairs
    (2, 64, 1024, 128),
    (2, 48, 1000, 8),
    (3, 288, 4100, 4),       # two channel tiles, ragged last pair tile
    (2, 40, 2048, 96),       # C_in not a multiple of 32: padded rows in the last chunk
    # d = 1 or 2 (L a multiple of 4): 16-byte loads of the 16 steps around four pairs
    (2, 64, 1024, 1),
    (3, 96, 2052, 2),        # ragged last pair tile
]


def _shifted(t):
    """A copy of t one float into a buffer: 4-byte aligned, never 16-byte aligned."""
    buf = torch.empty(t.numel() + 4, device="cuda", dtype=t.dtype)
    v = buf[1:1 + t.numel()].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 != 0
    return v


@pytest.mark.parametrize("N,C,L,d", STAGING_CASES)
def test_winograd_staging_forms_agree(N, C, L, d, monkeypatch):
    """With x 16-byte aligned the Winograd kernel stages four pairs with 16-byte loads;
    with x one float into a buffer, one pair per 4-byte load. Both stage the same values, so
    the outputs agree bit for bit (the residual, the same x, then takes the per-element
    epilogue, whose sums run in the same order), and both match the oracle."""
    monkeypatch.setenv("DCONV1D_WINOGRAD", "1")
    seed = 57_000 + N + C + L + d
    announce("prenorm_dconv1d_fwd winograd staging forms", (N, C, L, d), "seed", seed)
    p = prenorm_inputs(N, C, L, seed)
    aligned = run_block(p, d).cpu()
    q = to_dev(p)
    shifted = dc.prenorm_dconv1d_fwd(_shifted(q["x"]), q["running_mean"], q["running_var"],
                                     q["gamma"], q["beta"], q["eps"], q["W"], q["b"], d)
    torch.cuda.synchronize()
    assert torch.equal(shifted.cpu(), aligned)
    err = maxrel(aligned.numpy(), oracle_block(p, d))
    announce(f"   max rel err {err:.2e}")
    assert err <= TOL_F32, err


@pytest.mark.parametrize("N,C_in,C_out,T,G,d", [(2, 32, 64, 2048, 8, 4),
                                                (2, 32, 64, 2500, 4, 64),
                                                (2, 32, 64, 2048, 8, 1),
                                                (1, 48, 96, 3000, 12, 2)])
def test_groupnorm_two_kernel_staging_forms_agree(N, C_in, C_out, T, G, d, monkeypatch):
    """The same two staging forms in the two-kernel GroupNorm path's Winograd conv."""
    monkeypatch.setenv("DCONV1D_WINOGRAD", "1")
    seed = 57_500 + N + C_in + C_out + T + d
    announce("conv1d_groupnorm_fwd two kernels staging forms", (N, C_in, C_out, T, G, d),
             "seed", seed)
    p = groupnorm_inputs(N, C_in, C_out, T, seed, with_bias=True)
    q = to_dev(p)
    assert dc.dconv1d_groupnorm_method(N, C_in, C_out, T, G, d, d, x=q["x"], W=q["W"]) == \
        dc.DCONV1D_METHOD_WINOGRAD

    def run(x):
        o = dc.conv1d_groupnorm_fwd(x, q["W"], q["bias"], q["gamma"], q["beta"], q["eps"],
                                    G, d, d)
        torch.cuda.synchronize()
        return o.cpu()

    aligned = run(q["x"])
    assert torch.equal(run(_shifted(q["x"])), aligned)
    err = maxrel(aligned.numpy(), oracle_gn(p, G, d, d))
    announce(f"   max rel err {err:.2e}")
    assert err <= TOL_F32, err
