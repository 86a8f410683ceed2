"""Seeded random small shapes through every entry point, against the float64 oracle:
sizes that land anywhere relative to the tiles (ragged time tails, channel counts that are
not multiples of 16/32/64/128/256, dilations below, at and beyond L)."""
import numpy as np
import pytest
import torch

import normalisation_dilated_conv1d_amd as dc
import oracle
from normalisation_dilated_conv1d_amd.inputs import groupnorm_inputs, prenorm_inputs

from test_gpu_parity import TOL_BF16, TOL_F32, announce, maxrel, set_form, to_dev

pytestmark = pytest.mark.gpu

RNG = np.random.default_rng(20260101)
BLOCK_SHAPES = [(int(RNG.integers(1, 5)), int(RNG.integers(1, 150)), int(RNG.integers(1, 700)),
                 int(RNG.integers(1, 800))) for _ in range(24)]
# wide layers that take the 512-channel (8-wave) bf16 tile: 256 < C <= 512 and at least one
# workgroup per CU (N * ceil(L / 128) >= 256)
RNG_WIDE = np.random.default_rng(20261202)
WIDE_BF16_SHAPES = []
for _ in range(4):
    n_ = int(RNG_WIDE.integers(1, 3))
    WIDE_BF16_SHAPES.append((n_, int(RNG_WIDE.integers(257, 513)),
                             256 * 128 // n_ + int(RNG_WIDE.integers(0, 3000)),
                             int(RNG_WIDE.integers(1, 3000))))
GN_SHAPES = []
for _ in range(12):
    G = int(RNG.choice([1, 2, 3, 4, 8]))
    GN_SHAPES.append((int(RNG.integers(1, 4)), int(RNG.integers(1, 100)),
                      G * int(RNG.integers(1, 40)), int(RNG.integers(8, 600)), G,
                      int(RNG.integers(0, 4)), int(RNG.integers(1, 4)), bool(RNG.integers(0, 2))))

# shapes the single-launch GN kernel takes (C_in and C_out multiples of 16, channels per
# group dividing 16, T_out <= 1024) or just misses (T_out up to 1100): per-wave windows for
# small dil and pad, one shared window otherwise, the two-launch path past 1024 steps
RNG_GN1 = np.random.default_rng(20261203)
GN1_SHAPES = []
for _ in range(12):
    cpg = int(RNG_GN1.choice([1, 2, 4, 8, 16]))
    C_out = 16 * int(RNG_GN1.integers(1, 9))
    GN1_SHAPES.append((int(RNG_GN1.integers(1, 4)), 16 * int(RNG_GN1.integers(1, 9)), C_out,
                       int(RNG_GN1.integers(8, 1100)), C_out // cpg, int(RNG_GN1.integers(0, 6)),
                       int(RNG_GN1.integers(1, 7)), bool(RNG_GN1.integers(0, 2))))


@pytest.mark.parametrize("N,C,L,d", BLOCK_SHAPES)
@pytest.mark.parametrize("mode", ["eval", "eval_bf16", "train", "external", "eval_winograd",
                                  "train_winograd", "external_winograd"])
def test_random_block(N, C, L, d, mode, monkeypatch):
    """The *_winograd modes run the float32 block through the Winograd kernel
    (DCONV1D_WINOGRAD=1); these shapes are too small for the automatic choice to take it."""
    if mode.endswith("_winograd"):
        monkeypatch.setenv("DCONV1D_WINOGRAD", "1")
        mode = mode[:-len("_winograd")]
    else:
        monkeypatch.delenv("DCONV1D_WINOGRAD", raising=False)
    seed = 90_000 + N * 1000 + C * 7 + L + d
    announce("random block", mode, (N, C, L, d), "seed", seed)
    bf16 = mode == "eval_bf16"
    p = prenorm_inputs(N, C, L, seed, bf16=bf16)
    q = to_dev(p)
    if mode in ("eval", "eval_bf16"):
        fn = dc.prenorm_dconv1d_fwd_bf16 if bf16 else dc.prenorm_dconv1d_fwd
        out = fn(q["x"], q["running_mean"], q["running_var"], q["gamma"], q["beta"], q["eps"],
                 q["W"], q["b"], d)
        ref = oracle.prenorm_block(p["x"], p["running_mean"], p["running_var"], p["gamma"],
                                   p["beta"], p["eps"], p["W"], p["b"], d)
    elif mode == "train":
        if N * L < 2:
            pytest.skip("training mode needs more than one value per channel")
        out = dc.prenorm_dconv1d_fwd_train(q["x"], None, None, q["gamma"], q["beta"], q["eps"],
                                           0.1, q["W"], q["b"], d)
        ref = oracle.prenorm_block_train(p["x"], p["running_mean"], p["running_var"], p["gamma"],
                                         p["beta"], p["eps"], 0.1, p["W"], p["b"], d)[0]
    else:
        xn = (q["x"] * 0.9 + 0.05).contiguous()
        out = dc.relu_dconv1d_residual_fwd(xn, q["W"], q["b"], q["x"], d)
        ref = oracle.relu_conv_residual(xn.cpu(), p["W"], p["b"], p["x"], d)
    torch.cuda.synchronize()
    err = maxrel(out.float().cpu().numpy(), ref)
    assert err <= (TOL_BF16 if bf16 else TOL_F32), err


@pytest.mark.parametrize("N,C,L,d", WIDE_BF16_SHAPES)
def test_random_wide_bf16_block(N, C, L, d):
    seed = 97_000 + N * 1000 + C * 7 + L + d
    announce("random wide bf16 block", (N, C, L, d), "seed", seed)
    p = prenorm_inputs(N, C, L, seed, bf16=True)
    q = to_dev(p)
    out = dc.prenorm_dconv1d_fwd_bf16(q["x"], q["running_mean"], q["running_var"], q["gamma"],
                                      q["beta"], q["eps"], q["W"], q["b"], d)
    torch.cuda.synchronize()
    ref = oracle.prenorm_block(p["x"], p["running_mean"], p["running_var"], p["gamma"],
                               p["beta"], p["eps"], p["W"], p["b"], d)
    err = maxrel(out.float().cpu().numpy(), ref)
    assert err <= TOL_BF16, err


@pytest.mark.parametrize("N,C_in,C_out,T,G,pad,dil,bias", GN_SHAPES + GN1_SHAPES)
@pytest.mark.parametrize("form", ["auto", "three_tap"])
def test_random_groupnorm(N, C_in, C_out, T, G, pad, dil, bias, form, monkeypatch):
    if T + 2 * pad - 2 * dil < 1:
        pytest.skip("empty output")
    set_form(monkeypatch, form)
    seed = 95_000 + N + C_in + C_out + T + G
    announce("random groupnorm", form, (N, C_in, C_out, T, G, pad, dil, bias), "seed", seed)
    p = groupnorm_inputs(N, C_in, C_out, T, seed, with_bias=bias)
    q = to_dev(p)
    out = dc.conv1d_groupnorm_fwd(q["x"], q["W"], q["bias"], q["gamma"], q["beta"], q["eps"], G,
                                  pad, dil)
    torch.cuda.synchronize()
    ref = oracle.conv_groupnorm(p["x"], p["W"], p["bias"], p["gamma"], p["beta"], p["eps"], G,
                                pad, dil)
    err = maxrel(out.cpu().numpy(), ref)
    assert err <= TOL_F32, err
