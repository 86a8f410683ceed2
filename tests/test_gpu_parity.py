"""HIP path against the float64 CPU oracle, element by element, through the C ABI.

Bars: float32 storage max |gpu - ref| / (1 + |ref|) <= 2e-4; bfloat16 storage <= 2e-2.
Sizes span several tiles, ragged tails, multiple output-channel tiles, every dilation
regime (contiguous taps to taps entirely in the padding) and the five benchmark
workloads, each compared on every output."""
import sys

import numpy as np
import pytest
import torch

import normalisation_dilated_conv1d_amd as dc
import oracle
from normalisation_dilated_conv1d_amd.inputs import (WORKLOADS, groupnorm_inputs,
                                                      prenorm_inputs, seed_for)

pytestmark = pytest.mark.gpu

TOL_F32 = 2e-4
TOL_BF16 = 2e-2


def announce(*parts):
    print("[gpu-case]", *parts, file=sys.stderr, flush=True)


def to_dev(p):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in p.items()}


def maxrel(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    assert np.all(np.isfinite(got)), "non-finite output"
    return float(np.max(np.abs(got - ref) / (1.0 + np.abs(ref))))


def run_block(p, d, bf16=False, out=None):
    q = to_dev(p)
    fn = dc.prenorm_dconv1d_fwd_bf16 if bf16 else dc.prenorm_dconv1d_fwd
    o = fn(q["x"], q["running_mean"], q["running_var"], q["gamma"], q["beta"], q["eps"], q["W"],
           q["b"], d, out=out)
    torch.cuda.synchronize()
    return o


def oracle_block(p, d):
    return oracle.prenorm_block(p["x"], p["running_mean"], p["running_var"], p["gamma"],
                                p["beta"], p["eps"], p["W"], p["b"], d)


# ----------------------------------------------------------------- small and medium shapes

BLOCK_CASES = [
    # (N, C, L, d)
    (1, 1, 1, 1),
    (1, 3, 7, 2),
    (2, 16, 512, 128),       # the tiny workload's shape
    (3, 48, 1000, 1),
    (3, 48, 1000, 3),
    (3, 48, 1000, 100),
    (3, 48, 1000, 127),
    (3, 48, 1000, 129),
    (2, 48, 1000, 999),
    (2, 48, 1000, 1000),     # d = L: only the centre tap
    (2, 48, 1000, 5000),     # d > L
    (2, 300, 700, 64),       # two output-channel tiles, C not a multiple of 32
    (5, 256, 130, 7),
    (8, 64, 8200, 128),      # 128-wide time tiles with a ragged tail
    (2, 33, 257, 31),
    (8, 64, 5000, 77),       # 64-step x 256-channel tiles
    # odd chunk counts (C_in padded to 32 or 96: 3 or 9 chunks) with L % 4 == 0, where the
    # main loop ends without a barrier before the LDS-transposed epilogue
    (4, 96, 2048, 3),
    (6, 32, 4096, 64),
    (3, 16, 1024, 5),
]


@pytest.mark.parametrize("N,C,L,d", BLOCK_CASES)
def test_block_f32_matches_oracle(N, C, L, d):
    seed = 10_000 + N * 7 + C * 13 + L + d
    announce("prenorm_dconv1d_fwd", (N, C, L, d), "seed", seed)
    p = prenorm_inputs(N, C, L, seed)
    got = run_block(p, d).cpu().numpy()
    err = maxrel(got, oracle_block(p, d))
    assert err <= TOL_F32, err


# The last five run the 512-channel (8-wave) bf16 tile, which wide layers get when the
# grid still has a workgroup per CU: C=384 padded to 512 on the paired-load path; C=512
# with an odd dilation on the 2-byte-load path; C=300 with a 2-step ragged last tile
# (per-element epilogue); C=320 with L a multiple of 8 (16-byte epilogue); and an odd L.
BF16_CASES = [(1, 3, 7, 2), (2, 96, 777, 50), (8, 64, 8200, 128), (2, 300, 300, 300),
              (2, 16, 512, 128), (2, 384, 16384, 128), (4, 512, 8190, 7),
              (1, 300, 32770, 2), (1, 320, 32768, 130), (2, 288, 16383, 5)]


@pytest.mark.parametrize("N,C,L,d", BF16_CASES)
def test_block_bf16_matches_oracle(N, C, L, d):
    seed = 20_000 + N + C + L + d
    announce("prenorm_dconv1d_fwd_bf16", (N, C, L, d), "seed", seed)
    p = prenorm_inputs(N, C, L, seed, bf16=True)
    got = run_block(p, d, bf16=True).float().cpu().numpy()
    err = maxrel(got, oracle_block(p, d))
    assert err <= TOL_BF16, err


def test_block_padding_trap():
    """mean 0, gamma 1, beta +5: ReLU(BN(0)) = 5; padded taps must still be exactly 0."""
    N, C, L, d = 2, 64, 600, 100
    announce("prenorm_dconv1d_fwd padding trap", (N, C, L, d))
    p = prenorm_inputs(N, C, L, 31)
    p["running_mean"] = torch.zeros(C)
    p["running_var"] = torch.ones(C)
    p["gamma"] = torch.ones(C)
    p["beta"] = torch.full((C,), 5.0)
    got = run_block(p, d).cpu().numpy()
    err = maxrel(got, oracle_block(p, d))
    assert err <= TOL_F32, err


@pytest.mark.parametrize("bf16", [False, True])
def test_block_negative_infinity_in_last_channel(bf16):
    """x = -inf at some steps of the last input channel, C_in not a multiple of the
    kernels' 32-channel K-chunks (the padded channels then read that row): ReLU(BN(-inf))
    is 0 with a positive scale, so every output is finite except the residual itself."""
    N, C, L, d = 2, 40, 300, 3
    announce("prenorm block -inf in last channel", (N, C, L, d), "bf16", bf16)
    p = prenorm_inputs(N, C, L, 33, bf16=bf16)
    p["gamma"][C - 1] = p["gamma"][C - 1].abs() + 0.5
    p["x"][:, C - 1, 10:40:3] = float("-inf")
    got = run_block(p, d, bf16=bf16).float().cpu().numpy().astype(np.float64)
    ref = oracle_block(p, d)
    bad = ~np.isfinite(ref)
    assert bad.sum() == N * len(range(10, 40, 3))
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    assert np.all(np.isfinite(got[~bad]))
    err = maxrel(got[~bad], ref[~bad])
    assert err <= (TOL_BF16 if bf16 else TOL_F32), err


def test_block_zero_weights_exact():
    """W = 0: out = x + b, exactly (one float32 add)."""
    N, C, L, d = 2, 40, 300, 9
    announce("prenorm_dconv1d_fwd zero W", (N, C, L, d))
    p = prenorm_inputs(N, C, L, 32)
    p["W"] = torch.zeros(C, C, 3)
    got = run_block(p, d).cpu()
    exp = p["x"] + p["b"][None, :, None]
    assert torch.equal(got, exp)


def test_block_null_bias():
    N, C, L, d = 2, 40, 300, 9
    announce("prenorm_dconv1d_fwd b=NULL", (N, C, L, d))
    p = prenorm_inputs(N, C, L, 33)
    p["b"] = None
    err = maxrel(run_block(p, d).cpu().numpy(), oracle_block(p, d))
    assert err <= TOL_F32, err


def test_block_empty_batch():
    announce("prenorm_dconv1d_fwd N=0")
    p = prenorm_inputs(0, 16, 64, 34)
    assert run_block(p, 4).shape == (0, 16, 64)
    assert run_block(prenorm_inputs(0, 16, 64, 34, bf16=True), 4, bf16=True).shape == (0, 16, 64)
    g = groupnorm_inputs(0, 8, 16, 20, 35)
    assert run_gn(g, 4, 1, 1).shape == (0, 16, 20)


def test_block_guard_band_and_stream():
    """Writes stay inside out (sentinels around it survive) and work runs on a
    non-default stream."""
    N, C, L, d = 2, 64, 777, 33
    announce("prenorm_dconv1d_fwd guard band", (N, C, L, d))
    p = prenorm_inputs(N, C, L, 35)
    q = to_dev(p)
    n = N * C * L
    guard = 4096
    buf = torch.full((n + 2 * guard,), 12345.0, device="cuda")
    out = buf[guard:guard + n].view(N, C, L)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dc.prenorm_dconv1d_fwd(q["x"], q["running_mean"], q["running_var"], q["gamma"],
                               q["beta"], q["eps"], q["W"], q["b"], d, out=out)
    s.synchronize()
    b = buf.cpu()
    assert torch.all(b[:guard] == 12345.0) and torch.all(b[guard + n:] == 12345.0)
    err = maxrel(out.cpu().numpy(), oracle_block(p, d))
    assert err <= TOL_F32, err


def test_block_deterministic():
    N, C, L, d = 4, 256, 2048, 128
    announce("prenorm_dconv1d_fwd determinism", (N, C, L, d))
    q = to_dev(prenorm_inputs(N, C, L, 36))
    outs = [dc.prenorm_dconv1d_fwd(q["x"], q["running_mean"], q["running_var"], q["gamma"],
                                   q["beta"], q["eps"], q["W"], q["b"], d) for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], o) for o in outs[1:])


def test_block_alias_rejected():
    q = to_dev(prenorm_inputs(1, 8, 32, 37))
    with pytest.raises(dc.Dconv1dError) as e:
        dc.prenorm_dconv1d_fwd(q["x"], q["running_mean"], q["running_var"], q["gamma"],
                               q["beta"], q["eps"], q["W"], q["b"], 2, out=q["x"])
    assert e.value.code == dc.DCONV1D_EALIAS


# ----------------------------------------------------------------- GroupNorm sibling

GN_CASES = [
    # (N, C_in, C_out, T, G, padding, dilation, bias, affine)
    (2, 40, 96, 333, 12, 1, 1, False, True),
    (2, 40, 96, 333, 12, 1, 1, True, True),
    (2, 40, 96, 333, 12, 1, 1, False, False),
    (1, 16, 32, 77, 1, 3, 2, True, True),
    (1, 16, 32, 77, 32, 0, 1, False, True),
    (2, 64, 300, 150, 3, 1, 1, False, True),     # two output-channel tiles
    (3, 8, 16, 5, 4, 2, 3, False, True),         # T_out = 3
    (4, 128, 256, 1023, 32, 1, 1, False, True),  # ragged time tail
    (8, 32, 64, 5000, 8, 1, 1, True, True),      # 64-step x 256-channel tiles
    (2, 64, 300, 150, 3, 1, 1, False, True),     # 128-channel tiles, 3 channel tiles
    (2, 96, 128, 2048, 8, 1, 1, True, True),     # 9 chunks (odd), T_out % 4 == 0
    (4, 32, 256, 1026, 16, 0, 1, False, True),   # 3 chunks (odd), T_out = 1024
    # single-launch path (groups inside 16 channels, T_out <= 1024, C_in % 16 == 0, staged
    # window 128*ceil(T_out/128) + 2*dil <= 1216 steps); the cases above with C_in of 8,
    # 32 with T_out > 1024, 40, or 32 channels per group take the two-launch path:
    (2, 48, 48, 200, 6, 1, 1, True, True),       # 3 input-channel chunks (odd)
    (2, 16, 16, 1000, 8, 0, 1, False, True),     # one chunk, 2 channels per group
    (3, 16, 16, 5, 4, 2, 3, True, True),         # T_out = 3
    (1, 16, 32, 600, 16, 5, 200, True, True),    # taps 200 apart, pad != dil
    (1, 16, 32, 1100, 4, 0, 256, False, True),   # pad 0, T_out = 588
    (1, 16, 32, 1024, 2, 96, 96, True, False),   # widest staged window (1216 steps)
    (1, 16, 32, 1024, 2, 97, 97, True, True),    # one step past it: two-launch path
    (2, 16, 32, 100, 4, 3, 1, False, True),      # pad > dil
    (3, 64, 256, 1024, 32, 1, 1, True, True),    # the GN workload's layer with a bias
    (2, 32, 64, 512, 8, 2, 2, False, True),      # window shift 2 (16-byte loads)
    (40, 32, 128, 256, 16, 1, 1, True, True),    # 320 workgroups: more than one per CU
    # of the single-launch cases above, those with 128 + 2*dil + delta <= 136 (delta: 0..3
    # with 16-byte loads, 0 with 4-byte ones) stage per-wave windows; the rest (taps 200
    # or 256 apart, pad 96 or 97) and these share one window per workgroup:
    (2, 16, 32, 301, 4, 5, 5, True, True),       # shared window, 4-byte loads, 3 waves
    (2, 32, 64, 400, 8, 5, 5, False, True),      # shared window, 16-byte loads, delta 3
    # per-wave windows at their edges
    (2, 32, 64, 777, 8, 1, 1, True, True),       # 4-byte loads, 7 waves, ragged last wave
    (2, 16, 32, 1004, 4, 3, 3, False, True),     # 16-byte loads, 128 + 6 + 1 = 135 steps
    (2, 16, 32, 1006, 4, 4, 4, False, True),     # 4-byte loads, 128 + 8 = 136: widest
    (2, 16, 32, 1008, 4, 0, 1, True, True),      # pad 0: delta 0, T_out = 1006
    (1, 48, 16, 130, 16, 2, 1, True, True),      # two waves, the second with 4 steps
    # gamma or beta alone (the other NULL: gamma = 1 or beta = 0), on both paths
    (2, 32, 64, 512, 8, 1, 1, True, "beta"),     # single launch, gamma NULL
    (2, 32, 64, 512, 8, 1, 1, False, "gamma"),   # single launch, beta NULL
    (4, 64, 128, 2048, 16, 1, 1, True, "beta"),  # two launches (T_out > 1024), gamma NULL
    (4, 64, 128, 2048, 16, 1, 1, False, "gamma"),  # two launches, beta NULL
]


def set_form(monkeypatch, form):
    """The conv form: the library's choice ("auto") or the three-tap kernels ("three_tap")."""
    if form == "three_tap":
        monkeypatch.setenv("DCONV1D_WINOGRAD", "0")
    else:
        monkeypatch.delenv("DCONV1D_WINOGRAD", raising=False)


def run_gn(p, G, padding, dilation):
    q = to_dev(p)
    o = dc.conv1d_groupnorm_fwd(q["x"], q["W"], q["bias"], q["gamma"], q["beta"], q["eps"], G,
                                padding, dilation)
    torch.cuda.synchronize()
    return o


def oracle_gn(p, G, padding, dilation):
    return oracle.conv_groupnorm(p["x"], p["W"], p["bias"], p["gamma"], p["beta"], p["eps"], G,
                                 padding, dilation)


@pytest.mark.parametrize("N,C_in,C_out,T,G,pad,dil,bias,affine", GN_CASES)
@pytest.mark.parametrize("form", ["auto", "three_tap"])
def test_groupnorm_matches_oracle(N, C_in, C_out, T, G, pad, dil, bias, affine, form,
                                  monkeypatch):
    """form "auto": the library's choice (the single-launch kernel takes its Winograd form
    for dilations 1, 2 and 4 with per-wave windows); "three_tap": DCONV1D_WINOGRAD=0."""
    set_form(monkeypatch, form)
    seed = 30_000 + N + C_in + C_out + T + G + pad + dil
    announce("conv1d_groupnorm_fwd", form, (N, C_in, C_out, T, G, pad, dil, bias, affine),
             "seed", seed)
    p = groupnorm_inputs(N, C_in, C_out, T, seed, with_bias=bias)
    if affine is False:
        p["gamma"] = None
        p["beta"] = None
    elif affine == "beta":
        p["gamma"] = None
    elif affine == "gamma":
        p["beta"] = None
    got = run_gn(p, G, pad, dil).cpu().numpy()
    err = maxrel(got, oracle_gn(p, G, pad, dil))
    assert err <= TOL_F32, err


@pytest.mark.parametrize("form", ["auto", "three_tap"])
def test_groupnorm_unaligned_x(form, monkeypatch):
    """x and out only 4-byte aligned (views one float into buffers): the single-launch path
    then stages with 4-byte loads; same bar against the oracle, and the floats around out
    stay untouched."""
    set_form(monkeypatch, form)
    N, C_in, C_out, T, G, pad, dil = 2, 32, 64, 512, 8, 1, 1
    announce("conv1d_groupnorm_fwd unaligned x and out", form, (N, C_in, C_out, T, G, pad, dil))
    p = groupnorm_inputs(N, C_in, C_out, T, 30_777, with_bias=True)
    q = to_dev(p)
    buf = torch.empty(N * C_in * T + 4, device="cuda")
    x = buf[1:1 + N * C_in * T].view(N, C_in, T)
    x.copy_(q["x"])
    assert x.data_ptr() % 16 != 0
    T_out = T + 2 * pad - 2 * dil
    n_out = N * C_out * T_out
    obuf = torch.full((n_out + 8,), 12345.0, device="cuda")
    out = obuf[1:1 + n_out].view(N, C_out, T_out)
    assert out.data_ptr() % 16 != 0
    dc.conv1d_groupnorm_fwd(x, q["W"], q["bias"], q["gamma"], q["beta"], q["eps"], G, pad, dil,
                            out=out)
    torch.cuda.synchronize()
    ob = obuf.cpu()
    assert ob[0] == 12345.0 and torch.all(ob[1 + n_out:] == 12345.0)
    err = maxrel(out.cpu().numpy(), oracle_gn(p, G, pad, dil))
    assert err <= TOL_F32, err


@pytest.mark.parametrize("shape", [
    (16, 128, 256, 1024, 32, 1, 1),   # the GN workload: single-launch path
    (4, 64, 128, 2048, 16, 1, 1),     # T_out > 1024: two-launch path (tile partials)
])
@pytest.mark.parametrize("form", ["auto", "three_tap"])
def test_groupnorm_deterministic(shape, form, monkeypatch):
    """Bitwise-equal results over 10 calls in different launch orders: back to back, after
    another kernel, on a second stream, and after a call of another shape (which leaves
    other partials in the library's workspace on the two-launch path)."""
    set_form(monkeypatch, form)
    N, C_in, C_out, T, G, pad, dil = shape
    announce("conv1d_groupnorm_fwd determinism", form, shape)
    q = to_dev(groupnorm_inputs(N, C_in, C_out, T, 41))
    o = to_dev(groupnorm_inputs(2, C_in, C_out, T // 2 + 3, 42))
    blk = to_dev(prenorm_inputs(2, 64, 1000, 43))

    def gn():
        return dc.conv1d_groupnorm_fwd(q["x"], q["W"], q["bias"], q["gamma"], q["beta"],
                                       q["eps"], G, pad, dil)

    side = torch.cuda.Stream()
    outs = []
    for i in range(10):
        kind = i % 4
        if kind == 1:
            dc.prenorm_dconv1d_fwd(blk["x"], blk["running_mean"], blk["running_var"],
                                   blk["gamma"], blk["beta"], blk["eps"], blk["W"], blk["b"], 7)
        elif kind == 3:
            dc.conv1d_groupnorm_fwd(o["x"], o["W"], o["bias"], o["gamma"], o["beta"], o["eps"],
                                    G, pad, dil)
        if kind == 2:
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                outs.append(gn())
            torch.cuda.current_stream().wait_stream(side)
        else:
            outs.append(gn())
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], r) for r in outs[1:])


def test_block_bf16_deterministic():
    N, C, L, d = 2, 512, 1024, 128
    announce("prenorm_dconv1d_fwd_bf16 determinism", (N, C, L, d))
    q = to_dev(prenorm_inputs(N, C, L, 44, bf16=True))
    outs = [dc.prenorm_dconv1d_fwd_bf16(q["x"], q["running_mean"], q["running_var"],
                                        q["gamma"], q["beta"], q["eps"], q["W"], q["b"], d)
            for _ in range(3)]
    torch.cuda.synchronize()
    assert all(torch.equal(outs[0], r) for r in outs[1:])


@pytest.mark.parametrize("N,C,L,d", [(2, 512, 2048, 128), (2, 64, 1024, 8)])
def test_block_bf16_x_load_forms_agree(N, C, L, d):
    """The bf16 kernel's x load forms stage the same values: x 4-byte aligned (2 steps per
    buffer->LDS load) and 2-byte aligned (1 step per load into registers) give the same
    bits, and so do the 16-byte and per-element epilogues. x sits 2 or 1 elements into a
    buffer; the residual, the same x, then takes the per-element epilogue."""
    announce("prenorm_dconv1d_fwd_bf16 x load forms", (N, C, L, d))
    q = to_dev(prenorm_inputs(N, C, L, 45, bf16=True))

    def run(x):
        o = dc.prenorm_dconv1d_fwd_bf16(x, q["running_mean"], q["running_var"], q["gamma"],
                                        q["beta"], q["eps"], q["W"], q["b"], d)
        torch.cuda.synchronize()
        return o.cpu()

    ref = run(q["x"])
    for shift in (2, 1):
        buf = torch.empty(q["x"].numel() + 8, device="cuda", dtype=q["x"].dtype)
        x = buf[shift:shift + q["x"].numel()].view(q["x"].shape)
        x.copy_(q["x"])
        assert x.data_ptr() % 16 != 0
        assert torch.equal(run(x), ref), shift


# ----------------------------------------------------------------- full benchmark workloads

def test_workload0_tiny():
    w = WORKLOADS[0].dims
    announce("workload 0", w)
    p = prenorm_inputs(w["N"], w["C"], w["L"], seed_for(0))
    err = maxrel(run_block(p, w["d"]).cpu().numpy(), oracle_block(p, w["d"]))
    announce(f"workload 0: max rel err {err:.3g}")
    assert err <= TOL_F32, err


def test_workload1_full():
    """N=32, C=256, L=4096, d=128: every output against the oracle."""
    w = WORKLOADS[1].dims
    announce("workload 1 full compare", w)
    p = prenorm_inputs(w["N"], w["C"], w["L"], seed_for(1))
    got = run_block(p, w["d"]).cpu()
    err = full_compare_by_sample(p, got, w["d"])
    announce(f"workload 1: max rel err {err:.3g} over {got.numel()} outputs")
    assert err <= TOL_F32, err


def full_compare_by_sample(p, got, d):
    """Max relative error of `got` (CPU float32 or bfloat16 tensor [N][C][L]) against the
    oracle over every output, the oracle run one sample at a time to bound its memory."""
    worst = 0.0
    for n in range(got.shape[0]):
        ref = oracle.prenorm_block(p["x"][n:n + 1], p["running_mean"], p["running_var"],
                                   p["gamma"], p["beta"], p["eps"], p["W"], p["b"], d)
        worst = max(worst, maxrel(got[n:n + 1].float().numpy(), ref))
    return worst


@pytest.mark.parametrize("d", WORKLOADS[2].dims["ds"])
def test_workload2_dilation_sweep_full(d):
    """N=32, C=256, L=4096 at each swept dilation: every output against the oracle."""
    w = WORKLOADS[2].dims
    announce("workload 2 full compare", w, "d", d)
    p = prenorm_inputs(w["N"], w["C"], w["L"], seed_for(2, d))
    got = run_block(p, d).cpu()
    err = full_compare_by_sample(p, got, d)
    announce(f"workload 2 d={d}: max rel err {err:.3g} over {got.numel()} outputs")
    assert err <= TOL_F32, err


@pytest.mark.parametrize("form", ["auto", "three_tap"])
def test_workload3_groupnorm_full(form, monkeypatch):
    set_form(monkeypatch, form)
    w = WORKLOADS[3].dims
    announce("workload 3 full compare", form, w)
    p = groupnorm_inputs(w["N"], w["C_in"], w["C_out"], w["T"], seed_for(3))
    got = run_gn(p, w["G"], w["padding"], w["dilation"]).cpu().numpy()
    err = maxrel(got, oracle_gn(p, w["G"], w["padding"], w["dilation"]))
    announce(f"workload 3: max rel err {err:.3g} over {got.size} outputs")
    assert err <= TOL_F32, err


def test_workload4_bf16_full():
    """N=16, C=512, L=16384, d=128 with bfloat16 storage: every output against the oracle."""
    w = WORKLOADS[4].dims
    announce("workload 4 full compare", w)
    p = prenorm_inputs(w["N"], w["C"], w["L"], seed_for(4), bf16=True)
    got = run_block(p, w["d"], bf16=True).cpu()
    err = full_compare_by_sample(p, got, w["d"])
    announce(f"workload 4: max rel err {err:.3g} over {got.numel()} outputs")
    assert err <= TOL_BF16, err
