"""Training-mode BatchNorm block (prenorm_dconv1d_fwd_train / _train_bf16) against the
float64 oracle (oracle.prenorm_block_train), through the C ABI.

Bars: block output as for the eval-mode block (float32 storage 2e-4, bfloat16 storage
2e-2, relative to 1 + |ref|). The statistics are formed in double and rounded once to
float32, so the updated running statistics, the batch mean and 1/sqrt(var+eps) must
agree with the oracle to 1e-6 relative (a few float32 ulps)."""
import numpy as np
import pytest
import torch

import normalisation_dilated_conv1d_amd as dc
import oracle
from normalisation_dilated_conv1d_amd.inputs import WORKLOADS, prenorm_inputs, seed_for

from test_gpu_parity import TOL_BF16, TOL_F32, announce, maxrel, to_dev

pytestmark = pytest.mark.gpu

TOL_STATS = 1e-6


def run_train(p, d, momentum, bf16=False, with_running=True, with_saved=True):
    q = to_dev(p)
    C = q["x"].shape[1]
    rm = q["running_mean"].clone() if with_running else None
    rv = q["running_var"].clone() if with_running else None
    sm = torch.full((C,), float("nan"), device="cuda") if with_saved else None
    si = torch.full((C,), float("nan"), device="cuda") if with_saved else None
    fn = dc.prenorm_dconv1d_fwd_train_bf16 if bf16 else dc.prenorm_dconv1d_fwd_train
    out = fn(q["x"], rm, rv, q["gamma"], q["beta"], q["eps"], momentum, q["W"], q["b"], d,
             save_mean=sm, save_invstd=si)
    torch.cuda.synchronize()
    cpu = lambda t: None if t is None else t.float().cpu().numpy()
    return cpu(out), cpu(rm), cpu(rv), cpu(sm), cpu(si)


def oracle_train(p, d, momentum):
    return oracle.prenorm_block_train(p["x"], p["running_mean"], p["running_var"], p["gamma"],
                                      p["beta"], p["eps"], momentum, p["W"], p["b"], d)


def check(got, ref, eps, tol_out):
    out, rm, rv, sm, si = got
    o_out, o_rm, o_rv, o_mean, o_var = ref
    errs = {"out": maxrel(out, o_out)}
    if rm is not None:
        errs["running_mean"] = maxrel(rm, o_rm)
        errs["running_var"] = maxrel(rv, o_rv)
    if sm is not None:
        errs["save_mean"] = maxrel(sm, o_mean)
        errs["save_invstd"] = maxrel(si, 1.0 / np.sqrt(o_var + eps))
    bad = {k: v for k, v in errs.items()
           if v > (tol_out if k == "out" else TOL_STATS)}
    assert not bad, errs


TRAIN_CASES = [
    # (N, C, L, d)
    (1, 1, 2, 1),            # the fewest values per channel allowed
    (1, 3, 7, 2),
    (2, 16, 512, 128),       # the tiny workload's shape
    (3, 48, 1000, 3),        # L % 4 == 0
    (2, 33, 257, 31),        # odd L: scalar statistics loads
    (2, 300, 700, 64),       # C not a multiple of 32, two output-channel tiles
    (8, 64, 8200, 128),      # three statistics segments per row, ragged last one
    (1, 8, 12288, 5),        # three full segments
]


@pytest.mark.parametrize("N,C,L,d", TRAIN_CASES)
def test_train_f32_matches_oracle(N, C, L, d):
    seed = 30_000 + N * 7 + C * 13 + L + d
    announce("prenorm_dconv1d_fwd_train", (N, C, L, d), "seed", seed)
    p = prenorm_inputs(N, C, L, seed)
    # per-channel offsets and spreads so the batch statistics differ from the running ones
    g = np.random.default_rng(seed)
    p["x"] = p["x"] * torch.from_numpy(g.uniform(0.5, 2.0, (1, C, 1)).astype(np.float32)) \
        + torch.from_numpy(g.normal(0, 1.0, (1, C, 1)).astype(np.float32))
    check(run_train(p, d, 0.1), oracle_train(p, d, 0.1), p["eps"], TOL_F32)


# (2, 384, 16384, 128) runs the 512-channel (8-wave) bf16 tile
@pytest.mark.parametrize("N,C,L,d", [(1, 3, 7, 2), (2, 96, 777, 50), (8, 64, 8200, 128),
                                     (2, 16, 512, 128), (2, 384, 16384, 128)])
def test_train_bf16_matches_oracle(N, C, L, d):
    seed = 40_000 + N + C + L + d
    announce("prenorm_dconv1d_fwd_train_bf16", (N, C, L, d), "seed", seed)
    p = prenorm_inputs(N, C, L, seed, bf16=True)
    p["x"] = (p["x"].float() * 1.5 + 0.3).to(torch.bfloat16)
    check(run_train(p, d, 0.2, bf16=True), oracle_train(p, d, 0.2), p["eps"], TOL_BF16)


def test_train_large_offset():
    """|mean| >> std: the per-channel shift keeps the variance accurate."""
    N, C, L, d = 2, 40, 3000, 9
    announce("train large offset", (N, C, L, d))
    p = prenorm_inputs(N, C, L, 30_500)
    p["x"] = p["x"] * 0.01 + 1000.0
    check(run_train(p, d, 0.1), oracle_train(p, d, 0.1), p["eps"], TOL_F32)


def test_train_without_running_or_saved():
    """NULL running statistics and saved vectors: same output, nothing else touched."""
    N, C, L, d = 2, 64, 900, 17
    announce("train no running stats", (N, C, L, d))
    p = prenorm_inputs(N, C, L, 30_600)
    full = run_train(p, d, 0.1)
    bare = run_train(p, d, 0.1, with_running=False, with_saved=False)
    assert np.array_equal(full[0], bare[0])
    check(bare, oracle_train(p, d, 0.1), p["eps"], TOL_F32)


def test_train_running_update_accumulates():
    """Two calls in a row update the running statistics twice (momentum applied to the
    state the first call left)."""
    N, C, L, d = 2, 32, 600, 4
    announce("train two updates", (N, C, L, d))
    p = prenorm_inputs(N, C, L, 30_700)
    q = to_dev(p)
    rm, rv = q["running_mean"].clone(), q["running_var"].clone()
    for _ in range(2):
        dc.prenorm_dconv1d_fwd_train(q["x"], rm, rv, q["gamma"], q["beta"], q["eps"], 0.3, q["W"],
                                     q["b"], d)
    torch.cuda.synchronize()
    _, rm1, rv1, _, _ = oracle_train(p, d, 0.3)
    _, rm2, rv2, _, _ = oracle.prenorm_block_train(p["x"], rm1, rv1, p["gamma"], p["beta"],
                                                   p["eps"], 0.3, p["W"], p["b"], d)
    assert maxrel(rm.cpu().numpy(), rm2) <= TOL_STATS
    assert maxrel(rv.cpu().numpy(), rv2) <= TOL_STATS


def test_train_deterministic():
    N, C, L, d = 4, 128, 5000, 64
    announce("train determinism", (N, C, L, d))
    p = prenorm_inputs(N, C, L, 30_800)
    a = run_train(p, d, 0.1)
    for _ in range(3):
        b = run_train(p, d, 0.1)
        for u, v in zip(a, b):
            assert np.array_equal(u, v)


def test_train_empty_batch():
    announce("train empty batch")
    C = 8
    x = torch.empty((0, C, 16), device="cuda")
    rm = torch.ones(C, device="cuda")
    rv = torch.ones(C, device="cuda") * 2
    W = torch.zeros((C, C, 3), device="cuda")
    out = dc.prenorm_dconv1d_fwd_train(x, rm, rv, torch.ones(C, device="cuda"),
                                       torch.zeros(C, device="cuda"), 1e-5, 0.1, W, None, 3)
    torch.cuda.synchronize()
    assert out.shape == (0, C, 16)
    assert torch.equal(rm.cpu(), torch.ones(C)) and torch.equal(rv.cpu(), torch.ones(C) * 2)


def test_train_workload1_full():
    """The benchmark shape N=32, C=256, L=4096, d=128 with training-mode BN: every output,
    the running statistics and the saved vectors against the oracle."""
    w = WORKLOADS[1].dims
    announce("train workload 1 full compare", w)
    p = prenorm_inputs(w["N"], w["C"], w["L"], seed_for(1))
    check(run_train(p, w["d"], 0.1), oracle_train(p, w["d"], 0.1), p["eps"], TOL_F32)
