"""Checks that pin the CPU oracle to facts other than itself.

Each check takes an implementation (the oracle, or a deliberately broken copy of it)
and returns ``(ok, message)`` instead of asserting, so the same checks can be shown
to reject planted mistakes (``tests/test_oracle_mutants.py``).

Kinds of pin used here:
* hand-worked golden values (``tests/golden/*.json``, each with its derivation);
* pure-Python brute force on tiny inputs (``oracle/brute.py``);
* torch float64 CPU library routines (batch_norm, conv1d, group_norm,
  instance_norm, layer_norm), i.e. an independent implementation of the same
  definition;
* closed forms and invariants (zero weights, zero BN affine, d >= L, one-hot
  weights, linearity, GroupNorm moments and scale invariance).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import torch
import torch.nn.functional as F

from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _np(a):
    return np.asarray(a, dtype=np.float64)


def _rand_block(N, C, L, seed, beta_shift=0.0):
    rng = np.random.default_rng(seed)
    return dict(
        x=rng.standard_normal((N, C, L)),
        running_mean=rng.uniform(-0.5, 0.5, C),
        running_var=rng.uniform(0.5, 1.5, C),
        gamma=rng.uniform(0.5, 1.5, C),
        beta=rng.normal(0, 0.1, C) + beta_shift,
        eps=1e-5,
        W=rng.normal(0, 1 / math.sqrt(3 * C), (C, C, 3)),
        b=rng.normal(0, 0.01, C),
    )


def _call_block(fn, p, d):
    return _np(fn(p["x"], p["running_mean"], p["running_var"], p["gamma"], p["beta"],
                  p["eps"], p["W"], p["b"], d))


def _torch_block(p, d):
    t = {k: (torch.from_numpy(np.asarray(v, dtype=np.float64)) if not isinstance(v, float) else v)
         for k, v in p.items()}
    z = F.batch_norm(t["x"], t["running_mean"], t["running_var"], t["gamma"], t["beta"],
                     training=False, eps=p["eps"])
    z = F.relu(z)
    y = F.conv1d(z, t["W"], t["b"], stride=1, padding=d, dilation=d)
    return (t["x"] + y).numpy()


def _maxrel(a, b):
    a, b = _np(a), _np(b)
    if a.shape != b.shape:
        return float("inf")
    return float(np.max(np.abs(a - b) / (1.0 + np.abs(b)))) if a.size else 0.0


# --------------------------------------------------------------------------- block pins

def block_hand_golden(fn):
    g = json.load(open(os.path.join(GOLDEN, "prenorm_block_hand.json")))
    i = g["inputs"]
    out = _np(fn(_np(i["x"]), _np(i["running_mean"]), _np(i["running_var"]), _np(i["gamma"]),
                 _np(i["beta"]), i["eps"], _np(i["W"]), _np(i["b"]), i["d"]))
    err = _maxrel(out, g["expected"])
    return err <= 1e-14, f"hand golden max rel err {err:.3g}"


def block_brute_tiny(fn):
    worst = 0.0
    for (N, C, L, ds, seed) in [(1, 1, 5, (1, 2, 4, 5, 8), 1), (2, 3, 9, (1, 2, 3, 8, 9, 12), 2),
                                (2, 4, 16, (1, 3, 5, 15, 16, 19), 3)]:
        for d in ds:
            p = _rand_block(N, C, L, seed * 100 + d, beta_shift=0.3)
            ref = brute.prenorm_block_brute(p["x"], p["running_mean"], p["running_var"],
                                            p["gamma"], p["beta"], p["eps"], p["W"], p["b"], d)
            worst = max(worst, _maxrel(_call_block(fn, p, d), ref))
    return worst <= 1e-12, f"brute force (tiny shapes) max rel err {worst:.3g}"


def block_brute_config0(fn):
    """All of the tiny workload's shape (N=2, C=16, L=512, d=128) against brute force."""
    p = _rand_block(2, 16, 512, 7)
    ref = brute.prenorm_block_brute(p["x"], p["running_mean"], p["running_var"], p["gamma"],
                                    p["beta"], p["eps"], p["W"], p["b"], 128)
    err = _maxrel(_call_block(fn, p, 128), ref)
    return err <= 1e-12, f"brute force (2,16,512,d=128) max rel err {err:.3g}"


def block_torch_f64(fn):
    worst = 0.0
    for (N, C, L, d, seed) in [(2, 16, 512, 128, 11), (2, 64, 600, 1, 12), (1, 64, 600, 8, 13),
                               (1, 48, 700, 333, 14), (1, 32, 300, 300, 15), (1, 32, 300, 1000, 16),
                               (2, 40, 257, 64, 17)]:
        p = _rand_block(N, C, L, seed, beta_shift=0.2)
        worst = max(worst, _maxrel(_call_block(fn, p, d), _torch_block(p, d)))
    return worst <= 1e-10, f"torch float64 batch_norm/relu/conv1d max rel err {worst:.3g}"


def block_padding_trap(fn):
    """mean 0, gamma 1, beta +5: ReLU(BN(0)) = 5, so any padding applied before the BN
    would add 5*sum(W) at the first and last d outputs. Compared with torch float64."""
    N, C, L, d = 1, 8, 64, 16
    p = _rand_block(N, C, L, 21)
    p["running_mean"] = np.zeros(C)
    p["running_var"] = np.ones(C) - p["eps"]
    p["gamma"] = np.ones(C)
    p["beta"] = np.full(C, 5.0)
    err = _maxrel(_call_block(fn, p, d), _torch_block(p, d))
    return err <= 1e-10, f"beta=+5 padding trap max rel err {err:.3g}"


def block_zero_weights(fn):
    """W = 0 gives out = x + b exactly."""
    p = _rand_block(2, 8, 50, 31)
    p["W"] = np.zeros_like(p["W"])
    out = _call_block(fn, p, 7)
    exp = p["x"] + p["b"][None, :, None]
    err = float(np.max(np.abs(out - exp)))
    return err == 0.0, f"W=0: max |out - (x+b)| = {err:.3g}"


def block_zero_bn_affine(fn):
    """gamma = beta = 0 makes z = 0, so out = x + b exactly."""
    p = _rand_block(2, 8, 50, 32)
    p["gamma"] = np.zeros(8)
    p["beta"] = np.zeros(8)
    out = _call_block(fn, p, 3)
    exp = p["x"] + p["b"][None, :, None]
    err = float(np.max(np.abs(out - exp)))
    return err == 0.0, f"gamma=beta=0: max |out - (x+b)| = {err:.3g}"


def block_dilation_ge_length(fn):
    """d >= L: both outer taps fall in the padding, leaving a 1x1 conv with the centre
    tap: out = x + b + W[:, :, 1] @ relu(bn(x))."""
    worst = 0.0
    for d in (40, 41, 100):
        p = _rand_block(2, 6, 40, 33 + d)
        z = np.maximum(p["gamma"][None, :, None] * (p["x"] - p["running_mean"][None, :, None])
                       / np.sqrt(p["running_var"][None, :, None] + p["eps"])
                       + p["beta"][None, :, None], 0.0)
        exp = p["x"] + p["b"][None, :, None] + np.einsum("oc,nct->not", p["W"][:, :, 1], z)
        worst = max(worst, _maxrel(_call_block(fn, p, d), exp))
    return worst <= 1e-13, f"d>=L centre-tap-only max rel err {worst:.3g}"


def block_one_hot(fn):
    """A single 1 at W[co, ci, k] (b = 0) makes out[n, co] - x[n, co] the zero-filled
    shift of z[n, ci] by (k-1)*d, pinning the tap direction and the W layout."""
    N, C, L, d = 1, 3, 20, 4
    p = _rand_block(N, C, L, 41, beta_shift=0.5)
    p["b"] = np.zeros(C)
    z = np.maximum(p["gamma"][None, :, None] * (p["x"] - p["running_mean"][None, :, None])
                   / np.sqrt(p["running_var"][None, :, None] + p["eps"])
                   + p["beta"][None, :, None], 0.0)
    worst = 0.0
    for (co, ci, k) in [(0, 2, 0), (1, 0, 2), (2, 1, 1), (0, 1, 2)]:
        W = np.zeros((C, C, 3))
        W[co, ci, k] = 1.0
        q = dict(p, W=W)
        y = _call_block(fn, q, d) - p["x"]
        exp = np.zeros((N, C, L))
        s = (k - 1) * d
        for t in range(L):
            if 0 <= t + s < L:
                exp[:, co, t] = z[:, ci, t + s]
        worst = max(worst, float(np.max(np.abs(y - exp))))
    return worst <= 1e-14, f"one-hot W shift max abs err {worst:.3g}"


def block_relu_identity(fn):
    """mean 0, gamma 1, beta 0, var + eps = 1 (exactly, with eps = var = 0.5): z = relu(x)."""
    N, C, L, d = 1, 4, 24, 5
    p = _rand_block(N, C, L, 51)
    p.update(running_mean=np.zeros(C), running_var=np.full(C, 0.5), eps=0.5,
             gamma=np.ones(C), beta=np.zeros(C))
    z = np.maximum(p["x"], 0.0)
    t = torch.from_numpy
    exp = (t(p["x"]) + F.conv1d(t(z), t(p["W"]), t(p["b"]), padding=d, dilation=d)).numpy()
    err = _maxrel(_call_block(fn, p, d), exp)
    return err <= 1e-13, f"relu-identity BN max rel err {err:.3g}"


def block_linear_in_W(fn):
    """With b = 0, out - x is linear in W."""
    p = _rand_block(2, 5, 30, 61)
    p["b"] = np.zeros(5)
    rng = np.random.default_rng(62)
    W1, W2 = rng.standard_normal((5, 5, 3)), rng.standard_normal((5, 5, 3))
    f = lambda W: _call_block(fn, dict(p, W=W), 6) - p["x"]
    err = float(np.max(np.abs(f(W1 + 2.0 * W2) - (f(W1) + 2.0 * f(W2)))))
    return err <= 1e-12, f"linearity in W max abs err {err:.3g}"


def block_output_length(fn):
    p = _rand_block(1, 3, 37, 71)
    shapes = {d: _call_block(fn, p, d).shape for d in (1, 5, 36, 37, 90)}
    ok = all(s == (1, 3, 37) for s in shapes.values())
    return ok, f"output shapes {shapes}"


BLOCK_PINS = [block_hand_golden, block_brute_tiny, block_torch_f64, block_padding_trap,
              block_zero_weights, block_zero_bn_affine, block_dilation_ge_length,
              block_one_hot, block_relu_identity, block_linear_in_W, block_output_length]


# --------------------------------------------------------------------------- external-BN pins

def _rand_ext(N, C, L, seed):
    rng = np.random.default_rng(seed)
    return dict(xn=rng.standard_normal((N, C, L)) + 0.2,
                W=rng.normal(0, 1 / math.sqrt(3 * C), (C, C, 3)),
                b=rng.normal(0, 0.1, C),
                residual=rng.standard_normal((N, C, L)))


def _call_ext(fn, p, d):
    return _np(fn(p["xn"], p["W"], p["b"], p["residual"], d))


def ext_hand_golden(fn):
    g = json.load(open(os.path.join(GOLDEN, "relu_conv_residual_hand.json")))
    i = {k: _np(v) for k, v in g["inputs"].items()}
    err = max(_maxrel(_call_ext(fn, i, c["d"]), c["expected"]) for c in g["cases"])
    return err <= 1e-14, f"external-BN hand golden max rel err {err:.3g}"


def ext_brute_tiny(fn):
    worst = 0.0
    for (N, C, L, ds, seed) in [(1, 2, 6, (1, 2, 5, 6, 9), 1), (2, 3, 11, (1, 3, 10), 2)]:
        for d in ds:
            p = _rand_ext(N, C, L, seed * 10 + d)
            ref = brute.relu_conv_residual_brute(p["xn"], p["W"], p["b"], p["residual"], d)
            worst = max(worst, _maxrel(_call_ext(fn, p, d), ref))
    return worst <= 1e-12, f"external-BN brute force max rel err {worst:.3g}"


def ext_torch_f64(fn):
    worst = 0.0
    for (N, C, L, d, seed) in [(2, 16, 512, 128, 3), (1, 40, 300, 1, 4), (2, 24, 100, 150, 5)]:
        p = _rand_ext(N, C, L, seed)
        t = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
        exp = t(p["residual"]) + F.conv1d(F.relu(t(p["xn"])), t(p["W"]), t(p["b"]), padding=d,
                                          dilation=d)
        worst = max(worst, _maxrel(_call_ext(fn, p, d), exp.numpy()))
    return worst <= 1e-10, f"external-BN torch float64 max rel err {worst:.3g}"


def ext_is_block_with_bn_outside(fn):
    """With xn = BatchNorm1d_eval(x) (scalar loops) and residual = x, the result is the
    pre-norm block (brute force)."""
    N, C, L, d = 2, 3, 10, 3
    p = _rand_block(N, C, L, 61, beta_shift=0.2)
    x = p["x"]
    xn = (p["gamma"][None, :, None] * (x - p["running_mean"][None, :, None])
          / np.sqrt(p["running_var"][None, :, None] + p["eps"]) + p["beta"][None, :, None])
    ref = brute.prenorm_block_brute(x, p["running_mean"], p["running_var"], p["gamma"],
                                    p["beta"], p["eps"], p["W"], p["b"], d)
    err = _maxrel(_np(fn(xn, p["W"], p["b"], x, d)), ref)
    return err <= 1e-12, f"external-BN = block with BN outside, max rel err {err:.3g}"


def ext_residual_passthrough(fn):
    """out - residual does not depend on residual, and W = 0 gives residual + b exactly."""
    p = _rand_ext(2, 5, 30, 62)
    q = dict(p, residual=p["residual"] * 3.0 - 1.0)
    a = _call_ext(fn, p, 4) - p["residual"]
    b = _call_ext(fn, q, 4) - q["residual"]
    err = float(np.max(np.abs(a - b)))
    z = dict(p, W=np.zeros_like(p["W"]))
    err0 = float(np.max(np.abs(_call_ext(fn, z, 4) - (p["residual"] + p["b"][None, :, None]))))
    return err <= 1e-12 and err0 == 0.0, f"residual passthrough err {err:.3g}, W=0 err {err0:.3g}"


EXT_PINS = [ext_hand_golden, ext_brute_tiny, ext_torch_f64, ext_is_block_with_bn_outside,
            ext_residual_passthrough]


# --------------------------------------------------------------------------- train-mode BN pins

def _call_train(fn, p, d, momentum):
    out, rm, rv, m, v = fn(p["x"], p["running_mean"], p["running_var"], p["gamma"], p["beta"],
                           p["eps"], momentum, p["W"], p["b"], d)
    return _np(out), _np(rm), _np(rv), _np(m), _np(v)


def train_hand_golden(fn):
    g = json.load(open(os.path.join(GOLDEN, "prenorm_block_train_hand.json")))
    i = g["inputs"]
    p = {k: (_np(v) if isinstance(v, list) else v) for k, v in i.items()}
    out, rm, rv, m, v = _call_train(fn, p, i["d"], i["momentum"])
    err = max(_maxrel(out, g["expected"]), _maxrel(rm, g["expected_running_mean"]),
              _maxrel(rv, g["expected_running_var"]), _maxrel(m, g["expected_batch_mean"]),
              _maxrel(v, g["expected_batch_var"]))
    return err <= 1e-14, f"train hand golden max rel err {err:.3g}"


def train_torch_f64(fn):
    """torch float64 F.batch_norm(training=True) (which updates the running statistics in
    place), relu, conv1d, residual."""
    worst = 0.0
    for (N, C, L, d, mom, seed) in [(2, 16, 512, 128, 0.1, 1), (3, 24, 300, 7, 0.3, 2),
                                    (1, 8, 50, 60, 0.1, 3), (4, 12, 33, 1, 1.0, 4)]:
        p = _rand_block(N, C, L, seed, beta_shift=0.2)
        p["x"] = p["x"] * 1.7 + np.linspace(-1, 2, C)[None, :, None]
        t = lambda a: torch.from_numpy(np.array(a, dtype=np.float64))
        rm, rv = t(p["running_mean"]), t(p["running_var"])
        z = F.relu(F.batch_norm(t(p["x"]), rm, rv, t(p["gamma"]), t(p["beta"]), training=True,
                                momentum=mom, eps=p["eps"]))
        exp = t(p["x"]) + F.conv1d(z, t(p["W"]), t(p["b"]), padding=d, dilation=d)
        out, frm, frv, _, _ = _call_train(fn, p, d, mom)
        worst = max(worst, _maxrel(out, exp.numpy()), _maxrel(frm, rm.numpy()),
                    _maxrel(frv, rv.numpy()))
    return worst <= 1e-10, f"torch float64 training batch_norm max rel err {worst:.3g}"


def train_brute_tiny(fn):
    """Batch statistics by scalar loops, then the brute-force eval block with them."""
    worst = 0.0
    for (N, C, L, d, seed) in [(2, 3, 9, 2, 5), (1, 2, 7, 7, 6)]:
        p = _rand_block(N, C, L, seed, beta_shift=0.3)
        x = p["x"].tolist()
        mean, var = [], []
        for c in range(C):
            vals = [x[n][c][t] for n in range(N) for t in range(L)]
            m = sum(vals) / len(vals)
            mean.append(m)
            var.append(sum((v - m) ** 2 for v in vals) / len(vals))
        ref = brute.prenorm_block_brute(p["x"], np.array(mean), np.array(var), p["gamma"],
                                        p["beta"], p["eps"], p["W"], p["b"], d)
        out, _, _, m, v = _call_train(fn, p, d, 0.1)
        worst = max(worst, _maxrel(out, ref), _maxrel(m, mean), _maxrel(v, var))
    return worst <= 1e-12, f"train brute force max rel err {worst:.3g}"


def train_shift_invariance(fn):
    """Training-mode BN removes a per-channel constant: out(x + c) - (x + c) == out(x) - x."""
    p = _rand_block(2, 6, 40, 7)
    shift = np.linspace(-3, 5, 6)[None, :, None]
    q = dict(p, x=p["x"] + shift)
    o1 = _call_train(fn, p, 3, 0.1)[0] - p["x"]
    o2 = _call_train(fn, q, 3, 0.1)[0] - q["x"]
    err = float(np.max(np.abs(o1 - o2)))
    return err <= 1e-11, f"train shift invariance max abs err {err:.3g}"


def train_momentum_limits(fn):
    """momentum 0 keeps the running statistics; momentum 1 replaces them with the batch
    mean and the unbiased batch variance."""
    p = _rand_block(2, 5, 30, 8)
    _, rm0, rv0, _, _ = _call_train(fn, p, 2, 0.0)
    _, rm1, rv1, m, v = _call_train(fn, p, 2, 1.0)
    n = 2 * 30
    xs = p["x"].transpose(1, 0, 2).reshape(5, -1)
    err = max(float(np.max(np.abs(rm0 - p["running_mean"]))),
              float(np.max(np.abs(rv0 - p["running_var"]))),
              float(np.max(np.abs(rm1 - xs.mean(axis=1)))),
              float(np.max(np.abs(rv1 - xs.var(axis=1, ddof=1)))),
              float(np.max(np.abs(v * n / (n - 1) - xs.var(axis=1, ddof=1)))))
    return err <= 1e-12, f"momentum limits max abs err {err:.3g}"


TRAIN_PINS = [train_hand_golden, train_torch_f64, train_brute_tiny, train_shift_invariance,
              train_momentum_limits]


# --------------------------------------------------------------------------- GroupNorm pins

def _rand_gn(N, C_in, C_out, T, seed, bias=False):
    rng = np.random.default_rng(seed)
    return dict(x=rng.standard_normal((N, C_in, T)),
                W=rng.normal(0, 1 / math.sqrt(3 * C_in), (C_out, C_in, 3)),
                bias=rng.normal(0, 0.1, C_out) if bias else None,
                gamma=rng.uniform(0.5, 1.5, C_out), beta=rng.normal(0, 0.1, C_out), eps=1e-5)


def _call_gn(fn, p, G, padding=1, dilation=1):
    return _np(fn(p["x"], p["W"], p["bias"], p["gamma"], p["beta"], p["eps"], G,
                  padding, dilation))


def _torch_gn(p, G, padding=1, dilation=1):
    t = lambda a: None if a is None else torch.from_numpy(np.asarray(a, dtype=np.float64))
    y = F.conv1d(t(p["x"]), t(p["W"]), t(p["bias"]), padding=padding, dilation=dilation)
    return F.group_norm(y, G, t(p["gamma"]), t(p["beta"]), eps=p["eps"]).numpy()


def gn_hand_golden(fn):
    g = json.load(open(os.path.join(GOLDEN, "conv_groupnorm_hand.json")))
    i = g["inputs"]
    out = _np(fn(_np(i["x"]), _np(i["W"]), None, _np(i["gamma"]), _np(i["beta"]), i["eps"],
                 i["num_groups"], i["padding"], i["dilation"]))
    err = _maxrel(out, g["expected"])
    return err <= 1e-14, f"hand golden max rel err {err:.3g}"


def gn_brute_tiny(fn):
    worst = 0.0
    for (N, C_in, C_out, T, G, pad, dil, bias, seed) in [
            (1, 2, 4, 6, 2, 1, 1, False, 1), (2, 3, 6, 7, 3, 1, 1, True, 2),
            (1, 2, 4, 9, 1, 2, 2, False, 3), (2, 1, 4, 8, 4, 3, 1, True, 4),
            (1, 3, 6, 10, 2, 0, 2, False, 5)]:
        p = _rand_gn(N, C_in, C_out, T, seed, bias)
        ref = brute.conv_groupnorm_brute(p["x"], p["W"], p["bias"], p["gamma"], p["beta"],
                                         p["eps"], G, pad, dil)
        worst = max(worst, _maxrel(_call_gn(fn, p, G, pad, dil), ref))
    return worst <= 1e-11, f"GN brute force max rel err {worst:.3g}"


def gn_torch_f64(fn):
    worst = 0.0
    for (N, C_in, C_out, T, G, pad, dil, bias, seed) in [
            (16, 128, 256, 1024, 32, 1, 1, False, 11), (2, 16, 32, 77, 8, 1, 1, True, 12),
            (2, 12, 24, 50, 6, 3, 2, False, 13), (1, 8, 12, 33, 3, 0, 1, True, 14)]:
        p = _rand_gn(N, C_in, C_out, T, seed, bias)
        worst = max(worst, _maxrel(_call_gn(fn, p, G, pad, dil), _torch_gn(p, G, pad, dil)))
    return worst <= 1e-10, f"torch float64 conv1d/group_norm max rel err {worst:.3g}"


def gn_instance_and_layer_norm(fn):
    """G = C_out is instance norm per channel; G = 1 is layer norm over (C, T)."""
    p = _rand_gn(2, 6, 8, 40, 21)
    t = torch.from_numpy
    y = F.conv1d(t(p["x"]), t(p["W"]), None, padding=1)
    inst = F.instance_norm(y, eps=p["eps"]) * t(p["gamma"])[None, :, None] + t(p["beta"])[None, :, None]
    lay = F.layer_norm(y, y.shape[1:], eps=p["eps"]) * t(p["gamma"])[None, :, None] + t(p["beta"])[None, :, None]
    e1 = _maxrel(_call_gn(fn, p, 8), inst.numpy())
    e2 = _maxrel(_call_gn(fn, p, 1), lay.numpy())
    return max(e1, e2) <= 1e-10, f"instance_norm err {e1:.3g}, layer_norm err {e2:.3g}"


def gn_moments(fn):
    """gamma = 1, beta = 0: each (n, g) block of the output has mean 0 and biased
    variance v/(v + eps), where v is the block's variance before normalising."""
    p = _rand_gn(2, 5, 12, 30, 31)
    p.update(gamma=np.ones(12), beta=np.zeros(12), eps=0.3)
    G = 4
    out = _call_gn(fn, p, G).reshape(2, G, -1)
    y = F.conv1d(torch.from_numpy(p["x"]), torch.from_numpy(p["W"]), padding=1).numpy()
    v = y.reshape(2, G, -1).var(axis=2)
    e_mean = float(np.max(np.abs(out.mean(axis=2))))
    e_var = float(np.max(np.abs(out.var(axis=2) - v / (v + 0.3))))
    return max(e_mean, e_var) <= 1e-12, f"GN moments: mean err {e_mean:.3g}, var err {e_var:.3g}"


def gn_scale_invariance(fn):
    """GroupNorm(alpha*y; eps*alpha^2) == GroupNorm(y; eps) exactly in real arithmetic."""
    p = _rand_gn(2, 4, 8, 25, 41)
    a = 3.0
    q = dict(p, W=a * p["W"], eps=p["eps"] * a * a)
    err = _maxrel(_call_gn(fn, q, 2), _call_gn(fn, p, 2))
    return err <= 1e-12, f"scale invariance err {err:.3g}"


def gn_partial_affine_torch(fn):
    """gamma or beta absent on its own (None means gamma = 1 or beta = 0): torch float64
    group_norm with weight=None or bias=None, and the affine-free result scaled or shifted
    by hand (so a dropped or doubled beta, or a gamma applied to beta, fails)."""
    worst = 0.0
    for seed, drop in ((51, "gamma"), (52, "beta")):
        p = _rand_gn(2, 6, 12, 40, seed, bias=True)
        p[drop] = None
        worst = max(worst, _maxrel(_call_gn(fn, p, 4), _torch_gn(p, 4)))
        plain = _call_gn(fn, dict(p, gamma=None, beta=None), 4)
        if drop == "gamma":
            exp = plain + p["beta"][None, :, None]
        else:
            exp = plain * p["gamma"][None, :, None]
        worst = max(worst, _maxrel(_call_gn(fn, p, 4), exp))
    return worst <= 1e-12, f"partial affine max rel err {worst:.3g}"


GN_PINS = [gn_hand_golden, gn_brute_tiny, gn_torch_f64, gn_instance_and_layer_norm,
           gn_moments, gn_scale_invariance, gn_partial_affine_torch]
