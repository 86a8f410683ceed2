"""Pure-Python scalar-loop versions of the two operations, for tiny inputs only.

TEST INFRASTRUCTURE, NOT PRODUCT CODE (same import rule as ``oracle/reference.py``).

These loops restate the PyTorch Conv1d definition one output element at a time, with
the zero padding expressed as a bounds test on the unpadded input index
t - padding + k*dilation instead of a padded array, and GroupNorm statistics as
explicit two-pass sums. They share nothing with ``reference.py`` beyond the
definitions, so agreement between the two pins the vectorised oracle's indexing,
padding and reductions. Sources: POPCORNBENCH "Kimi-K2.6__l2_p12" first turn (block
definition and BN/ReLU formula); "FW-GLM-5-1__l2_p35" problem analysis (conv index
formula, GroupNorm statistics).
"""
from __future__ import annotations

import math


def _tolist(a):
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().cpu()
        if str(a.dtype) == "torch.bfloat16":
            a = a.float()
        a = a.double().tolist()
    elif hasattr(a, "tolist"):
        a = a.astype("float64").tolist()
    return a


def prenorm_block_brute(x, running_mean, running_var, gamma, beta, eps, W, b, d):
    x, W = _tolist(x), _tolist(W)
    rm, rv = _tolist(running_mean), _tolist(running_var)
    ga, be = _tolist(gamma), _tolist(beta)
    bb = _tolist(b)
    N, C, L = len(x), len(x[0]), len(x[0][0])
    pad = d
    out = [[[0.0] * L for _ in range(C)] for _ in range(N)]
    for n in range(N):
        # activation z = relu(bn(x)) of every in-range input position
        z = [[max(ga[c] * (x[n][c][t] - rm[c]) / math.sqrt(rv[c] + eps) + be[c], 0.0)
              for t in range(L)] for c in range(C)]
        for co in range(C):
            for t in range(L):
                acc = 0.0 if bb is None else bb[co]
                for ci in range(C):
                    for k in range(3):
                        t_in = t - pad + k * d
                        if 0 <= t_in < L:
                            acc += W[co][ci][k] * z[ci][t_in]
                out[n][co][t] = x[n][co][t] + acc
    return out


def relu_conv_residual_brute(xn, W, b, residual, d):
    xn, W, r = _tolist(xn), _tolist(W), _tolist(residual)
    bb = _tolist(b)
    N, C, L = len(xn), len(xn[0]), len(xn[0][0])
    out = [[[0.0] * L for _ in range(C)] for _ in range(N)]
    for n in range(N):
        for co in range(C):
            for t in range(L):
                acc = 0.0 if bb is None else bb[co]
                for ci in range(C):
                    for k in range(3):
                        t_in = t - d + k * d
                        if 0 <= t_in < L:
                            acc += W[co][ci][k] * max(xn[n][ci][t_in], 0.0)
                out[n][co][t] = r[n][co][t] + acc
    return out


def conv_groupnorm_brute(x, W, bias, gamma, beta, eps, num_groups, padding=1, dilation=1):
    x, W = _tolist(x), _tolist(W)
    bias, gamma, beta = _tolist(bias), _tolist(gamma), _tolist(beta)
    N, C_in, T = len(x), len(x[0]), len(x[0][0])
    C_out = len(W)
    T_out = T + 2 * padding - 2 * dilation
    cpg = C_out // num_groups
    y = [[[0.0] * T_out for _ in range(C_out)] for _ in range(N)]
    for n in range(N):
        for co in range(C_out):
            for t in range(T_out):
                acc = 0.0 if bias is None else bias[co]
                for ci in range(C_in):
                    for k in range(3):
                        t_in = t - padding + k * dilation
                        if 0 <= t_in < T:
                            acc += x[n][ci][t_in] * W[co][ci][k]
                y[n][co][t] = acc
    out = [[[0.0] * T_out for _ in range(C_out)] for _ in range(N)]
    for n in range(N):
        for g in range(num_groups):
            chans = range(g * cpg, (g + 1) * cpg)
            count = cpg * T_out
            s = 0.0
            for c in chans:
                for t in range(T_out):
                    s += y[n][c][t]
            mean = s / count
            q = 0.0
            for c in chans:
                for t in range(T_out):
                    q += (y[n][c][t] - mean) ** 2
            var = q / count
            inv = 1.0 / math.sqrt(var + eps)
            for c in chans:
                for t in range(T_out):
                    v = (y[n][c][t] - mean) * inv
                    if gamma is not None:
                        v = v * gamma[c]
                    if beta is not None:
                        v = v + beta[c]
                    out[n][c][t] = v
    return out
