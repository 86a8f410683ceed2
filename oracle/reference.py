"""Plain float64 CPU oracle for the pre-norm dilated Conv1d block and Conv1d+GroupNorm.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call anything in ``oracle/``.
The HIP library and its Python binding never touch it, and it shares no code with them.

Every function computes its definition directly, in float64 numpy, in the order the
source pages state it:

* Pre-norm residual block (POPCORNBENCH page "Kimi-K2.6__l2_p12", the pre-norm
  residual block problem; first turn): keep x as the residual, apply BatchNorm1d with
  the running statistics, then ReLU, then Conv1d C->C with kernel 3, dilation d and
  padding d (the conv pads its own input, i.e. after the ReLU), then add the residual.
* Conv1d + GroupNorm (POPCORNBENCH page "FW-GLM-5-1__l2_p35"; its single turn):
  Conv1d(k=3) with no bias, then GroupNorm with per-(sample, group) mean and biased
  variance over the group's channels and all time steps, then the affine gamma/beta.

The conv is written as PyTorch defines it: output t reads padded input t + k*dilation,
which is the unpadded input t - padding + k*dilation, zero outside the input
(FW-GLM-5-1__l2_p35, the conv index formula in its problem analysis). The zero
padding is materialised as an explicit zero-filled array so that padded taps are
exactly zero, not ReLU(BN(0)).

Parity status: every public function here is pinned by tests in
``tests/test_oracle_pins.py`` (hand-worked golden values, brute force, torch float64
library routines, closed forms and invariants).
"""
from __future__ import annotations

import numpy as np

KERNEL_SIZE = 3


def _f64(a):
    """Upcast to a float64 numpy array (accepts numpy arrays and CPU torch tensors;
    a bfloat16 tensor is taken at its exact value)."""
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().cpu()
        if str(a.dtype) == "torch.bfloat16":
            a = a.float()
        a = a.numpy()
    return np.asarray(a, dtype=np.float64)


def conv_output_length(L: int, padding: int, dilation: int,
                       kernel_size: int = KERNEL_SIZE, stride: int = 1) -> int:
    """Conv1d output length floor((L + 2p - d(k-1) - 1)/s + 1).

    Kimi-K2.6__l2_p12, first turn (output-length check for padding = dilation, which
    gives L_out = L); FW-GLM-5-1__l2_p35, the module's T_out expression.
    """
    return (L + 2 * padding - dilation * (kernel_size - 1) - 1) // stride + 1


def bn_eval_relu(x, running_mean, running_var, gamma, beta, eps):
    """ReLU(BatchNorm1d in eval mode), channel axis 1.

    Per channel c: normalise with the running statistics, (x - mean[c]) divided by
    sqrt(var[c] + eps), scale by gamma[c], shift by beta[c], then clamp below at 0.
    Kimi-K2.6__l2_p12, first turn: the per-channel fused BN/ReLU formula.
    """
    x = _f64(x)
    mean = _f64(running_mean)[None, :, None]
    var = _f64(running_var)[None, :, None]
    g = _f64(gamma)[None, :, None]
    b = _f64(beta)[None, :, None]
    normalised = (x - mean) / np.sqrt(var + float(eps))
    y = g * normalised + b
    return np.maximum(y, 0.0)


def zero_pad_time(a, padding: int):
    """Return a new array with `padding` zeros before and after the last (time) axis."""
    a = _f64(a)
    N, C, L = a.shape
    out = np.zeros((N, C, L + 2 * padding), dtype=np.float64)
    out[:, :, padding:padding + L] = a
    return out


def conv1d_k3_padded(xpad, W, bias, dilation: int, L_out: int):
    """Stride-1, kernel-3 Conv1d over an already zero-padded input.

    y[n, co, t] = bias[co] + sum_k sum_ci W[co, ci, k] * xpad[n, ci, t + k*dilation],
    i.e. the unpadded index t - padding + k*dilation (FW-GLM-5-1__l2_p35, conv index
    formula). Each tap k is one matrix product of W[:, :, k] (C_out x C_in) with the
    shifted window of the padded input; the three taps are summed.
    """
    xpad = _f64(xpad)
    W = _f64(W)
    N, C_in, _ = xpad.shape
    C_out = W.shape[0]
    assert W.shape == (C_out, C_in, KERNEL_SIZE), W.shape
    y = np.zeros((N, C_out, L_out), dtype=np.float64)
    for k in range(KERNEL_SIZE):
        Wk = np.ascontiguousarray(W[:, :, k])   # layout only: BLAS wants unit stride
        window = xpad[:, :, k * dilation:k * dilation + L_out]
        y += np.matmul(Wk, window)
    if bias is not None:
        y += _f64(bias)[None, :, None]
    return y


def prenorm_block(x, running_mean, running_var, gamma, beta, eps, W, b, d: int):
    """out = x + Conv1d_{k=3, dilation=d, padding=d}(ReLU(BatchNorm1d_eval(x))).

    Kimi-K2.6__l2_p12, first turn: residual kept from the input, BN with running
    statistics, ReLU, C->C conv (kernel 3, padding = dilation = d, groups 1, with
    bias), residual added. ``b`` may be None (no conv bias).
    """
    x64 = _f64(x)
    N, C, L = x64.shape
    z = bn_eval_relu(x64, running_mean, running_var, gamma, beta, eps)
    zpad = zero_pad_time(z, d)                      # pad AFTER the ReLU
    L_out = conv_output_length(L, padding=d, dilation=d)
    y = conv1d_k3_padded(zpad, W, b, d, L_out)
    assert y.shape == x64.shape, (y.shape, x64.shape)
    return x64 + y


def prenorm_block_points(x, running_mean, running_var, gamma, beta, eps, W, b, d: int,
                         points):
    """The same block, evaluated only at the listed output points (n, co, t).

    For each point: out = x[n, co, t] + b[co] + sum_k W[co, :, k] . z[n, :, t-d+k*d],
    where z = ReLU(BN_eval(x)) and a tap outside [0, L) contributes 0 (the zero padding
    of the conv input). Used to check full-size runs on a sample of outputs; x and W are
    only indexed (one column of x and one row of W per tap), so they may be any array-like
    that supports that, including tensors too large to upcast whole.
    """
    xs = x
    b64 = None if b is None else _f64(b)
    rm, rv = _f64(running_mean), _f64(running_var)
    g, be = _f64(gamma), _f64(beta)
    N, C, L = tuple(xs.shape)
    pts = np.asarray(points, dtype=np.int64).reshape(-1, 3)
    out = np.empty(len(pts), dtype=np.float64)
    for i, (n, co, t) in enumerate(pts):
        acc = 0.0 if b64 is None else b64[co]
        for k in range(KERNEL_SIZE):
            t_in = t - d + k * d
            if 0 <= t_in < L:
                col = _f64(xs[n, :, t_in])                      # all input channels
                normalised = (col - rm) / np.sqrt(rv + float(eps))
                z = np.maximum(g * normalised + be, 0.0)
                acc += float(np.dot(_f64(W[co, :, k]), z))      # one row of W at a time
        out[i] = float(_f64(xs[n, co, t])) + acc
    return out


def relu_conv_residual(xn, W, b, residual, d: int):
    """out = residual + Conv1d_{k=3, dilation=d, padding=d}(ReLU(xn)).

    The block with its normalisation done by the caller (POPCORNBENCH "Kimi-K2.6__l2_p12",
    correctness-debugging turn: the fallback that leaves BN to the framework, so that it
    follows the module's train/eval mode, and fuses ReLU, the conv and the residual add
    from the block's input, passed separately). The conv input is zero-padded after
    the ReLU, as in prenorm_block.
    """
    xn64 = _f64(xn)
    N, C, L = xn64.shape
    z = np.maximum(xn64, 0.0)
    zpad = zero_pad_time(z, d)
    L_out = conv_output_length(L, padding=d, dilation=d)
    y = conv1d_k3_padded(zpad, W, b, d, L_out)
    res = _f64(residual)
    assert res.shape == y.shape, (res.shape, y.shape)
    return res + y


def batch_stats(x):
    """Per-channel batch mean and biased variance over the batch and time axes, taken
    two-pass in float64 (POPCORNBENCH "Kimi-K2.6__l2_p97", BatchNorm in training mode:
    normalise with the batch mean and the biased variance)."""
    x = _f64(x)
    mean = x.mean(axis=(0, 2))
    var = ((x - mean[None, :, None]) ** 2).mean(axis=(0, 2))
    return mean, var


def running_stats_update(running_mean, running_var, batch_mean, batch_var, count: int,
                         momentum: float):
    """Training-mode update of the running statistics: an exponential average with weight
    `momentum` on the new batch, where the running variance takes the unbiased batch
    variance var * n / (n - 1) (Kimi-K2.6__l2_p97, first turn: running_var is updated
    with the n/(n-1)-corrected variance, momentum 0.1)."""
    m = float(momentum)
    rm = (1.0 - m) * _f64(running_mean) + m * _f64(batch_mean)
    rv = (1.0 - m) * _f64(running_var) + m * _f64(batch_var) * count / (count - 1)
    return rm, rv


def prenorm_block_train(x, running_mean, running_var, gamma, beta, eps, momentum, W, b,
                        d: int):
    """The pre-norm block with BatchNorm1d in training mode.

    BN uses the batch statistics of x (mean and biased variance per channel over N and L)
    instead of the running ones; the rest of the block is prenorm_block's. Also returns
    the updated running statistics and the batch statistics:
    (out, new_running_mean, new_running_var, batch_mean, batch_var).
    Kimi-K2.6__l2_p12, correctness-debugging turn: the batch-statistics hypothesis for
    the block (mean over batch and time, unbiased=False); Kimi-K2.6__l2_p97: training-mode
    semantics and the running-statistics update.
    """
    x64 = _f64(x)
    N, C, L = x64.shape
    mean, var = batch_stats(x64)
    out = prenorm_block(x64, mean, var, gamma, beta, eps, W, b, d)
    rm, rv = running_stats_update(running_mean, running_var, mean, var, N * L, momentum)
    return out, rm, rv, mean, var


def group_norm(y, num_groups: int, gamma, beta, eps):
    """GroupNorm over (N, C, T): groups are contiguous channel blocks of C/num_groups.

    For each (n, g): mean and biased variance (divide by the element count) over the
    group's channels and all time steps, both taken two-pass in float64; then
    (y - mean)/sqrt(var + eps), then gamma[c]*. + beta[c] (FW-GLM-5-1__l2_p35,
    GroupNorm definition and its normalise kernel). That kernel applies gamma and beta
    together, or neither when gamma is absent; each may be None here on its own, meaning
    gamma = 1 or beta = 0 (PyTorch's group_norm convention, an extension of the page).
    """
    y = _f64(y)
    N, C, T = y.shape
    assert C % num_groups == 0
    cpg = C // num_groups
    yg = y.reshape(N, num_groups, cpg * T)
    mean = yg.mean(axis=2, keepdims=True)
    var = ((yg - mean) ** 2).mean(axis=2, keepdims=True)
    yhat = ((yg - mean) / np.sqrt(var + float(eps))).reshape(N, C, T)
    if gamma is not None:
        yhat = yhat * _f64(gamma)[None, :, None]
    if beta is not None:
        yhat = yhat + _f64(beta)[None, :, None]
    return yhat


def conv_groupnorm(x, W, bias, gamma, beta, eps, num_groups: int,
                   padding: int = 1, dilation: int = 1):
    """GroupNorm(Conv1d_{k=3, stride 1}(x)) (FW-GLM-5-1__l2_p35 problem statement:
    kernel 3, stride 1, padding 1, dilation 1, no bias, then GroupNorm)."""
    x64 = _f64(x)
    N, C_in, T = x64.shape
    T_out = conv_output_length(T, padding=padding, dilation=dilation)
    assert T_out >= 1
    xpad = zero_pad_time(x64, padding)
    y = conv1d_k3_padded(xpad, W, bias, dilation, T_out)
    return group_norm(y, num_groups, gamma, beta, eps)
