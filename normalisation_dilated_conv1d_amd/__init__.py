"""MI355X (gfx950) library for the fused pre-norm dilated Conv1d block and Conv1d+GroupNorm.

The compute lives in the HIP shared library ``libdconv1d.so`` (C ABI, ``include/dconv1d.h``).
This module is only its Python binding: it checks tensors, allocates outputs with torch
and passes device pointers plus torch's current HIP stream to the C entry points of the
same names. There is no fallback: if the library is not built, every call raises.

Build it with ``python -m normalisation_dilated_conv1d_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdconv1d.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "dconv1d.h")

DCONV1D_OK = 0
DCONV1D_EINVAL = -1
DCONV1D_EALIAS = -2
DCONV1D_EHIP = -3
DCONV1D_ENOMEM = -4

_lib = None


class Dconv1dError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"dconv1d error {code}: {message}")
        self.code = code


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdconv1d.so and declare its C signatures. Raises if it is not built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library not built: {path} is missing "
                           "(run python -m normalisation_dilated_conv1d_amd.build)")
    lib = ctypes.CDLL(path)
    P, F, I64, S = ctypes.c_void_p, ctypes.c_float, ctypes.c_int64, ctypes.c_void_p
    lib.prenorm_dconv1d_fwd.argtypes = [P, P, P, P, P, F, P, P, P, I64, I64, I64, I64, S]
    lib.prenorm_dconv1d_fwd.restype = ctypes.c_int
    lib.prenorm_dconv1d_fwd_noalloc.argtypes = [P, P, P, P, P, F, P, P, P, I64, I64, I64, I64, S]
    lib.prenorm_dconv1d_fwd_noalloc.restype = ctypes.c_int
    lib.prenorm_dconv1d_fwd_bf16.argtypes = [P, P, P, P, P, F, P, P, P, I64, I64, I64, I64, S]
    lib.prenorm_dconv1d_fwd_bf16.restype = ctypes.c_int
    train_args = [P, P, P, P, P, F, F, P, P, P, P, P, I64, I64, I64, I64, S]
    lib.prenorm_dconv1d_fwd_train.argtypes = train_args
    lib.prenorm_dconv1d_fwd_train.restype = ctypes.c_int
    lib.prenorm_dconv1d_fwd_train_bf16.argtypes = train_args
    lib.prenorm_dconv1d_fwd_train_bf16.restype = ctypes.c_int
    ext_args = [P, P, P, P, P, I64, I64, I64, I64, S]
    lib.relu_dconv1d_residual_fwd.argtypes = ext_args
    lib.relu_dconv1d_residual_fwd.restype = ctypes.c_int
    lib.relu_dconv1d_residual_fwd_bf16.argtypes = ext_args
    lib.relu_dconv1d_residual_fwd_bf16.restype = ctypes.c_int
    lib.conv1d_groupnorm_fwd.argtypes = [P, P, P, P, P, F, I64, P, I64, I64, I64, I64, I64, I64, S]
    lib.conv1d_groupnorm_fwd.restype = ctypes.c_int
    lib.dconv1d_last_error.argtypes = []
    lib.dconv1d_last_error.restype = ctypes.c_char_p
    lib.dconv1d_release.argtypes = []
    lib.dconv1d_release.restype = None
    lib.dconv1d_timer_enable.argtypes = [ctypes.c_int]
    lib.dconv1d_timer_enable.restype = ctypes.c_int
    lib.dconv1d_timer_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    lib.dconv1d_timer_read.restype = ctypes.c_int
    lib.dconv1d_block_method.argtypes = [I64, I64, I64, I64]
    lib.dconv1d_block_method.restype = ctypes.c_int
    lib.dconv1d_groupnorm_method.argtypes = [ctypes.c_void_p, ctypes.c_void_p] + [I64] * 7
    lib.dconv1d_groupnorm_method.restype = ctypes.c_int
    if path == LIB_PATH:
        _lib = lib
    return lib


def header_functions(path: str = HEADER_PATH) -> list[str]:
    """Names of the functions include/dconv1d.h declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


def _check(code: int) -> None:
    if code != DCONV1D_OK:
        msg = _lib.dconv1d_last_error().decode() if _lib is not None else ""
        raise Dconv1dError(code, msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev_tensor(name, t, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _prenorm(fn_name, x, running_mean, running_var, gamma, beta, eps, W, b, d, out, xdtype):
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be (N, C, L)")
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    N, C, L = x.shape
    dev = x.device
    _dev_tensor("x", x, xdtype, (N, C, L), dev)
    for name, t in (("running_mean", running_mean), ("running_var", running_var),
                    ("gamma", gamma), ("beta", beta)):
        _dev_tensor(name, t, torch.float32, (C,), dev)
    _dev_tensor("W", W, torch.float32, (C, C, 3), dev)
    if b is not None:
        _dev_tensor("b", b, torch.float32, (C,), dev)
    if out is None:
        out = torch.empty_like(x)
    else:
        _dev_tensor("out", out, xdtype, (N, C, L), dev)
    with torch.cuda.device(dev):
        code = getattr(lib, fn_name)(_ptr(x), _ptr(running_mean), _ptr(running_var), _ptr(gamma),
                                     _ptr(beta), float(eps), _ptr(W), _ptr(b), _ptr(out),
                                     N, C, L, int(d), _stream(dev))
    _check(code)
    return out


def prenorm_dconv1d_fwd(x, running_mean, running_var, gamma, beta, eps, W, b, d, out=None):
    """out = x + Conv1d_{k=3, dilation=d, padding=d}(ReLU(BatchNorm1d_eval(x))), float32.

    x: (N, C, L) float32 device tensor; BN vectors (C,); W (C, C, 3); b (C,) or None.
    Runs on torch's current stream of x's device; returns ``out`` (allocated if None)."""
    return _prenorm("prenorm_dconv1d_fwd", x, running_mean, running_var, gamma, beta, eps, W,
                    b, d, out, torch.float32)


def prenorm_dconv1d_fwd_noalloc(x, running_mean, running_var, gamma, beta, eps, W, b, d,
                                out=None):
    """prenorm_dconv1d_fwd through the entry point that allocates no device memory (its
    scratch is a fixed array inside the library; C <= 512). Pass ``out`` to keep the call
    free of allocations on the torch side too."""
    return _prenorm("prenorm_dconv1d_fwd_noalloc", x, running_mean, running_var, gamma, beta,
                    eps, W, b, d, out, torch.float32)


def prenorm_dconv1d_fwd_bf16(x, running_mean, running_var, gamma, beta, eps, W, b, d, out=None):
    """The same block with bfloat16 x and out (float32 parameters, float32 accumulation)."""
    return _prenorm("prenorm_dconv1d_fwd_bf16", x, running_mean, running_var, gamma, beta, eps,
                    W, b, d, out, torch.bfloat16)


def _prenorm_train(fn_name, x, running_mean, running_var, gamma, beta, eps, momentum, W, b, d,
                   out, save_mean, save_invstd, xdtype):
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be (N, C, L)")
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    N, C, L = x.shape
    dev = x.device
    _dev_tensor("x", x, xdtype, (N, C, L), dev)
    for name, t in (("running_mean", running_mean), ("running_var", running_var),
                    ("save_mean", save_mean), ("save_invstd", save_invstd)):
        if t is not None:
            _dev_tensor(name, t, torch.float32, (C,), dev)
    for name, t in (("gamma", gamma), ("beta", beta)):
        _dev_tensor(name, t, torch.float32, (C,), dev)
    _dev_tensor("W", W, torch.float32, (C, C, 3), dev)
    if b is not None:
        _dev_tensor("b", b, torch.float32, (C,), dev)
    if out is None:
        out = torch.empty_like(x)
    else:
        _dev_tensor("out", out, xdtype, (N, C, L), dev)
    with torch.cuda.device(dev):
        code = getattr(lib, fn_name)(_ptr(x), _ptr(running_mean), _ptr(running_var), _ptr(gamma),
                                     _ptr(beta), float(eps), float(momentum), _ptr(W), _ptr(b),
                                     _ptr(out), _ptr(save_mean), _ptr(save_invstd), N, C, L,
                                     int(d), _stream(dev))
    _check(code)
    return out


def prenorm_dconv1d_fwd_train(x, running_mean, running_var, gamma, beta, eps, momentum, W, b, d,
                              out=None, save_mean=None, save_invstd=None):
    """The float32 block with BatchNorm1d in training mode (batch statistics over N and L).

    running_mean / running_var (C,) are updated in place when given (both or neither);
    save_mean / save_invstd (C,), when given, receive the batch mean and 1/sqrt(var+eps).
    Returns ``out``."""
    return _prenorm_train("prenorm_dconv1d_fwd_train", x, running_mean, running_var, gamma,
                          beta, eps, momentum, W, b, d, out, save_mean, save_invstd,
                          torch.float32)


def prenorm_dconv1d_fwd_train_bf16(x, running_mean, running_var, gamma, beta, eps, momentum, W,
                                   b, d, out=None, save_mean=None, save_invstd=None):
    """The training-mode block with bfloat16 x and out."""
    return _prenorm_train("prenorm_dconv1d_fwd_train_bf16", x, running_mean, running_var, gamma,
                          beta, eps, momentum, W, b, d, out, save_mean, save_invstd,
                          torch.bfloat16)


def _relu_residual(fn_name, xn, W, b, residual, d, out, xdtype):
    lib = load_library()
    if xn.dim() != 3:
        raise ValueError("xn must be (N, C, L)")
    if not xn.is_cuda:
        raise ValueError("xn must be a device tensor")
    N, C, L = xn.shape
    dev = xn.device
    _dev_tensor("xn", xn, xdtype, (N, C, L), dev)
    _dev_tensor("residual", residual, xdtype, (N, C, L), dev)
    _dev_tensor("W", W, torch.float32, (C, C, 3), dev)
    if b is not None:
        _dev_tensor("b", b, torch.float32, (C,), dev)
    if out is None:
        out = torch.empty_like(xn)
    else:
        _dev_tensor("out", out, xdtype, (N, C, L), dev)
    with torch.cuda.device(dev):
        code = getattr(lib, fn_name)(_ptr(xn), _ptr(W), _ptr(b), _ptr(residual), _ptr(out), N, C,
                                     L, int(d), _stream(dev))
    _check(code)
    return out


def relu_dconv1d_residual_fwd(xn, W, b, residual, d, out=None):
    """out = residual + Conv1d_{k=3, dilation=d, padding=d}(ReLU(xn)), float32, with the
    normalisation done by the caller. ``out`` may be ``residual`` (in-place add)."""
    return _relu_residual("relu_dconv1d_residual_fwd", xn, W, b, residual, d, out, torch.float32)


def relu_dconv1d_residual_fwd_bf16(xn, W, b, residual, d, out=None):
    """The same with bfloat16 xn, residual and out."""
    return _relu_residual("relu_dconv1d_residual_fwd_bf16", xn, W, b, residual, d, out,
                          torch.bfloat16)


def conv1d_groupnorm_fwd(x, W, bias, gamma, beta, eps, num_groups, padding=1, dilation=1,
                         out=None):
    """GroupNorm(Conv1d_{k=3, stride 1, padding, dilation}(x)), float32.

    x: (N, C_in, T); W: (C_out, C_in, 3); bias, gamma, beta: (C_out,) or None.
    Returns ``out`` of shape (N, C_out, T + 2*padding - 2*dilation)."""
    lib = load_library()
    if x.dim() != 3 or W.dim() != 3:
        raise ValueError("x must be (N, C_in, T) and W (C_out, C_in, 3)")
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    N, C_in, T = x.shape
    C_out = W.shape[0]
    dev = x.device
    _dev_tensor("x", x, torch.float32, (N, C_in, T), dev)
    _dev_tensor("W", W, torch.float32, (C_out, C_in, 3), dev)
    for name, t in (("bias", bias), ("gamma", gamma), ("beta", beta)):
        if t is not None:
            _dev_tensor(name, t, torch.float32, (C_out,), dev)
    T_out = T + 2 * int(padding) - 2 * int(dilation)
    if out is None:
        out = torch.empty((N, C_out, max(T_out, 0)), dtype=torch.float32, device=dev)
    else:
        _dev_tensor("out", out, torch.float32, (N, C_out, T_out), dev)
    with torch.cuda.device(dev):
        code = lib.conv1d_groupnorm_fwd(_ptr(x), _ptr(W), _ptr(bias), _ptr(gamma), _ptr(beta),
                                        float(eps), int(num_groups), _ptr(out), N, C_in, C_out, T,
                                        int(padding), int(dilation), _stream(dev))
    _check(code)
    return out


DCONV1D_METHOD_DIRECT = 0
DCONV1D_METHOD_WINOGRAD = 1


def dconv1d_block_method(N: int, C: int, L: int, d: int) -> int:
    """Which form of the conv a float32 block call of shape (N, C, L) and dilation d
    takes: DCONV1D_METHOD_WINOGRAD or DCONV1D_METHOD_DIRECT (host only, no GPU needed)."""
    code = load_library().dconv1d_block_method(int(N), int(C), int(L), int(d))
    if code < 0:
        _check(code)
    return code


def dconv1d_groupnorm_method(N: int, C_in: int, C_out: int, T: int, num_groups: int,
                             padding: int, dilation: int, x=None, W=None) -> int:
    """Which form of the conv conv1d_groupnorm_fwd takes for these sizes and, when given,
    the alignment of the tensors x and W (None: aligned like every allocation):
    DCONV1D_METHOD_WINOGRAD or DCONV1D_METHOD_DIRECT (host only, no GPU needed)."""
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    code = load_library().dconv1d_groupnorm_method(ptr(x), ptr(W), int(num_groups), int(N),
                                                   int(C_in), int(C_out), int(T), int(padding),
                                                   int(dilation))
    if code < 0:
        _check(code)
    return code


def release() -> None:
    """Free the library's per-device workspace."""
    load_library().dconv1d_release()


class KernelTimer:
    """HIP-event timing of the dominant conv kernel of every call made while active."""

    def __enter__(self):
        _check(load_library().dconv1d_timer_enable(1))
        return self

    def read(self):
        ms, n = ctypes.c_double(), ctypes.c_int64()
        _check(load_library().dconv1d_timer_read(ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value

    def __exit__(self, *exc):
        load_library().dconv1d_timer_enable(0)
        return False
