"""The C-ABI library loads and exports every function include/dconv1d.h declares, and
rejects invalid arguments on the host before any HIP call. CPU only: every call here
fails validation (or is an empty batch), so no device work is issued."""
import ctypes

import pytest

import normalisation_dilated_conv1d_amd as dc

pytestmark = pytest.mark.skipif(not __import__("os").path.exists(dc.LIB_PATH),
                                reason="libdconv1d.so not built")

EXPECTED = {"prenorm_dconv1d_fwd", "prenorm_dconv1d_fwd_noalloc", "prenorm_dconv1d_fwd_bf16", "prenorm_dconv1d_fwd_train",
            "prenorm_dconv1d_fwd_train_bf16", "relu_dconv1d_residual_fwd",
            "relu_dconv1d_residual_fwd_bf16", "conv1d_groupnorm_fwd",
            "dconv1d_last_error", "dconv1d_release", "dconv1d_timer_enable",
            "dconv1d_timer_read", "dconv1d_block_method", "dconv1d_groupnorm_method"}

FAKE_X = 0x10000000
FAKE_OUT = 0x20000000
FAKE_P = 0x30000000



def test_header_declares_expected_functions():
    assert set(dc.header_functions()) == EXPECTED


def test_every_declared_symbol_is_exported():
    lib = dc.load_library()
    for name in dc.header_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def _block(lib, x=FAKE_X, out=FAKE_OUT, N=2, C=16, L=512, d=128, eps=1e-5, b=FAKE_P, W=FAKE_P,
           rm=FAKE_P, fn="prenorm_dconv1d_fwd"):
    return getattr(lib, fn)(x, rm, FAKE_P, FAKE_P, FAKE_P, eps, W, b, out, N, C, L, d, None)


@pytest.mark.parametrize("fn", ["prenorm_dconv1d_fwd", "prenorm_dconv1d_fwd_noalloc",
                                "prenorm_dconv1d_fwd_bf16"])
@pytest.mark.parametrize("kw,code", [
    (dict(x=None), dc.DCONV1D_EINVAL), (dict(out=None), dc.DCONV1D_EINVAL),
    (dict(W=None), dc.DCONV1D_EINVAL), (dict(rm=None), dc.DCONV1D_EINVAL),
    (dict(N=-1), dc.DCONV1D_EINVAL), (dict(C=0), dc.DCONV1D_EINVAL),
    (dict(L=0), dc.DCONV1D_EINVAL), (dict(d=0), dc.DCONV1D_EINVAL),
    (dict(eps=-1.0), dc.DCONV1D_EINVAL), (dict(eps=float("nan")), dc.DCONV1D_EINVAL),
    (dict(C=100000), dc.DCONV1D_EINVAL), (dict(C=16384, L=1 << 18), dc.DCONV1D_EINVAL),
    (dict(out=FAKE_X), dc.DCONV1D_EALIAS), (dict(out="last_element"), dc.DCONV1D_EALIAS),
    (dict(N=0), dc.DCONV1D_OK), (dict(N=0, x=None, out=None), dc.DCONV1D_OK),
])
def test_block_validation(fn, kw, code):
    lib = dc.load_library()
    elem = 2 if fn.endswith("bf16") else 4
    nbytes = elem * 2 * 16 * 512
    if kw.get("out") == "last_element":
        kw = dict(out=FAKE_X + nbytes - elem)
    assert _block(lib, fn=fn, **kw) == code
    if code != dc.DCONV1D_OK:
        assert lib.dconv1d_last_error().decode()


def test_block_null_bias_is_valid_argument():
    lib = dc.load_library()
    # an empty batch with b = NULL passes validation and issues no work
    assert _block(lib, N=0, b=None) == dc.DCONV1D_OK


FAKE_RM = 0x40000000
FAKE_RV = 0x40001000


def _train(lib, fn="prenorm_dconv1d_fwd_train", x=FAKE_X, out=FAKE_OUT, rm=FAKE_RM, rv=FAKE_RV,
           sm=None, si=None, N=2, C=16, L=512, d=128, eps=1e-5, mom=0.1, W=FAKE_P):
    return getattr(lib, fn)(x, rm, rv, FAKE_P, FAKE_P, eps, mom, W, None, out, sm, si, N, C, L,
                            d, None)


@pytest.mark.parametrize("fn", ["prenorm_dconv1d_fwd_train", "prenorm_dconv1d_fwd_train_bf16"])
@pytest.mark.parametrize("kw,code", [
    (dict(x=None), dc.DCONV1D_EINVAL), (dict(out=None), dc.DCONV1D_EINVAL),
    (dict(W=None), dc.DCONV1D_EINVAL), (dict(rm=None), dc.DCONV1D_EINVAL),
    (dict(rv=None), dc.DCONV1D_EINVAL), (dict(mom=float("nan")), dc.DCONV1D_EINVAL),
    (dict(mom=float("inf")), dc.DCONV1D_EINVAL),
    (dict(N=1, L=1), dc.DCONV1D_EINVAL),                 # one value per channel
    (dict(rm=FAKE_OUT + 64), dc.DCONV1D_EALIAS), (dict(sm=FAKE_X), dc.DCONV1D_EALIAS),
    (dict(si=FAKE_RV + 32), dc.DCONV1D_EALIAS), (dict(out=FAKE_X + 8), dc.DCONV1D_EALIAS),
    (dict(N=0), dc.DCONV1D_OK), (dict(N=0, x=None, out=None, rm=None, rv=None), dc.DCONV1D_OK),
    (dict(N=0, rm=None, rv=None, sm=FAKE_P, si=FAKE_P + 4096), dc.DCONV1D_OK),
])
def test_train_validation(fn, kw, code):
    lib = dc.load_library()
    assert _train(lib, fn=fn, **kw) == code
    if code != dc.DCONV1D_OK:
        assert lib.dconv1d_last_error().decode()


FAKE_RES = 0x50000000


def _ext(lib, fn="relu_dconv1d_residual_fwd", xn=FAKE_X, res=FAKE_RES, out=FAKE_OUT, W=FAKE_P,
         N=2, C=16, L=512, d=128):
    return getattr(lib, fn)(xn, W, None, res, out, N, C, L, d, None)


@pytest.mark.parametrize("fn", ["relu_dconv1d_residual_fwd", "relu_dconv1d_residual_fwd_bf16"])
@pytest.mark.parametrize("kw,code", [
    (dict(xn=None), dc.DCONV1D_EINVAL), (dict(res=None), dc.DCONV1D_EINVAL),
    (dict(out=None), dc.DCONV1D_EINVAL), (dict(W=None), dc.DCONV1D_EINVAL),
    (dict(d=0), dc.DCONV1D_EINVAL), (dict(L=0), dc.DCONV1D_EINVAL),
    (dict(out=FAKE_X + 64), dc.DCONV1D_EALIAS),           # out overlaps xn
    (dict(out=FAKE_RES + 64), dc.DCONV1D_EALIAS),         # shifted view of residual
    (dict(N=0), dc.DCONV1D_OK), (dict(N=0, xn=None, res=None, out=None), dc.DCONV1D_OK),
    (dict(N=0, out=FAKE_RES), dc.DCONV1D_OK),             # in-place residual is allowed
    (dict(N=0, res=FAKE_X), dc.DCONV1D_OK),               # residual may be xn
])
def test_external_bn_validation(fn, kw, code):
    lib = dc.load_library()
    assert _ext(lib, fn=fn, **kw) == code
    if code != dc.DCONV1D_OK:
        assert lib.dconv1d_last_error().decode()


def _gn(lib, x=FAKE_X, out=FAKE_OUT, N=16, C_in=128, C_out=256, T=1024, G=32, p=1, dil=1,
        eps=1e-5, W=FAKE_P):
    return lib.conv1d_groupnorm_fwd(x, W, None, None, None, eps, G, out, N, C_in, C_out, T, p,
                                    dil, None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), dc.DCONV1D_EINVAL), (dict(W=None), dc.DCONV1D_EINVAL),
    (dict(out=None), dc.DCONV1D_EINVAL), (dict(G=0), dc.DCONV1D_EINVAL),
    (dict(G=3), dc.DCONV1D_EINVAL), (dict(T=0), dc.DCONV1D_EINVAL),
    (dict(p=-1), dc.DCONV1D_EINVAL), (dict(dil=0), dc.DCONV1D_EINVAL),
    (dict(T=4, p=0, dil=2), dc.DCONV1D_EINVAL), (dict(eps=float("inf")), dc.DCONV1D_EINVAL),
    (dict(out=FAKE_X + 1024), dc.DCONV1D_EALIAS), (dict(N=0), dc.DCONV1D_OK),
    (dict(N=0, x=None, out=None), dc.DCONV1D_OK),
])
def test_groupnorm_validation(kw, code):
    lib = dc.load_library()
    assert _gn(lib, **kw) == code


def test_last_error_is_cleared_on_success():
    lib = dc.load_library()
    assert _block(lib, C=0) == dc.DCONV1D_EINVAL
    assert b"C must be" in lib.dconv1d_last_error()
    assert _block(lib, N=0) == dc.DCONV1D_OK
    assert lib.dconv1d_last_error() == b""


@pytest.mark.parametrize("N,C,L,d,method", [
    # Winograd when 3 * pairs <= 2 * L, pairs = ceil(L / 2e) * e, e = min(d, L), and at
    # least 160 workgroups
    (32, 256, 4096, 128, dc.DCONV1D_METHOD_WINOGRAD), (32, 256, 4096, 1, dc.DCONV1D_METHOD_WINOGRAD),
    (32, 256, 4096, 8, dc.DCONV1D_METHOD_WINOGRAD), (32, 256, 4096, 2048, dc.DCONV1D_METHOD_WINOGRAD),
    (32, 256, 4096, 96, dc.DCONV1D_METHOD_WINOGRAD), (32, 256, 4096, 100, dc.DCONV1D_METHOD_WINOGRAD),
    (32, 256, 4096, 48, dc.DCONV1D_METHOD_WINOGRAD), (32, 256, 4096, 20, dc.DCONV1D_METHOD_WINOGRAD),
    (32, 256, 4096, 3, dc.DCONV1D_METHOD_WINOGRAD), (32, 256, 4096, 5, dc.DCONV1D_METHOD_WINOGRAD),
    (32, 256, 4096, 2500, dc.DCONV1D_METHOD_WINOGRAD),  # pairs 2500: 7500 <= 8192
    (32, 256, 4096, 1500, dc.DCONV1D_METHOD_DIRECT),    # pairs 3000: 9000 > 8192
    (32, 256, 4096, 3000, dc.DCONV1D_METHOD_DIRECT),
    (512, 16, 7, 2, dc.DCONV1D_METHOD_WINOGRAD),        # pairs 4: 12 <= 14
    # the Winograd grid overruns one round of 512 workgroups by 32 (17 pair tiles x 32
    # samples) while the direct grid fills exactly one: the round factor (1.88) decides
    (32, 256, 1024, 97, dc.DCONV1D_METHOD_DIRECT),
    (512, 16, 5, 2, dc.DCONV1D_METHOD_DIRECT),          # pairs 4: 12 > 10
    # d >= L acts as d = L: every pair's second output lies past the end
    (512, 16, 256, 1000, dc.DCONV1D_METHOD_DIRECT), (512, 16, 1, 7, dc.DCONV1D_METHOD_DIRECT),
    (32, 256, 4096, 4096, dc.DCONV1D_METHOD_DIRECT),
    # small grids: both kernels halve their channel tiles, and the rule does not count
    # workgroups
    (1, 256, 4096, 128, dc.DCONV1D_METHOD_WINOGRAD), (2, 256, 4096, 128, dc.DCONV1D_METHOD_WINOGRAD),
    (3, 256, 4096, 128, dc.DCONV1D_METHOD_WINOGRAD), (2, 512, 4096, 128, dc.DCONV1D_METHOD_WINOGRAD),
    (1, 16, 62, 40, dc.DCONV1D_METHOD_WINOGRAD),        # pairs 40: 3 * 40 * 6881 <= 2 * 62 * 6736
    (1, 16, 62, 50, dc.DCONV1D_METHOD_DIRECT),          # pairs 50: over it
    (0, 256, 4096, 128, dc.DCONV1D_METHOD_DIRECT),
    # channel counts off multiples of 256: both kernels take 64- or 128-channel tiles, so
    # the grid condition counts those; the costs keep the Winograd form
    (32, 64, 4096, 128, dc.DCONV1D_METHOD_WINOGRAD), (32, 320, 4096, 128, dc.DCONV1D_METHOD_WINOGRAD),
    (3, 64, 4096, 128, dc.DCONV1D_METHOD_WINOGRAD), (2, 64, 4096, 128, dc.DCONV1D_METHOD_WINOGRAD),
    (2, 320, 4096, 128, dc.DCONV1D_METHOD_WINOGRAD),    # five 64-channel tiles: 640 workgroups
    # lengths from 2^28 on keep the direct kernel (32-bit offsets of two rows)
    (1, 1, (1 << 28) - 1, 64, dc.DCONV1D_METHOD_WINOGRAD), (1, 1, 1 << 28, 64, dc.DCONV1D_METHOD_DIRECT),
    (1, 1, (1 << 30) - 1, 64, dc.DCONV1D_METHOD_DIRECT),
])
def test_block_method(N, C, L, d, method, monkeypatch):
    monkeypatch.delenv("DCONV1D_WINOGRAD", raising=False)
    assert dc.dconv1d_block_method(N, C, L, d) == method


def test_block_method_switch_and_errors(monkeypatch):
    monkeypatch.setenv("DCONV1D_WINOGRAD", "0")
    assert dc.dconv1d_block_method(32, 256, 4096, 128) == dc.DCONV1D_METHOD_DIRECT
    monkeypatch.setenv("DCONV1D_WINOGRAD", "1")
    assert dc.dconv1d_block_method(1, 16, 62, 1) == dc.DCONV1D_METHOD_WINOGRAD
    assert dc.dconv1d_block_method(1, 16, 62, 1000) == dc.DCONV1D_METHOD_WINOGRAD
    assert dc.dconv1d_block_method(1, 16, 1 << 28, 1) == dc.DCONV1D_METHOD_DIRECT
    for v in ("", "2", "yes"):    # anything else: the automatic choice
        monkeypatch.setenv("DCONV1D_WINOGRAD", v)
        assert dc.dconv1d_block_method(1, 16, 62, 50) == dc.DCONV1D_METHOD_DIRECT
        assert dc.dconv1d_block_method(32, 256, 4096, 128) == dc.DCONV1D_METHOD_WINOGRAD
    lib = dc.load_library()
    assert lib.dconv1d_block_method(-1, 16, 16, 1) == dc.DCONV1D_EINVAL
    assert lib.dconv1d_block_method(1, 0, 16, 1) == dc.DCONV1D_EINVAL
    assert lib.dconv1d_block_method(1, 16385, 16, 1) == dc.DCONV1D_EINVAL
    assert lib.dconv1d_block_method(1, 16, 0, 1) == dc.DCONV1D_EINVAL
    assert lib.dconv1d_block_method(1, 16, 16, 0) == dc.DCONV1D_EINVAL


class _Addr:
    """Stands in for a tensor where only the address (its alignment) is read."""
    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


GN_W, GN_D = dc.DCONV1D_METHOD_WINOGRAD, dc.DCONV1D_METHOD_DIRECT


@pytest.mark.parametrize("N,C_in,C_out,T,G,pad,dil,x_addr,W_addr,method", [
    # the Winograd form: single-kernel path, per-wave windows (128 + 2*dil + s <= 136,
    # s = (4 - pad % 4) % 4 with 16-byte x loads, else 0), dil 1, 2 or 4, W 16-byte aligned
    (16, 128, 256, 1024, 32, 1, 1, None, None, GN_W),    # the GN workload's layer
    (2, 32, 64, 512, 8, 2, 2, None, None, GN_W),         # s = 2: 134 steps
    (2, 16, 32, 1008, 4, 4, 4, None, None, GN_W),        # s = 0: 136 steps
    (2, 16, 32, 1008, 4, 1, 4, None, None, GN_D),        # s = 3: 139 > 136, one shared window
    (2, 16, 32, 1008, 4, 1, 4, 4100, None, GN_W),        # 4-byte x loads: s = 0
    (2, 16, 32, 1004, 4, 3, 3, None, None, GN_D),        # dilation 3
    (16, 128, 256, 1024, 32, 1, 1, None, 4104, GN_D),    # W only 8-byte aligned
    # the two-kernel path: the Winograd conv when padding = dilation, else three taps
    (16, 128, 256, 1024, 32, 1, 1, None, 4100, GN_W),    # W 4-byte aligned: two kernels
    (4, 64, 128, 2048, 16, 1, 1, None, None, GN_W),      # T_out > 1024
    (2, 40, 96, 333, 12, 1, 1, None, None, GN_W),        # C_in not a multiple of 16
    (2, 128, 256, 1024, 8, 1, 1, None, None, GN_W),      # 32 channels per group
    (4, 32, 256, 2050, 16, 0, 1, None, None, GN_D),      # padding 0, dilation 1
    (2, 16, 48, 400, 4, 100, 100, None, None, GN_W),     # 12 channels per group
    (2, 16, 48, 300, 4, 400, 400, None, None, GN_D),     # dilation past T: pairs = T
    (2, 16, 48, 3000, 4, 3, 2, None, None, GN_D),        # padding != dilation
    (0, 128, 256, 1024, 32, 1, 1, None, None, GN_D),     # nothing to compute
])
def test_groupnorm_method(N, C_in, C_out, T, G, pad, dil, x_addr, W_addr, method, monkeypatch):
    monkeypatch.delenv("DCONV1D_WINOGRAD", raising=False)
    x = None if x_addr is None else _Addr(x_addr)
    W = None if W_addr is None else _Addr(W_addr)
    assert dc.dconv1d_groupnorm_method(N, C_in, C_out, T, G, pad, dil, x=x, W=W) == method


def test_groupnorm_method_switch_and_errors(monkeypatch):
    shape = (16, 128, 256, 1024, 32, 1, 1)
    monkeypatch.setenv("DCONV1D_WINOGRAD", "0")
    assert dc.dconv1d_groupnorm_method(*shape) == GN_D
    for v in ("1", "", "2"):      # "1" and anything else: the automatic choice
        monkeypatch.setenv("DCONV1D_WINOGRAD", v)
        assert dc.dconv1d_groupnorm_method(*shape) == GN_W
    lib = dc.load_library()
    ok = (32, 16, 128, 256, 1024, 1, 1)   # num_groups, N, C_in, C_out, T, padding, dilation
    assert lib.dconv1d_groupnorm_method(None, None, *ok) == GN_W
    for i, bad in [(1, -1), (2, 0), (2, 16385), (3, 0), (0, 0), (0, 3), (4, 0), (4, 1 << 29),
                   (5, -1), (5, 1 << 29), (6, 0), (6, 513)]:
        args = list(ok)
        args[i] = bad
        assert lib.dconv1d_groupnorm_method(None, None, *args) == dc.DCONV1D_EINVAL, (i, bad)
    with pytest.raises(Exception):
        dc.dconv1d_groupnorm_method(-1, 128, 256, 1024, 32, 1, 1)
