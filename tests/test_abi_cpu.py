"""The C-ABI library on a host without a GPU: it loads, exports every declared symbol and
rejects invalid arguments before any HIP call. No compute call is made here."""
import ctypes
import math
import os

import pytest

from pairwise_reductions_amd import _lib

F32, F16 = _lib.KEOPS_F32, _lib.KEOPS_F16
INVALID, UNSUPPORTED = _lib.KEOPS_ERR_INVALID_ARG, _lib.KEOPS_ERR_UNSUPPORTED

# Fake, never-dereferenced device addresses far apart from each other (validation only).
X, Y, B, G, OUT, WS, IDX, DIST = (0x10000000 * k for k in range(1, 9))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from pairwise_reductions_amd import build
        build.build()
    return _lib.load()


def _err(lib):
    return lib.keops_last_error().decode()


def test_exports_every_declared_symbol(lib):
    names = _lib.header_symbols()
    assert set(names) == {"keops_gauss_sum", "keops_lse", "keops_argkmin", "keops_gauss_sum_grad_x",
                          "keops_gauss_sum_grad_y", "keops_gauss_sum_grad_b", "keops_argkmin_lse",
                          "keops_gauss_sum_scaled", "keops_gauss_sum_backward", "keops_diffusion_scaling",
                          "keops_argkmin_weighted", "keops_gauss_sum_noalloc",
                          "keops_workspace_bytes", "keops_status_string", "keops_last_error", "keops_version",
                          "keops_sweep_timing", "keops_sweep_timing_read"}
    for name in names:
        assert hasattr(lib, name), name
    # the same names, resolved by the dynamic loader straight from the file
    raw = ctypes.CDLL(_lib.LIB_PATH)
    for name in names:
        getattr(raw, name)


def test_status_strings_and_version(lib):
    assert lib.keops_status_string(0) == b"ok"
    assert lib.keops_status_string(1) == b"invalid argument"
    assert lib.keops_status_string(2) == b"unsupported configuration"
    assert lib.keops_status_string(3) == b"HIP runtime error"
    assert lib.keops_status_string(99) == b"unknown status"
    assert b"gfx950" in lib.keops_version()


def test_sweep_timing_host_logic(lib):
    """The measurement aid's bookkeeping (no event is created without a sweep launch)."""
    ms, n = ctypes.c_float(-1.0), ctypes.c_int(-1)
    assert lib.keops_sweep_timing(1) == 0
    assert lib.keops_sweep_timing_read(ctypes.byref(ms), ctypes.byref(n)) == 0
    assert ms.value == 0.0 and n.value == 0
    assert lib.keops_sweep_timing_read(None, ctypes.byref(n)) == 1
    assert "must not be NULL" in _err(lib)
    assert lib.keops_sweep_timing(0) == 0


def test_workspace_bytes(lib):
    ws = lib.keops_workspace_bytes
    n_cols = ws(0, 1, 1_000_000, 1_000_000, 3, 1, 0, F32)
    assert n_cols >= 1_000_000 * 4 * 8           # float64 column table (4 doubles a column)
    assert ws(0, 1, 0, 1000, 3, 1, 0, F32) == 0   # M = 0 needs nothing
    assert ws(0, 1, 10, 0, 3, 1, 0, F32) == 0     # N = 0 needs nothing
    assert ws(0, 1, 10, 10, 129, 1, 0, F32) == 0  # D out of range
    assert ws(0, 1, 10, 10, 3, 0, 0, F32) == 0    # C out of range
    assert ws(0, 2, 10, 10, 3, 1, 0, F32) == 0    # batched float32 unsupported
    assert ws(2, 1, 10, 10, 3, 1, 11, F32) == 0   # K > N
    assert ws(2, 1, 10, 100, 3, 1, 65, F32) == 0  # K > 64
    assert ws(1, 1, -1, 10, 3, 1, 0, F32) == 0    # negative M
    # small M: the columns are split across workgroups, which needs partial buffers
    assert ws(0, 1, 100, 100_000, 3, 1, 0, F32) > 100_000 * 32
    assert ws(3, 1, 100, 100_000, 3, 1, 0, F32) > 0
    # fp16 matrix-core path: key norms (float) and the permuted fp16 copy of v
    assert ws(0, 4, 16384, 16384, 32, 32, 0, F16) >= 4 * 16384 * (4 + 32 * 2)
    assert ws(0, 4, 16384, 16384, 48, 32, 0, F16) > 0     # D padded to 64 inside
    # D not a multiple of 16: the padded copies of the points come first
    assert ws(0, 4, 16384, 16384, 40, 32, 0, F16) >= ws(0, 4, 16384, 16384, 48, 32, 0, F16) + 4 * 2 * 16384 * 48 * 2
    assert ws(0, 4, 16384, 16384, 144, 32, 0, F16) == 0   # D > 128
    assert ws(0, 4, 16384, 16384, 32, 32, 0, 2) > 0       # bf16
    assert ws(0, 4, 16384, 16384, 32, 32, 0, F32) >= 4 * 16384 * (4 + 2 * 32 * 2)   # hi + lo weight tables


def _gs(lib, x=X, y=Y, b=B, out=OUT, Bt=1, M=100, N=100, D=3, C=1, sigma=0.1, dtype=F32, ws=WS, wsb=1 << 30):
    return lib.keops_gauss_sum(x, y, b, out, Bt, M, N, D, C, sigma, dtype, ws, wsb, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(x=None), INVALID), (dict(y=None), INVALID), (dict(b=None), INVALID), (dict(out=None), INVALID),
    (dict(M=-1), INVALID), (dict(N=-5), INVALID), (dict(Bt=-1), INVALID),
    (dict(sigma=0.0), INVALID), (dict(sigma=-1.0), INVALID), (dict(sigma=math.nan), INVALID),
    (dict(sigma=math.inf), INVALID),
    (dict(D=129), UNSUPPORTED), (dict(D=0), UNSUPPORTED), (dict(C=0), UNSUPPORTED), (dict(C=9), UNSUPPORTED),
    (dict(Bt=2), UNSUPPORTED), (dict(dtype=F16, D=0), UNSUPPORTED), (dict(dtype=7), INVALID),
    (dict(dtype=2, D=130, C=32), UNSUPPORTED), (dict(dtype=F16, D=40, C=0), UNSUPPORTED),
    (dict(dtype=F32, D=24, C=65), UNSUPPORTED), (dict(dtype=2, D=32, C=65), UNSUPPORTED),
    (dict(dtype=F32, D=32, C=4, Bt=2, x=X + 4), INVALID),     # matrix-core path: 16-byte alignment
    (dict(dtype=F16, D=144, C=32), UNSUPPORTED),
    (dict(dtype=F16, D=32, C=65), UNSUPPORTED),
    (dict(dtype=F16, D=32, C=32, x=X + 8), INVALID),
    (dict(x=X + 2), INVALID), (dict(out=X + 4), INVALID), (dict(M=1 << 31), UNSUPPORTED),
    (dict(ws=None, wsb=0), INVALID), (dict(wsb=16), INVALID), (dict(ws=WS + 8), INVALID),
])
def test_gauss_sum_rejects(lib, kwargs, code):
    assert _gs(lib, **kwargs) == code
    assert _err(lib) != ""


def test_empty_rows_is_a_noop(lib):
    assert _gs(lib, M=0) == 0
    assert _err(lib) == ""
    assert lib.keops_lse(X, Y, OUT, 0, 10, 3, 0.1, None, 0, None) == 0
    assert lib.keops_argkmin(X, Y, IDX, None, 0, 10, 3, 4, None, 0, None) == 0
    assert lib.keops_gauss_sum_grad_x(X, Y, B, G, OUT, 0, 10, 3, 1, 0.1, None, 0, None) == 0


def test_lse_rejects(lib):
    f = lib.keops_lse
    assert f(None, Y, OUT, 10, 10, 3, 0.1, WS, 1 << 30, None) == INVALID
    assert f(X, Y, None, 10, 10, 3, 0.1, WS, 1 << 30, None) == INVALID
    assert f(X, Y, OUT, 10, 10, 0, 0.1, WS, 1 << 30, None) == UNSUPPORTED
    assert f(X, Y, OUT, 10, 10, 3, -0.1, WS, 1 << 30, None) == INVALID
    assert f(X, Y, X, 10, 10, 3, 0.1, WS, 1 << 30, None) == INVALID   # out aliases x
    assert f(X, Y, OUT, 10, 10, 3, 0.1, None, 0, None) == INVALID     # workspace needed


def test_argkmin_rejects(lib):
    f = lib.keops_argkmin
    assert f(X, Y, IDX, None, 10, 10, 3, 0, WS, 1 << 30, None) == INVALID
    assert f(X, Y, IDX, None, 10, 10, 3, 11, WS, 1 << 30, None) == INVALID
    assert f(X, Y, IDX, None, 10, 100, 3, 65, WS, 1 << 30, None) == UNSUPPORTED
    assert f(X, Y, IDX, None, 10, 0, 3, 1, WS, 1 << 30, None) == INVALID  # N = 0: K > N
    assert f(X, Y, None, None, 10, 10, 3, 4, WS, 1 << 30, None) == INVALID
    assert f(X, Y, IDX, DIST + 2, 10, 10, 3, 4, WS, 1 << 30, None) == INVALID
    assert f(X, Y, IDX, IDX + 8, 10, 10, 3, 4, WS, 1 << 30, None) == INVALID  # idx and dist overlap
    assert f(X, Y, IDX, None, 10, 10, 9, 4, WS, 1 << 30, None) == UNSUPPORTED


def test_grad_rejects(lib):
    f = lib.keops_gauss_sum_grad_x
    assert f(X, Y, B, None, OUT, 10, 10, 3, 1, 0.1, WS, 1 << 30, None) == INVALID
    assert f(X, Y, B, G, OUT, 10, 10, 3, 0, 0.1, WS, 1 << 30, None) == UNSUPPORTED
    assert f(X, Y, B, G, G, 10, 10, 3, 1, 0.1, WS, 1 << 30, None) == INVALID  # grad aliases g
    assert f(X, Y, B, G, OUT, 10, 10, 3, 1, 0.0, WS, 1 << 30, None) == INVALID


def test_error_is_thread_local(lib):
    import threading
    assert _gs(lib, D=129) == UNSUPPORTED
    seen = []

    def worker():
        seen.append(_err(lib))

    t = threading.Thread(target=worker)
    t.start()
    t.join()
    assert seen == [""]
    assert "D=129" in _err(lib)


def test_grad_yb_reject(lib):
    fy, fb = lib.keops_gauss_sum_grad_y, lib.keops_gauss_sum_grad_b
    assert fy(X, Y, B, None, OUT, 10, 10, 3, 1, 0.1, WS, 1 << 30, None) == INVALID
    assert fy(X, Y, B, G, OUT, 10, 10, 9, 1, 0.1, WS, 1 << 30, None) == UNSUPPORTED
    assert fy(X, Y, B, G, Y, 10, 10, 3, 1, 0.1, WS, 1 << 30, None) == INVALID   # grad_y aliases y
    assert fy(X, Y, B, G, OUT, 10, 0, 3, 1, 0.1, None, 0, None) == 0             # N = 0: no-op
    assert fb(X, Y, None, OUT, 10, 10, 3, 1, 0.1, WS, 1 << 30, None) == INVALID
    assert fb(X, Y, G, OUT, 10, 10, 3, 1, -1.0, WS, 1 << 30, None) == INVALID
    assert fb(X, Y, G, OUT, 10, 10, 3, 0, 0.1, WS, 1 << 30, None) == UNSUPPORTED
    assert fb(X, Y, G, OUT, 10, 0, 3, 1, 0.1, None, 0, None) == 0
    ws = lib.keops_workspace_bytes
    assert ws(4, 1, 100_000, 100, 3, 1, 0, F32) > 0 and ws(5, 1, 100_000, 100, 3, 2, 0, F32) > 0


def test_argkmin_lse_rejects(lib):
    f = lib.keops_argkmin_lse
    assert f(X, Y, IDX, None, None, 10, 10, 3, 4, 0.1, WS, 1 << 30, None) == INVALID   # lse NULL
    assert f(X, Y, IDX, None, OUT, 10, 10, 3, 4, 0.0, WS, 1 << 30, None) == INVALID   # sigma
    assert f(X, Y, IDX, None, IDX, 10, 10, 3, 4, 0.1, WS, 1 << 30, None) == INVALID   # lse aliases idx
    assert f(X, Y, IDX, None, OUT, 10, 10, 3, 11, 0.1, WS, 1 << 30, None) == INVALID  # K > N
    assert f(X, Y, IDX, None, OUT, 0, 10, 3, 4, 0.1, None, 0, None) == 0              # M = 0
    assert lib.keops_workspace_bytes(6, 1, 100, 100_000, 3, 1, 10, F32) > lib.keops_workspace_bytes(2, 1, 100, 100_000, 3, 1, 10, F32)


R, CS, GX, GY, GB, S, Q, DD = (0x10000000 * k for k in range(9, 17))


def test_gauss_sum_scaled_rejects(lib):
    f = lib.keops_gauss_sum_scaled
    args = lambda **kw: dict(dict(x=X, y=Y, b=B, r=R, c=CS, out=OUT, Bt=1, M=100, N=100, D=3, C=1, sigma=0.1,
                                  dtype=F32, ws=WS, wsb=1 << 30), **kw)
    call = lambda a: f(a["x"], a["y"], a["b"], a["r"], a["c"], a["out"], a["Bt"], a["M"], a["N"], a["D"], a["C"],
                       a["sigma"], a["dtype"], a["ws"], a["wsb"], None)
    assert call(args(r=R + 2)) == INVALID            # misaligned row scale
    assert call(args(c=CS + 1)) == INVALID
    assert call(args(out=R)) == INVALID              # out aliases the row scale
    assert call(args(D=129)) == UNSUPPORTED
    assert call(args(dtype=F16, D=32, C=32, Bt=2, x=X + 8)) == INVALID   # fp16 inputs need 16-byte alignment
    assert call(args(dtype=F16, D=136, C=32, Bt=2)) == UNSUPPORTED
    assert call(args(M=0)) == 0                      # no rows: no-op
    ws = lib.keops_workspace_bytes
    assert ws(7, 1, 1000, 1000, 3, 2, 0, F32) > ws(0, 1, 1000, 1000, 3, 2, 0, F32)   # scaled weights copy
    assert ws(7, 2, 1000, 1000, 32, 8, 0, F16) >= ws(0, 2, 1000, 1000, 32, 8, 0, F16)


def test_gauss_sum_backward_rejects(lib):
    f = lib.keops_gauss_sum_backward
    call = lambda **kw: f(*[dict(dict(x=X, y=Y, b=B, g=G, gx=GX, gy=GY, gb=GB, Bt=1, M=100, N=100, D=3, C=1,
                                      sigma=0.1, dtype=F32, ws=WS, wsb=1 << 30), **kw)[k]
                            for k in ("x", "y", "b", "g", "gx", "gy", "gb", "Bt", "M", "N", "D", "C", "sigma",
                                      "dtype", "ws", "wsb")], None)
    assert call(g=None) == INVALID
    assert call(gx=X) == INVALID                       # a gradient aliases an input
    assert call(gx=GX, gy=GX) == INVALID               # gradients overlap each other
    assert call(D=9) == UNSUPPORTED and call(Bt=2) == UNSUPPORTED
    assert call(dtype=F16, D=136, C=4) == UNSUPPORTED
    assert call(dtype=2, D=32, C=4) == UNSUPPORTED                # bf16 backward is not built
    assert call(dtype=F32, D=32, C=4) == UNSUPPORTED              # nor the float32 matrix-core one
    assert call(dtype=F16, D=32, C=4, gx=GX + 4) == INVALID   # fp16 path needs 16-byte aligned outputs
    assert call(sigma=-1.0) == INVALID
    assert call(gx=None, gy=None, gb=None, ws=None, wsb=0) == 0   # nothing requested
    assert call(ws=None, wsb=0) == INVALID             # workspace needed
    ws = lib.keops_workspace_bytes
    assert ws(8, 1, 1000, 200, 3, 1, 0, F32) > 0
    assert ws(8, 4, 16384, 16384, 32, 1, 0, F16) > ws(0, 4, 16384, 16384, 32, 1, 0, F16)
    assert ws(8, 4, 16384, 16384, 40, 1, 0, F16) > ws(8, 4, 16384, 16384, 48, 1, 0, F16)   # padded copies
    assert ws(8, 4, 16384, 16384, 129, 1, 0, F16) == 0


def test_diffusion_scaling_rejects(lib):
    f = lib.keops_diffusion_scaling
    call = lambda **kw: f(*[dict(dict(x=X, s=S, q=Q, d=DD, Bt=1, N=100, D=3, sigma=0.1, alpha=0.5, dtype=F32,
                                      ws=WS, wsb=1 << 30), **kw)[k]
                            for k in ("x", "s", "q", "d", "Bt", "N", "D", "sigma", "alpha", "dtype", "ws", "wsb")],
                          None)
    assert call(s=None) == INVALID
    assert call(alpha=math.nan) == INVALID
    assert call(q=S) == INVALID                         # q aliases s
    assert call(D=129) == UNSUPPORTED and call(Bt=3) == UNSUPPORTED
    assert call(dtype=F16, D=0) == UNSUPPORTED
    assert call(N=0, ws=None, wsb=0) == 0
    assert call(ws=None, wsb=0) == INVALID
    ws = lib.keops_workspace_bytes
    assert ws(9, 1, 0, 5000, 3, 1, 0, F32) >= 4 * 5000 * 4
    assert ws(9, 2, 0, 5000, 32, 1, 0, F16) > 0 and ws(9, 2, 0, 5000, 3, 1, 0, F16) > 0
    assert ws(9, 2, 0, 5000, 129, 1, 0, F16) == 0


def test_argkmin_weighted_rejects(lib):
    f = lib.keops_argkmin_weighted
    W = 0x10000000 * 17
    assert f(X, Y, None, IDX, None, 10, 10, 3, 4, WS, 1 << 30, None) == INVALID      # w NULL
    assert f(X, Y, W + 2, IDX, None, 10, 10, 3, 4, WS, 1 << 30, None) == INVALID     # misaligned w
    assert f(X, Y, IDX, IDX, None, 10, 10, 3, 4, WS, 1 << 30, None) == INVALID      # idx aliases w
    assert f(X, Y, W, IDX, None, 10, 10, 3, 11, WS, 1 << 30, None) == INVALID       # K > N
    assert f(X, Y, W, IDX, None, 10, 10, 9, 4, WS, 1 << 30, None) == UNSUPPORTED
    assert f(X, Y, W, IDX, None, 0, 10, 3, 4, None, 0, None) == 0                    # M = 0
    ws = lib.keops_workspace_bytes
    assert ws(10, 1, 100, 100_000, 3, 1, 10, F32) == ws(2, 1, 100, 100_000, 3, 1, 10, F32) > 0


# --------------------------------------------------------------- the header's support rules
# Each row restates one rule of include/keops_mi355x.h for keops_gauss_sum (and the calls that
# share its families). An accepted configuration passes every shape check and then stops at the
# workspace check (a 16-byte workspace is too small for any non-empty call), so nothing is
# launched; a refused one returns KEOPS_ERR_UNSUPPORTED first.
BF16 = 2
SUPPORT_RULES = [
    # (dtype, B, D, C, accepted)
    (F32, 1, 1, 1, True), (F32, 1, 3, 1, True), (F32, 1, 8, 8, True),       # low-D float32
    (F32, 2, 3, 1, False),                                                   # low-D needs B = 1
    (F32, 1, 3, 9, False),                                                   # low-D needs C <= 8
    (F32, 1, 9, 1, True), (F32, 4, 12, 3, True), (F32, 4, 32, 32, True),     # float32 matrix cores
    (F32, 2, 100, 64, True), (F32, 1, 128, 1, True),
    (F32, 1, 129, 1, False), (F32, 4, 32, 65, False),
    (F16, 4, 32, 32, True), (F16, 1, 1, 1, True), (F16, 2, 20, 5, True),    # any D <= 128
    (F16, 3, 50, 64, True), (F16, 1, 100, 17, True), (F16, 1, 128, 64, True),
    (F16, 1, 129, 1, False), (F16, 1, 32, 65, False), (F16, 1, 32, 0, False), (F16, 1, 0, 1, False),
    (BF16, 4, 32, 32, True), (BF16, 1, 9, 2, True), (BF16, 1, 136, 2, False),
]


@pytest.mark.parametrize("dtype,Bt,D,C,accepted", SUPPORT_RULES)
def test_header_support_rules(lib, dtype, Bt, D, C, accepted):
    code = _gs(lib, dtype=dtype, Bt=Bt, D=D, C=C, wsb=16)
    if accepted:
        assert code == INVALID and "workspace too small" in _err(lib), (code, _err(lib))
        assert lib.keops_workspace_bytes(0, Bt, 100, 100, D, C, 0, dtype) > 16
        # the scaled form shares the families
        sc = lib.keops_gauss_sum_scaled(X, Y, B, None, None, OUT, Bt, 100, 100, D, C, 0.1, dtype, WS, 16, None)
        assert sc == INVALID and "workspace too small" in _err(lib)
    else:
        assert code == UNSUPPORTED, (code, _err(lib))
        assert lib.keops_workspace_bytes(0, Bt, 100, 100, D, C, 0, dtype) == 0


@pytest.mark.parametrize("dtype,D,accepted", [(F32, 3, True), (F32, 9, False), (F16, 20, True), (F16, 32, True),
                                              (F16, 128, True), (F16, 129, False), (BF16, 32, False)])
def test_header_support_rules_backward(lib, dtype, D, accepted):
    Bt = 1 if dtype == F32 else 2
    code = lib.keops_gauss_sum_backward(X, Y, B, G, GX, GY, GB, Bt, 100, 100, D, 1, 0.1, dtype, WS, 16, None)
    if accepted:
        assert code == INVALID and "workspace too small" in _err(lib), (code, _err(lib))
    else:
        assert code == UNSUPPORTED, (code, _err(lib))


@pytest.mark.parametrize("D,accepted", [(1, True), (8, True), (9, False)])
def test_header_support_rules_lowd_calls(lib, D, accepted):
    """keops_lse, keops_argkmin and keops_gauss_sum_grad_x take float32 with 1 <= D <= 8."""
    codes = [lib.keops_lse(X, Y, OUT, 100, 100, D, 0.1, WS, 16, None),
             lib.keops_argkmin(X, Y, IDX, None, 100, 100, D, 4, WS, 16, None),
             lib.keops_gauss_sum_grad_x(X, Y, B, G, OUT, 100, 100, D, 1, 0.1, WS, 16, None)]
    for code in codes:
        assert code == (INVALID if accepted else UNSUPPORTED)


def test_noalloc_rejects_before_any_hip_call(lib):
    """The allocation-free entry point validates like keops_gauss_sum and refuses sizes whose
    workspace exceeds its scratch, all before touching the device."""
    f = lib.keops_gauss_sum_noalloc
    assert f(None, Y, B, OUT, 1, 100, 100, 3, 1, 0.1, F32, None) == INVALID
    assert f(X, Y, B, OUT, 1, 100, 100, 129, 1, 0.1, F32, None) == UNSUPPORTED
    assert f(X, Y, B, OUT, 1, 100, 100, 3, 1, -1.0, F32, None) == INVALID
    assert f(X, Y, B, X, 1, 100, 100, 3, 1, 0.1, F32, None) == INVALID          # out aliases x
    assert f(X, Y, B, OUT, 1, 0, 100, 3, 1, 0.1, F32, None) == 0                 # M = 0: no-op
    assert f(X, Y, B, OUT, 1, 1_000_000, 1_000_000, 3, 1, 0.01, F32, None) == UNSUPPORTED
    assert "scratch" in _err(lib)
    assert lib.keops_workspace_bytes(0, 1, 1_000_000, 1_000_000, 3, 1, 0, F32) > 64 << 20
