"""ctypes loader for libkeops_mi355x.so and the raw C-ABI signatures.

The library is built in-tree by pairwise_reductions_amd/build.py. Importing this module
never builds anything: a missing library raises at first use, so nothing silently falls
back to another implementation.
"""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkeops_mi355x.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "keops_mi355x.h")

KEOPS_F32, KEOPS_F16, KEOPS_BF16 = 0, 1, 2
KEOPS_OK, KEOPS_ERR_INVALID_ARG, KEOPS_ERR_UNSUPPORTED, KEOPS_ERR_HIP = 0, 1, 2, 3
OP_GAUSS_SUM, OP_LSE, OP_ARGKMIN, OP_GAUSS_SUM_GRAD_X, OP_GAUSS_SUM_GRAD_Y, OP_GAUSS_SUM_GRAD_B = 0, 1, 2, 3, 4, 5
OP_ARGKMIN_LSE, OP_GAUSS_SUM_SCALED, OP_GAUSS_SUM_BACKWARD, OP_DIFFUSION_SCALING = 6, 7, 8, 9
OP_ARGKMIN_WEIGHTED = 10

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_f32 = ctypes.c_float
_sz = ctypes.c_size_t

_SIGNATURES = {
    "keops_gauss_sum": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _f32, ctypes.c_int,
                                       _vp, _sz, _vp]),
    "keops_gauss_sum_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _f32, ctypes.c_int,
                                               _vp]),
    "keops_lse": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i32, _f32, _vp, _sz, _vp]),
    "keops_argkmin": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _vp, _sz, _vp]),
    "keops_argkmin_weighted": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _vp, _sz, _vp]),
    "keops_argkmin_lse": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _f32, _vp, _sz, _vp]),
    "keops_gauss_sum_grad_x": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _f32, _vp, _sz,
                                              _vp]),
    "keops_gauss_sum_grad_y": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _f32, _vp, _sz,
                                              _vp]),
    "keops_gauss_sum_grad_b": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _i32, _f32, _vp, _sz, _vp]),
    "keops_gauss_sum_scaled": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _f32,
                                              ctypes.c_int, _vp, _sz, _vp]),
    "keops_gauss_sum_backward": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32,
                                                _f32, ctypes.c_int, _vp, _sz, _vp]),
    "keops_diffusion_scaling": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i32, _f32, _f32, ctypes.c_int, _vp,
                                               _sz, _vp]),
    "keops_workspace_bytes": (_sz, [ctypes.c_int, _i64, _i64, _i64, _i32, _i32, _i32, ctypes.c_int]),
    "keops_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "keops_last_error": (ctypes.c_char_p, []),
    "keops_version": (ctypes.c_char_p, []),
    "keops_sweep_timing": (ctypes.c_int, [ctypes.c_int]),
    "keops_sweep_timing_read": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_int)]),
}

_lib = None


class KeopsError(RuntimeError):
    """A C-ABI call returned a non-zero status."""

    def __init__(self, status: int, fn: str, detail: str):
        self.status = status
        super().__init__(f"{fn} failed with status {status} ({status_name(status)}): {detail}")


def status_name(status: int) -> str:
    return {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "HIP error"}.get(status, "unknown")


def load(path: str = LIB_PATH):
    """Load the shared library (once) and attach the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def header_symbols(path: str = HEADER_PATH):
    """Names of the functions the public header declares."""
    with open(path) as f:
        text = f.read()
    return re.findall(r"KEOPS_API\s+[\w\s\*]+?\b(keops_\w+)\s*\(", text)


def check(status: int, fn: str):
    if status != KEOPS_OK:
        detail = load().keops_last_error().decode()
        raise KeopsError(status, fn, detail)
