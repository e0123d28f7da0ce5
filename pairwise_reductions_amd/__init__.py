"""Fused pairwise kernel reductions on AMD MI355X (gfx950).

Thin Python binding over the C ABI declared in include/keops_mi355x.h. PyTorch supplies
device memory and the current HIP stream; every arithmetic step runs in the library's HIP
kernels. Each function takes CUDA (HIP) tensors, allocates its output and workspace from
PyTorch's allocator (or uses the ones passed in) and enqueues the work on the current stream.
"""
from __future__ import annotations

from typing import Optional, Tuple

from . import _lib
from ._lib import KeopsError  # noqa: F401

__all__ = ["gauss_sum", "gauss_sum_noalloc", "gauss_sum_scaled", "lse", "argkmin", "argkmin_weighted", "argkmin_lse", "gauss_sum_grad_x", "gauss_sum_grad_y",
           "gauss_sum_grad_b", "gauss_sum_backward", "diffusion_scaling", "gauss_sum_autograd", "workspace_bytes",
           "KeopsError", "version"]


def _torch():
    import torch
    return torch


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _dims(t, rank):
    if t.dim() != rank:
        raise ValueError(f"expected a {rank}-D tensor, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.shape


def _workspace(nbytes: int, device, workspace=None):
    torch = _torch()
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, "
                             f"{nbytes} needed")
        return workspace, workspace.numel() * workspace.element_size()
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, nbytes


def version() -> str:
    return _lib.load().keops_version().decode()


def workspace_bytes(op: int, B: int, M: int, N: int, D: int, C: int = 1, K: int = 0, dtype: int = 0) -> int:
    return int(_lib.load().keops_workspace_bytes(op, B, M, N, D, C, K, dtype))


def _gauss_shapes(x, y, b):
    """(B, M, N, D, C, dtype code, batched) of a Gauss-sum call: float32 (M, D) points, or
    batched (B, M, D) points in float16, bfloat16 or float32."""
    torch = _torch()
    if x.dtype == torch.float32 and x.dim() == 2:
        M, D = _dims(x, 2)
        N, _ = _dims(y, 2)
        _, C = _dims(b, 2)
        return 1, M, N, D, C, _lib.KEOPS_F32, False
    dt = {torch.float16: _lib.KEOPS_F16, torch.bfloat16: _lib.KEOPS_BF16, torch.float32: _lib.KEOPS_F32}.get(x.dtype)
    if dt is None:
        raise ValueError(f"unsupported dtype {x.dtype}")
    if y.dtype != x.dtype or b.dtype != x.dtype:
        raise ValueError("x, y and b must share one dtype")
    B, M, D = _dims(x, 3)
    _, N, _ = _dims(y, 3)
    _, _, C = _dims(b, 3)
    return B, M, N, D, C, dt, True


def gauss_sum(x, y, b, sigma: float, out=None, workspace=None):
    """s[i, c] = sum_j exp(-|x_i - y_j|^2 / (2 sigma^2)) b[j, c].

    float32: x (M, D), y (N, D), b (N, C) -> (M, C) (D <= 8 runs the float32 VALU kernels,
    9 <= D <= 128 the matrix-core kernels).
    batched: x (B, M, D), y (B, N, D), b (B, N, C) in float16, bfloat16 or float32 with
    1 <= D <= 128 and 1 <= C <= 64 (the matrix-core kernels) -> (B, M, C) float32.
    """
    torch = _torch()
    lib = _lib.load()
    B, M, N, D, C, dt, batched = _gauss_shapes(x, y, b)
    if out is None:
        out = torch.empty((B, M, C) if batched else (M, C), dtype=torch.float32, device=x.device)
    nbytes = lib.keops_workspace_bytes(_lib.OP_GAUSS_SUM, B, M, N, D, C, 0, dt)
    ws, have = _workspace(nbytes, x.device, workspace)
    st = lib.keops_gauss_sum(_ptr(x), _ptr(y), _ptr(b), _ptr(out), B, M, N, D, C, float(sigma), dt,
                             _ptr(ws), have, _stream(x.device))
    _lib.check(st, "keops_gauss_sum")
    return out


def gauss_sum_noalloc(x, y, b, sigma: float, out):
    """gauss_sum through the allocation-free entry point: the library's fixed scratch array
    replaces the workspace, so nothing is allocated (the caller passes the output). Same
    shapes, limits and results as gauss_sum; sizes whose workspace exceeds the scratch raise
    KeopsError (unsupported)."""
    lib = _lib.load()
    B, M, N, D, C, dt, _ = _gauss_shapes(x, y, b)
    st = lib.keops_gauss_sum_noalloc(_ptr(x), _ptr(y), _ptr(b), _ptr(out), B, M, N, D, C, float(sigma), dt,
                                     _stream(x.device))
    _lib.check(st, "keops_gauss_sum_noalloc")
    return out


def gauss_sum_scaled(x, y, b, sigma: float, row_scale=None, col_scale=None, out=None, workspace=None):
    """out[i, c] = row_scale[i] sum_j k_ij col_scale[j] b[j, c] (either scale may be None).

    Shapes as gauss_sum; row_scale is (M,) or (B, M), col_scale (N,) or (B, N), float32.
    """
    torch = _torch()
    lib = _lib.load()
    B, M, N, D, C, dt, batched = _gauss_shapes(x, y, b)
    for t, n in ((row_scale, M), (col_scale, N)):
        if t is not None and (t.dtype != torch.float32 or t.numel() != B * n or not t.is_contiguous()):
            raise ValueError("scales must be contiguous float32 with one entry per row / column")
    if out is None:
        out = torch.empty((B, M, C) if batched else (M, C), dtype=torch.float32, device=x.device)
    nbytes = lib.keops_workspace_bytes(_lib.OP_GAUSS_SUM_SCALED, B, M, N, D, C, 0, dt)
    ws, have = _workspace(nbytes, x.device, workspace)
    st = lib.keops_gauss_sum_scaled(_ptr(x), _ptr(y), _ptr(b), _ptr(row_scale), _ptr(col_scale), _ptr(out), B, M, N,
                                    D, C, float(sigma), dt, _ptr(ws), have, _stream(x.device))
    _lib.check(st, "keops_gauss_sum_scaled")
    return out


def gauss_sum_backward(x, y, b, g, sigma: float, need=("x", "y", "b"), workspace=None):
    """Gradients of out = gauss_sum(x, y, b) for the upstream gradient g = dL/d out (float32).

    Returns a dict with the requested keys among "x", "y", "b" (float32 tensors shaped like
    x, y and b). Works for both the float32 and the fp16 (batched) path.
    """
    torch = _torch()
    lib = _lib.load()
    B, M, N, D, C, dt, batched = _gauss_shapes(x, y, b)
    if g.dtype != torch.float32 or tuple(g.shape) != ((B, M, C) if batched else (M, C)) or not g.is_contiguous():
        raise ValueError("g must be contiguous float32 shaped like the forward output")
    res = {}
    for key, t in (("x", x), ("y", y), ("b", b)):
        if key in need:
            res[key] = torch.empty(t.shape, dtype=torch.float32, device=x.device)
    nbytes = lib.keops_workspace_bytes(_lib.OP_GAUSS_SUM_BACKWARD, B, M, N, D, C, 0, dt)
    ws, have = _workspace(nbytes, x.device, workspace)
    st = lib.keops_gauss_sum_backward(_ptr(x), _ptr(y), _ptr(b), _ptr(g), _ptr(res.get("x")), _ptr(res.get("y")),
                                      _ptr(res.get("b")), B, M, N, D, C, float(sigma), dt, _ptr(ws), have,
                                      _stream(x.device))
    _lib.check(st, "keops_gauss_sum_backward")
    return res


def diffusion_scaling(x, sigma: float, alpha: float, workspace=None):
    """(s, q, d) of the alpha-normalised diffusion operator diag(s) K diag(s), K_ij = k(x_i, x_j):
    q = K 1, p = q^-alpha, d = p (K p), s = p / sqrt(d). x is float32 (N, D) or batched
    (B, N, D) in float16, bfloat16 or float32 (D a multiple of 16)."""
    torch = _torch()
    lib = _lib.load()
    if x.dtype == torch.float32 and x.dim() == 2:
        N, D = _dims(x, 2)
        B, dt, shape = 1, _lib.KEOPS_F32, (N,)
    elif x.dtype in (torch.float16, torch.bfloat16, torch.float32):
        B, N, D = _dims(x, 3)
        dt = {torch.float16: _lib.KEOPS_F16, torch.bfloat16: _lib.KEOPS_BF16, torch.float32: _lib.KEOPS_F32}[x.dtype]
        shape = (B, N)
    else:
        raise ValueError(f"unsupported dtype {x.dtype}")
    s, q, d = (torch.empty(shape, dtype=torch.float32, device=x.device) for _ in range(3))
    nbytes = lib.keops_workspace_bytes(_lib.OP_DIFFUSION_SCALING, B, N, N, D, 1, 0, dt)
    ws, have = _workspace(nbytes, x.device, workspace)
    st = lib.keops_diffusion_scaling(_ptr(x), _ptr(s), _ptr(q), _ptr(d), B, N, D, float(sigma), float(alpha), dt,
                                     _ptr(ws), have, _stream(x.device))
    _lib.check(st, "keops_diffusion_scaling")
    return s, q, d


def lse(x, y, sigma: float, out=None, workspace=None):
    """out[i] = log sum_j exp(-|x_i - y_j|^2 / (2 sigma^2)); x (M, D), y (N, D) float32."""
    torch = _torch()
    lib = _lib.load()
    M, D = _dims(x, 2)
    N, _ = _dims(y, 2)
    if out is None:
        out = torch.empty((M,), dtype=torch.float32, device=x.device)
    nbytes = lib.keops_workspace_bytes(_lib.OP_LSE, 1, M, N, D, 1, 0, _lib.KEOPS_F32)
    ws, have = _workspace(nbytes, x.device, workspace)
    st = lib.keops_lse(_ptr(x), _ptr(y), _ptr(out), M, N, D, float(sigma), _ptr(ws), have, _stream(x.device))
    _lib.check(st, "keops_lse")
    return out


def argkmin(x, y, K: int, with_dist: bool = False, idx=None, dist=None, workspace=None):
    """Indices (int32) of the K nearest columns per row, ascending, ties to the lower index."""
    torch = _torch()
    lib = _lib.load()
    M, D = _dims(x, 2)
    N, _ = _dims(y, 2)
    if idx is None:
        idx = torch.empty((M, K), dtype=torch.int32, device=x.device)
    if with_dist and dist is None:
        dist = torch.empty((M, K), dtype=torch.float32, device=x.device)
    nbytes = lib.keops_workspace_bytes(_lib.OP_ARGKMIN, 1, M, N, D, 1, K, _lib.KEOPS_F32)
    ws, have = _workspace(nbytes, x.device, workspace)
    st = lib.keops_argkmin(_ptr(x), _ptr(y), _ptr(idx), _ptr(dist), M, N, D, int(K), _ptr(ws), have,
                           _stream(x.device))
    _lib.check(st, "keops_argkmin")
    return (idx, dist) if with_dist else idx


def argkmin_weighted(x, y, w, K: int, with_dist: bool = False, idx=None, dist=None, workspace=None):
    """Indices (int32) of the K smallest keys |x_i - y_j|^2 - w_j per row, ascending, ties to
    the lower index; w is float32 (N,). K = 1 gives the weighted min / argmin."""
    torch = _torch()
    lib = _lib.load()
    M, D = _dims(x, 2)
    N, _ = _dims(y, 2)
    if w.dtype != torch.float32 or w.numel() != N or not w.is_contiguous():
        raise ValueError("w must be contiguous float32 with one entry per column")
    if idx is None:
        idx = torch.empty((M, K), dtype=torch.int32, device=x.device)
    if with_dist and dist is None:
        dist = torch.empty((M, K), dtype=torch.float32, device=x.device)
    nbytes = lib.keops_workspace_bytes(_lib.OP_ARGKMIN_WEIGHTED, 1, M, N, D, 1, K, _lib.KEOPS_F32)
    ws, have = _workspace(nbytes, x.device, workspace)
    st = lib.keops_argkmin_weighted(_ptr(x), _ptr(y), _ptr(w), _ptr(idx), _ptr(dist), M, N, D, int(K), _ptr(ws),
                                    have, _stream(x.device))
    _lib.check(st, "keops_argkmin_weighted")
    return (idx, dist) if with_dist else idx


def argkmin_lse(x, y, K: int, sigma: float, with_dist: bool = False, idx=None, dist=None, lse_out=None,
                workspace=None):
    """argKmin and the log-sum-exp reduction in one sweep; returns (idx, lse) or (idx, dist, lse)."""
    torch = _torch()
    lib = _lib.load()
    M, D = _dims(x, 2)
    N, _ = _dims(y, 2)
    if idx is None:
        idx = torch.empty((M, K), dtype=torch.int32, device=x.device)
    if with_dist and dist is None:
        dist = torch.empty((M, K), dtype=torch.float32, device=x.device)
    if lse_out is None:
        lse_out = torch.empty((M,), dtype=torch.float32, device=x.device)
    nbytes = lib.keops_workspace_bytes(_lib.OP_ARGKMIN_LSE, 1, M, N, D, 1, K, _lib.KEOPS_F32)
    ws, have = _workspace(nbytes, x.device, workspace)
    st = lib.keops_argkmin_lse(_ptr(x), _ptr(y), _ptr(idx), _ptr(dist), _ptr(lse_out), M, N, D, int(K), float(sigma),
                               _ptr(ws), have, _stream(x.device))
    _lib.check(st, "keops_argkmin_lse")
    return (idx, dist, lse_out) if with_dist else (idx, lse_out)


def gauss_sum_grad_x(x, y, b, g, sigma: float, out=None, workspace=None):
    """grad[i] = -(1/sigma^2) sum_j k_ij (g_i . b_j)(x_i - y_j); all float32, returns (M, D)."""
    torch = _torch()
    lib = _lib.load()
    M, D = _dims(x, 2)
    N, _ = _dims(y, 2)
    _, C = _dims(b, 2)
    _dims(g, 2)
    if out is None:
        out = torch.empty((M, D), dtype=torch.float32, device=x.device)
    nbytes = lib.keops_workspace_bytes(_lib.OP_GAUSS_SUM_GRAD_X, 1, M, N, D, C, 0, _lib.KEOPS_F32)
    ws, have = _workspace(nbytes, x.device, workspace)
    st = lib.keops_gauss_sum_grad_x(_ptr(x), _ptr(y), _ptr(b), _ptr(g), _ptr(out), M, N, D, C, float(sigma),
                                    _ptr(ws), have, _stream(x.device))
    _lib.check(st, "keops_gauss_sum_grad_x")
    return out


def gauss_sum_grad_y(x, y, b, g, sigma: float, out=None, workspace=None):
    """grad_y[j] = (1/sigma^2) sum_i k_ij (g_i . b_j)(x_i - y_j); all float32, returns (N, D)."""
    torch = _torch()
    lib = _lib.load()
    M, D = _dims(x, 2)
    N, _ = _dims(y, 2)
    _, C = _dims(b, 2)
    _dims(g, 2)
    if out is None:
        out = torch.empty((N, D), dtype=torch.float32, device=y.device)
    nbytes = lib.keops_workspace_bytes(_lib.OP_GAUSS_SUM_GRAD_Y, 1, M, N, D, C, 0, _lib.KEOPS_F32)
    ws, have = _workspace(nbytes, y.device, workspace)
    st = lib.keops_gauss_sum_grad_y(_ptr(x), _ptr(y), _ptr(b), _ptr(g), _ptr(out), M, N, D, C, float(sigma),
                                    _ptr(ws), have, _stream(y.device))
    _lib.check(st, "keops_gauss_sum_grad_y")
    return out


def gauss_sum_grad_b(x, y, g, sigma: float, out=None, workspace=None):
    """grad_b[j] = sum_i k_ij g_i; all float32, returns (N, C)."""
    torch = _torch()
    lib = _lib.load()
    M, D = _dims(x, 2)
    N, _ = _dims(y, 2)
    _, C = _dims(g, 2)
    if out is None:
        out = torch.empty((N, C), dtype=torch.float32, device=y.device)
    nbytes = lib.keops_workspace_bytes(_lib.OP_GAUSS_SUM_GRAD_B, 1, M, N, D, C, 0, _lib.KEOPS_F32)
    ws, have = _workspace(nbytes, y.device, workspace)
    st = lib.keops_gauss_sum_grad_b(_ptr(x), _ptr(y), _ptr(g), _ptr(out), M, N, D, C, float(sigma),
                                    _ptr(ws), have, _stream(y.device))
    _lib.check(st, "keops_gauss_sum_grad_b")
    return out


def gauss_sum_autograd(x, y, b, sigma: float):
    """The float32 Gauss sum as a differentiable PyTorch op: forward and the gradients with
    respect to x, y and b all run in this library's kernels."""
    from .autograd import GaussSum
    return GaussSum.apply(x, y, b, float(sigma))
