"""Plain float64 CPU oracle for fused pairwise kernel reductions.

TEST INFRASTRUCTURE ONLY. Nothing in the product package imports this module; only the
tests, the smoke check and the benchmark's CPU-baseline leg may call it. It shares no code
with the device path: every quantity is computed here from its textbook definition in
numpy float64, row block by row block, with no fusion, reordering or expansion of
||x - y||^2 beyond what the definition states.

Sources (cited by page title and section):
  [KMR]  "Kernel matrix reduction" (concept page): Overview (the reduction
         a_i = Reduction_j F(p, x_i, y_j) and its list of reductions: sums, log-sum-exp,
         maxima/minima, indices of the K smallest entries), Variants (autodiff), and the
         Implementation sketch (eq. 1, the Gaussian kernel matrix-vector product; eq. 2,
         the double-loop meaning of a generic reduction).
  [KEOPS] "KeOps: a symbolic tensor that never materialises the matrix it represents":
         the LazyTensor example (K_ij = exp(-D_ij), a_i = sum_j K_ij, and the gradient of
         sum_i a_i^2 with respect to x).
  [RUX]  "Fast Gauss Sums via Flash Attention" (Rux & Neumayer): abstract and the Output
         row of Algorithms 1 and 2, s_m = sum_n Phi_tau(q_m, k_n) v_n with signed weights;
         Figure 2 times the same sum's forward and backward.
  [FD]   "FlashDiffusion: Fused Tiled Kernel Spectral Decomposition", section 2.2: the
         diffusion operator diag(s) K diag(s) applied to a block V, and its q and d
         normalisation passes (kernel applications with V replaced by 1 and by q^-alpha).

Inputs are the exact float32 / float16 arrays the device receives, widened exactly to
float64. sigma is whatever value the caller passes (pass float(np.float32(sigma)) so both
sides see the same bandwidth).

Parity pins for every function live in tests/test_oracle.py; none is unpinned.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from typing import Callable, Optional, Tuple

import numpy as np

# Rows per block are chosen so that one (rows x N) float64 temporary stays near 32 MiB.
_BLOCK_ELEMS = 1 << 22


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _row_blocks(M: int, N: int):
    step = max(1, _BLOCK_ELEMS // max(N, 1))
    for r0 in range(0, M, step):
        yield slice(r0, min(M, r0 + step))


def squared_distances(xr: np.ndarray, y: np.ndarray) -> np.ndarray:
    """d2[i, j] = sum_d (x[i, d] - y[j, d])^2 for a block of rows.

    The differences are taken first and the squares are summed over d in increasing order,
    each operation rounded in IEEE float64 (numpy applies no fused multiply-add):
    d2 = ((dx0*dx0 + dx1*dx1) + dx2*dx2) + ... This is the key the argKmin reduction ranks
    by; when the inputs lie on a fine enough dyadic grid (see ``keys_are_exact``) every one
    of these operations is exact and d2 is the true squared distance.
    """
    m, n, D = xr.shape[0], y.shape[0], xr.shape[1]
    d2 = np.zeros((m, n), dtype=np.float64)
    for d in range(D):
        diff = xr[:, d][:, None] - y[:, d][None, :]
        d2 += diff * diff
    return d2


def keys_are_exact(x, y) -> bool:
    """True when float64 evaluates every squared distance between rows of x and y exactly.

    Sufficient condition: all coordinates are integer multiples of 2^-p with magnitude
    below 2^r, so each difference is a multiple of 2^-p below 2^(r+1), each square a
    multiple of 2^-2p below 2^(2r+2), and a sum of D squares needs at most
    2(r+p) + 2 + ceil(log2 D) significant bits; exact when that is <= 53.
    """
    x = _f64(x)
    y = _f64(y)
    allv = np.concatenate([x.ravel(), y.ravel()])
    if allv.size == 0:
        return True
    if not np.all(np.isfinite(allv)):
        return False
    mag = float(np.max(np.abs(allv)))
    r = 0 if mag == 0.0 else int(np.floor(np.log2(mag))) + 1
    D = x.shape[1]
    for p in range(0, 60):
        scaled = allv * (2.0 ** p)
        if np.all(scaled == np.round(scaled)):
            bits = 2 * (r + p) + 2 + int(np.ceil(np.log2(max(D, 1))))
            return bits <= 53
    return False


def _parallel_rows(fn: Callable[[slice], None], M: int, N: int, workers: Optional[int]):
    """Run ``fn`` over row blocks, serially or on ``workers`` threads.

    BLAS is held to one thread in both modes so the result does not depend on the worker
    count (numpy releases the GIL inside its array loops; no process is forked).
    """
    blocks = list(_row_blocks(M, N))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover - threadpoolctl is optional
        limiter = None
    try:
        if workers is None or workers <= 1 or len(blocks) <= 1:
            for sl in blocks:
                fn(sl)
        else:
            with _cf.ThreadPoolExecutor(max_workers=workers) as ex:
                list(ex.map(fn, blocks))
    finally:
        if limiter is not None:
            limiter.restore_original_limits()


def gauss_sum(x, y, b, sigma: float, workers: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Gaussian kernel matrix-vector product [KMR, Implementation sketch, eq. 1].

    s[i, c] = sum_j exp(-||x_i - y_j||^2 / (2 sigma^2)) * b[j, c]
    Returns (s, n) where n[i, c] = sum_j |k_ij * b[j, c]| is the row normaliser the
    tolerance is measured against. x: (M, D), y: (N, D), b: (N,) or (N, C).
    """
    x = _f64(x)
    y = _f64(y)
    b = _f64(b)
    if b.ndim == 1:
        b = b[:, None]
    M, N, C = x.shape[0], y.shape[0], b.shape[1]
    s = np.zeros((M, C))
    n = np.zeros((M, C))
    two_sigma2 = 2.0 * float(sigma) * float(sigma)
    absb = np.abs(b)

    def block(sl):
        d2 = squared_distances(x[sl], y)
        k = np.exp(-d2 / two_sigma2)
        s[sl] = k @ b
        n[sl] = k @ absb

    if N > 0:
        _parallel_rows(block, M, N, workers)
    return s, n


def gauss_sum_batched(q, k, v, tau: float, workers: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Batched Gauss sum with signed weights [RUX, Algorithm 1/2 Output row].

    s[t, m, c] = sum_n Phi_tau(q[t, m], k[t, n]) v[t, n, c], Phi_tau(q, k) = exp(-tau/2 ||q-k||^2),
    independently for every batch index t. Returns (s, n) with n = sum_n |Phi v|.
    q: (B, M, D), k: (B, N, D), v: (B, N, C), any float dtype (widened exactly).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    B, M, C = q.shape[0], q.shape[1], v.shape[2]
    s = np.zeros((B, M, C))
    n = np.zeros((B, M, C))
    half_tau = 0.5 * float(tau)
    for t in range(B):
        kt, vt, absv = k[t], v[t], np.abs(v[t])
        qt = q[t]

        def block(sl, qt=qt, kt=kt, vt=vt, absv=absv, t=t):
            phi = np.exp(-half_tau * squared_distances(qt[sl], kt))
            s[t, sl] = phi @ vt
            n[t, sl] = phi @ absv

        if kt.shape[0] > 0:
            _parallel_rows(block, M, kt.shape[0], workers)
    return s, n


def logsumexp_reduction(x, y, sigma: float, workers: Optional[int] = None) -> np.ndarray:
    """Log-sum-exp reduction [KMR, Overview, list of reductions].

    out[i] = log sum_j exp(f_ij), f_ij = -||x_i - y_j||^2 / (2 sigma^2), evaluated with the
    row maximum m_i = max_j f_ij factored out: out_i = m_i + log sum_j exp(f_ij - m_i).
    An empty column set gives -inf.
    """
    x = _f64(x)
    y = _f64(y)
    M, N = x.shape[0], y.shape[0]
    out = np.full(M, -np.inf)
    two_sigma2 = 2.0 * float(sigma) * float(sigma)

    def block(sl):
        f = -squared_distances(x[sl], y) / two_sigma2
        m = f.max(axis=1)
        out[sl] = m + np.log(np.exp(f - m[:, None]).sum(axis=1))

    if N > 0:
        _parallel_rows(block, M, N, workers)
    return out


def argkmin(x, y, K: int, workers: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Indices of the K smallest squared distances per row [KMR, Overview].

    Row i ranks the columns j by the key (d2_ij, j) ascending, i.e. a stable sort of the
    row of squared distances, so equal distances keep the lower index first. Returns
    (idx (M, K) int64, d2 (M, K) float64). Requires 1 <= K <= N.
    """
    x = _f64(x)
    y = _f64(y)
    M, N = x.shape[0], y.shape[0]
    if not (1 <= K <= N):
        raise ValueError("argkmin needs 1 <= K <= N")
    idx = np.zeros((M, K), dtype=np.int64)
    dist = np.zeros((M, K))

    def block(sl):
        d2 = squared_distances(x[sl], y)
        order = np.argsort(d2, axis=1, kind="stable")[:, :K]
        idx[sl] = order
        dist[sl] = np.take_along_axis(d2, order, axis=1)

    _parallel_rows(block, M, N, workers)
    return idx, dist


def argkmin_weighted(x, y, w, K: int, workers: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Indices of the K smallest additively weighted squared distances per row [KMR, Overview:
    minima and indices of the K smallest entries of a pairwise formula].

    Row i ranks the columns j by the key (d2_ij - w_j, j) ascending (a stable sort of the row
    of keys), d2_ij as in ``squared_distances`` and the difference taken in float64. Returns
    (idx (M, K) int64, keys (M, K) float64). Requires 1 <= K <= N.
    """
    x = _f64(x)
    y = _f64(y)
    w = _f64(w)
    M, N = x.shape[0], y.shape[0]
    if not (1 <= K <= N):
        raise ValueError("argkmin needs 1 <= K <= N")
    idx = np.zeros((M, K), dtype=np.int64)
    keys = np.zeros((M, K))

    def block(sl):
        kk = squared_distances(x[sl], y) - w[None, :]
        order = np.argsort(kk, axis=1, kind="stable")[:, :K]
        idx[sl] = order
        keys[sl] = np.take_along_axis(kk, order, axis=1)

    _parallel_rows(block, M, N, workers)
    return idx, keys


def gauss_sum_grad_x(x, y, b, g, sigma: float, workers: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Gradient of the Gauss sum with respect to x, contracted with an upstream gradient.

    [KMR, Variants: each partial derivative is its own reduction] and [KEOPS, the
    autograd example]: for s_i = sum_j k_ij b_j with k_ij = exp(-||x_i - y_j||^2/(2 sigma^2)),
    d k_ij / d x_i = -k_ij (x_i - y_j) / sigma^2, so the vector-Jacobian product with an
    upstream gradient g (M, C) is
        grad[i, :] = -(1/sigma^2) sum_j k_ij (g_i . b_j) (x_i - y_j).
    Returns (grad (M, D), n (M, D)) with n[i, d] = (1/sigma^2) sum_j |k_ij (g_i . b_j)(x_id - y_jd)|.
    """
    x = _f64(x)
    y = _f64(y)
    b = _f64(b)
    g = _f64(g)
    if b.ndim == 1:
        b = b[:, None]
    if g.ndim == 1:
        g = g[:, None]
    M, N, D = x.shape[0], y.shape[0], x.shape[1]
    grad = np.zeros((M, D))
    n = np.zeros((M, D))
    sigma2 = float(sigma) * float(sigma)

    def block(sl):
        k = np.exp(-squared_distances(x[sl], y) / (2.0 * sigma2))
        w = k * (g[sl] @ b.T)
        for d in range(D):
            diff = x[sl, d][:, None] - y[:, d][None, :]
            term = w * diff
            grad[sl, d] = -term.sum(axis=1) / sigma2
            n[sl, d] = np.abs(term).sum(axis=1) / sigma2

    if N > 0:
        _parallel_rows(block, M, N, workers)
    return grad, n


def gauss_sum_grad_y(x, y, b, g, sigma: float, workers: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Gradient of the Gauss sum with respect to the columns y, contracted with g.

    [KMR, Variants: each partial derivative is its own reduction]: d k_ij / d y_j =
    +k_ij (x_i - y_j) / sigma^2, so
        grad_y[j, :] = (1/sigma^2) sum_i k_ij (g_i . b_j) (x_i - y_j),
    a reduction over the rows i for every column j.
    Returns (grad_y (N, D), n (N, D)) with n[j, d] = (1/sigma^2) sum_i |k_ij (g_i . b_j)(x_id - y_jd)|.
    """
    x = _f64(x)
    y = _f64(y)
    b = _f64(b)
    g = _f64(g)
    if b.ndim == 1:
        b = b[:, None]
    if g.ndim == 1:
        g = g[:, None]
    M, N, D = x.shape[0], y.shape[0], y.shape[1]
    grad = np.zeros((N, D))
    n = np.zeros((N, D))
    sigma2 = float(sigma) * float(sigma)

    def block(sl):  # a block of columns j
        k = np.exp(-squared_distances(y[sl], x) / (2.0 * sigma2))   # (cols, M)
        w = k * (b[sl] @ g.T)
        for d in range(D):
            diff = x[:, d][None, :] - y[sl, d][:, None]
            term = w * diff
            grad[sl, d] = term.sum(axis=1) / sigma2
            n[sl, d] = np.abs(term).sum(axis=1) / sigma2

    if M > 0:
        _parallel_rows(block, N, M, workers)
    return grad, n


def gauss_sum_grad_b(x, y, g, sigma: float, workers: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Gradient of the Gauss sum with respect to the weights b, contracted with g.

    s_ic = sum_j k_ij b_jc is linear in b, so grad_b[j, c] = sum_i k_ij g_ic: the Gauss sum
    with the roles of rows and columns exchanged. Returns (grad_b (N, C), n = sum_i |k_ij g_ic|).
    """
    x = _f64(x)
    y = _f64(y)
    g = _f64(g)
    if g.ndim == 1:
        g = g[:, None]
    M, N, C = x.shape[0], y.shape[0], g.shape[1]
    grad = np.zeros((N, C))
    n = np.zeros((N, C))
    two_sigma2 = 2.0 * float(sigma) * float(sigma)
    absg = np.abs(g)

    def block(sl):
        k = np.exp(-squared_distances(y[sl], x) / two_sigma2)         # (cols, M)
        grad[sl] = k @ g
        n[sl] = k @ absg

    if M > 0:
        _parallel_rows(block, N, M, workers)
    return grad, n


def gauss_sum_scaled(x, y, b, sigma: float, row_scale=None, col_scale=None,
                     workers: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Two-sided scaled Gauss sum [FD, section 2.2]: out = diag(r) K diag(c) b.

    s[i, c'] = r_i sum_j k_ij c_j b[j, c'], evaluated as the plain Gauss sum of the weights
    c_j b_j, then scaled row by row. A missing scale is all ones. Returns (s, n) with
    n[i, c'] = |r_i| sum_j |k_ij c_j b[j, c']|.
    """
    b = _f64(b)
    if b.ndim == 1:
        b = b[:, None]
    if col_scale is not None:
        b = _f64(col_scale)[:, None] * b
    s, n = gauss_sum(x, y, b, sigma, workers)
    if row_scale is not None:
        r = _f64(row_scale)[:, None]
        s = r * s
        n = np.abs(r) * n
    return s, n


def diffusion_scaling(x, sigma: float, alpha: float,
                      workers: Optional[int] = None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Normalisation of the diffusion operator [FD, section 2.2], for K_ij = k(x_i, x_j).

    The q pass applies K to ones and the d pass applies the alpha-normalised kernel
    K_alpha = diag(q^-alpha) K diag(q^-alpha) to ones; the symmetric operator is then
    diag(s) K diag(s) with s = q^-alpha d^-1/2:
        q = K 1,  p = q^-alpha,  d = p * (K p),  s = p / sqrt(d).
    Returns (s, q, d).
    """
    x = _f64(x)
    N = x.shape[0]
    q = gauss_sum(x, x, np.ones(N), sigma, workers)[0][:, 0]
    p = q ** (-float(alpha))
    d = p * gauss_sum(x, x, p, sigma, workers)[0][:, 0]
    return p / np.sqrt(d), q, d


def gauss_sum_batched_backward(x, y, b, g, sigma: float, workers: Optional[int] = None) -> dict:
    """Gradients of the batched Gauss sum [RUX, eq. (1); Figure 2 times forward + backward].

    For every batch index t independently, the gradients of s = sum_j k_ij b_j contracted
    with the upstream g (B, M, C), as in gauss_sum_grad_x / _grad_y / _grad_b. Returns
    {"x": (grad, n), "y": (grad, n), "b": (grad, n)}, each stacked over the batch.
    """
    x = _f64(x)
    y = _f64(y)
    b = _f64(b)
    g = _f64(g)
    parts = {"x": [], "y": [], "b": []}
    for t in range(x.shape[0]):
        parts["x"].append(gauss_sum_grad_x(x[t], y[t], b[t], g[t], sigma, workers))
        parts["y"].append(gauss_sum_grad_y(x[t], y[t], b[t], g[t], sigma, workers))
        parts["b"].append(gauss_sum_grad_b(x[t], y[t], g[t], sigma, workers))
    return {key: (np.stack([p[0] for p in v]), np.stack([p[1] for p in v])) for key, v in parts.items()}


def default_workers() -> int:
    """Host threads the oracle uses when asked to run in parallel."""
    return max(1, os.cpu_count() or 1)
