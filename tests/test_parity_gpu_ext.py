"""Parity of the extended entry points (through the C ABI) with the float64 oracle:
the fp16 matrix-core backward, the fp16 path at every feature width, the two-sided scaled
Gauss sum and the diffusion normalisation passes.

Tolerances: fp16 path 2e-3 of the oracle relative to the normaliser (sum_j |k_ij b_j| for
sums, sum_j |k_ij (g_i.b_j)(x_i - y_j)| / sigma^2 for gradients); float32 path 1e-4; the
diffusion scalings (positive sums and their powers) within 4e-3 (fp16) / 2e-4 (float32)
relative.
"""
import numpy as np
import pytest

import oracle
from pairwise_reductions_amd import workloads
from test_parity_gpu import TOL_F16, TOL_F32, _announce, _dev, _highd_inputs, _host, _rand, assert_normalised

pytestmark = pytest.mark.gpu


def _oracle_backward(x, y, b, g, sigma):
    return oracle.gauss_sum_batched_backward(x, y, b, g, sigma, workers=8)


# ------------------------------------------------------------------ fp16 forward widths
WIDTH_SHAPES = [
    # (B, M, N, D, C, sigma): D not a multiple of 32 reads padded features as zero
    (2, 300, 1000, 16, 32, 0.7), (1, 513, 2000, 48, 16, 1.0), (2, 257, 1500, 96, 32, 1.2),
    (1, 700, 3000, 128, 64, 1.5), (3, 129, 777, 128, 1, 1.0), (1, 1000, 4096, 80, 8, 1.0),
]


@pytest.mark.parametrize("B,M,N,D,C,sigma", WIDTH_SHAPES)
def test_gauss_sum_fp16_feature_widths(B, M, N, D, C, sigma):
    import pairwise_reductions_amd as pr
    _announce("gauss_sum_fp16_width", B=B, M=M, N=N, D=D, C=C, sigma=sigma)
    q, k, v = _highd_inputs(B * 7 + M + D, B, M, N, D, C)
    sig = float(np.float32(sigma))
    got = _host(pr.gauss_sum(_dev(q), _dev(k), _dev(v), sig))
    want, norm = oracle.gauss_sum_batched(q, k, v, 1.0 / (sig * sig), workers=8)
    assert_normalised(got, want, norm, TOL_F16, "fp16 width")


# ---------------------------------------------------- fp16 forward: folded and FMA waves
def _norm_ramp_inputs(seed, B, M, N, D, C, rmax):
    """Keys ~ N(0, I/D); queries in random directions with norms rising linearly from 0 to rmax
    along the row index, so the waves of one launch go from small to large |q| (the folded form
    of the fp16 forward is open to the first and closed to the last); weights ~ N(0, 1)."""
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((B, M, D))
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    r = np.linspace(0.0, rmax, M)[None, :, None]
    q = (u * r).astype(np.float16)
    k = (rng.standard_normal((B, N, D)) / np.sqrt(D)).astype(np.float16)
    v = rng.standard_normal((B, N, C)).astype(np.float16)
    return q, k, v


FOLD_CASES = [
    # (kind, B, M, N, D, C, sigma): "plain" N(0, I/D) points, "ramp" query norms 0..4, "offset"
    # every point moved by +1.5 per feature (|q| ~ 8: no wave folds)
    ("plain", 2, 2100, 6000, 32, 32, 1.0), ("ramp", 2, 2100, 6000, 32, 32, 1.0), ("ramp", 1, 3000, 4100, 24, 20, 0.8),
    ("offset", 1, 1100, 3000, 32, 32, 1.0), ("plain", 1, 1025, 20000, 32, 32, 0.6),
    # the 16x16x32 forward (C <= 16, or D > 32): the same two forms
    ("plain", 2, 2100, 6000, 32, 1, 1.0), ("ramp", 1, 3000, 4100, 64, 8, 0.8), ("ramp", 2, 1500, 3000, 128, 64, 1.2),
    ("plain", 1, 1025, 9000, 96, 16, 1.0), ("offset", 1, 1100, 3000, 64, 3, 1.0), ("plain", 3, 700, 2500, 20, 2, 0.7),
    # the decision right before a last stage holding one key, or a ragged one; tiny row counts
    ("plain", 1, 33, 129, 32, 32, 1.0), ("ramp", 2, 1025, 257, 32, 17, 1.0), ("plain", 1, 17, 130, 32, 1, 1.0),
    ("plain", 2, 100, 200, 64, 8, 0.9), ("ramp", 1, 5, 65, 128, 3, 1.1),
]


@pytest.mark.parametrize("kind,B,M,N,D,C,sigma", FOLD_CASES)
def test_gauss_sum_fp16_folded_and_fma_waves(kind, B, M, N, D, C, sigma):
    """The fp16 forward sweeps (32x32x16 and 16x16x32 tiles) keep cs S + alpha per value or, per
    wave, fold cs into the query operands and move the row shifts into the output scale; both
    forms, mixed in one launch, against the oracle."""
    import pairwise_reductions_amd as pr
    _announce("fp16_fold", kind=kind, B=B, M=M, N=N, D=D, C=C, sigma=sigma)
    if kind == "ramp":
        q, k, v = _norm_ramp_inputs(B * 11 + M + N, B, M, N, D, C, 4.0)
    else:
        q, k, v = _highd_inputs(B * 13 + M + N, B, M, N, D, C)
        if kind == "offset":
            q = (q.astype(np.float32) + 1.5).astype(np.float16)
            k = (k.astype(np.float32) + 1.5).astype(np.float16)
    sig = float(np.float32(sigma))
    got = _host(pr.gauss_sum(_dev(q), _dev(k), _dev(v), sig))
    want, norm = oracle.gauss_sum_batched(q, k, v, 1.0 / (sig * sig), workers=8)
    assert_normalised(got, want, norm, TOL_F16, f"fp16 forward {kind}")


BWD_RAMP_CASES = [
    # (kind, B, M, N, D, C, sigma): query norms rising along the rows, plain and offset points
    ("ramp", 2, 2100, 3000, 32, 1, 1.0), ("ramp", 1, 1500, 2000, 64, 3, 0.8), ("plain", 1, 1100, 2500, 32, 16, 1.0),
    ("offset", 1, 700, 1500, 32, 2, 1.0),
]


@pytest.mark.parametrize("kind,B,M,N,D,C,sigma", BWD_RAMP_CASES)
def test_gauss_sum_backward_fp16_norm_ramp_and_offset(kind, B, M, N, D, C, sigma):
    """x, y and b gradients for queries whose norms rise from 0 to 4 along the rows (row shifts
    of every size in one launch), plain N(0, I/D) points and points moved far from the origin."""
    import pairwise_reductions_amd as pr
    _announce("backward_fp16_ramp", kind=kind, B=B, M=M, N=N, D=D, C=C, sigma=sigma)
    if kind == "ramp":
        q, k, v = _norm_ramp_inputs(B * 17 + M + N, B, M, N, D, C, 4.0)
    else:
        q, k, v = _highd_inputs(B * 19 + M + N, B, M, N, D, C)
        if kind == "offset":
            q = (q.astype(np.float32) + 1.5).astype(np.float16)
            k = (k.astype(np.float32) + 1.5).astype(np.float16)
    g = workloads.upstream_gradient(M, C, seed=M + N + D, B=B)
    sig = float(np.float32(sigma))
    got = pr.gauss_sum_backward(_dev(q), _dev(k), _dev(v), _dev(g), sig)
    want = _oracle_backward(q, k, v, g, sig)
    for key in ("x", "y", "b"):
        assert_normalised(_host(got[key]), want[key][0], want[key][1], TOL_F16, f"backward {kind} {key}")


# ------------------------------------------------------------------ fp16 backward
BWD_SHAPES = [
    # (B, M, N, D, C, sigma)
    (1, 1, 1, 32, 1, 1.0), (1, 100, 77, 32, 1, 1.0), (2, 300, 1000, 32, 32, 0.7),
    (4, 513, 2049, 32, 1, 1.0), (1, 1024, 3000, 64, 32, 1.5), (2, 257, 300, 32, 64, 1.0),
    (1, 700, 1500, 16, 3, 0.8), (1, 400, 900, 96, 17, 1.2), (2, 333, 1200, 128, 48, 1.5),
    (1, 2000, 600, 48, 2, 0.9),
]


@pytest.mark.parametrize("B,M,N,D,C,sigma", BWD_SHAPES)
def test_gauss_sum_backward_fp16_shapes(B, M, N, D, C, sigma):
    import pairwise_reductions_amd as pr
    _announce("backward_fp16", B=B, M=M, N=N, D=D, C=C, sigma=sigma)
    q, k, v = _highd_inputs(B * 5 + M * 3 + N, B, M, N, D, C)
    g = workloads.upstream_gradient(M, C, seed=M + N, B=B)
    sig = float(np.float32(sigma))
    got = pr.gauss_sum_backward(_dev(q), _dev(k), _dev(v), _dev(g), sig)
    want = _oracle_backward(q, k, v, g, sig)
    for key in ("x", "y", "b"):
        assert_normalised(_host(got[key]), want[key][0], want[key][1], TOL_F16, f"backward fp16 {key}")


def test_gauss_sum_backward_fp16_subsets_and_large_weights():
    """Only some gradients requested; weights far outside the fp16 range of products
    (|v| ~ 3e3, |g| ~ 1e5) and zero weight rows / columns, which the normalisation handles."""
    import pairwise_reductions_amd as pr
    _announce("backward_fp16_large")
    B, M, N, D, C = 2, 600, 1100, 32, 4
    q, k, v = _highd_inputs(91, B, M, N, D, C)
    v = (v.astype(np.float32) * 3000.0).astype(np.float16)
    v[:, 5:40] = 0
    g = workloads.upstream_gradient(M, C, seed=92, B=B) * np.float32(1e5)
    g[:, 7:19] = 0
    sig = 1.0
    want = _oracle_backward(q, k, v, g, sig)
    for need in (("x",), ("y", "b"), ("x", "y", "b")):
        got = pr.gauss_sum_backward(_dev(q), _dev(k), _dev(v), _dev(g), sig, need=need)
        assert set(got) == set(need)
        for key in need:
            assert_normalised(_host(got[key]), want[key][0], want[key][1], TOL_F16, f"large {key}")


def test_gauss_sum_backward_fp16_far_rows():
    """Rows far from every key: the kernel values underflow fp16 without the running shift."""
    import pairwise_reductions_amd as pr
    _announce("backward_fp16_far")
    q, k, v = _highd_inputs(93, 2, 500, 2000, 32, 1, shift=1.0)
    g = workloads.upstream_gradient(500, 1, seed=94, B=2)
    got = pr.gauss_sum_backward(_dev(q), _dev(k), _dev(v), _dev(g), 1.0)
    want = _oracle_backward(q, k, v, g, 1.0)
    for key in ("x", "y", "b"):
        assert_normalised(_host(got[key]), want[key][0], want[key][1], TOL_F16, f"far {key}")


def test_gauss_sum_backward_fp16_workload_sampled():
    """The B=4, M=N=16384, D=32, C=1 forward + backward at full size: gradients with respect
    to x on sampled rows, with respect to y and b on sampled columns."""
    import pairwise_reductions_amd as pr
    inp = workloads.make_inputs("batched_gauss_sum_fp16_fwd_bwd")
    B, M, N, C = inp["B"], inp["M"], inp["N"], inp["C"]
    _announce("backward_fp16_workload", B=B, M=M, N=N, C=C)
    sig = float(inp["sigma"])
    xd, yd, bd = _dev(inp["x"]), _dev(inp["y"]), _dev(inp["b"])
    s = pr.gauss_sum(xd, yd, bd, sig)
    g = workloads.upstream_gradient(M, C, seed=4, B=B)
    got = pr.gauss_sum_backward(xd, yd, bd, _dev(g), sig)
    rows = workloads.sample_rows(M, 128, seed=5)
    cols = workloads.sample_rows(N, 128, seed=6)
    x, y, b = inp["x"], inp["y"], inp["b"]
    want_s, norm_s = oracle.gauss_sum_batched(x[:, rows], y, b, 1.0 / (sig * sig), workers=8)
    assert_normalised(_host(s)[:, rows], want_s, norm_s, TOL_F16, "workload forward")
    gx, gy, gb = _host(got["x"]), _host(got["y"]), _host(got["b"])
    for t in range(B):
        wx, nx = oracle.gauss_sum_grad_x(x[t, rows], y[t], b[t], g[t, rows], sig, workers=8)
        assert_normalised(gx[t, rows], wx, nx, TOL_F16, "workload grad x")
        wy, ny = oracle.gauss_sum_grad_y(x[t], y[t, cols], b[t, cols], g[t], sig, workers=8)
        assert_normalised(gy[t, cols], wy, ny, TOL_F16, "workload grad y")
        wb, nb = oracle.gauss_sum_grad_b(x[t], y[t, cols], g[t], sig, workers=8)
        assert_normalised(gb[t, cols], wb, nb, TOL_F16, "workload grad b")


def test_autograd_fp16():
    """The autograd wrapper on fp16 batched inputs: forward and fp16-cast gradients."""
    import torch
    import pairwise_reductions_amd as pr
    _announce("autograd_fp16")
    q, k, v = _highd_inputs(95, 2, 300, 700, 32, 2)
    w = workloads.upstream_gradient(300, 2, seed=96, B=2)
    qd = _dev(q).requires_grad_(True)
    kd = _dev(k).requires_grad_(True)
    vd = _dev(v).requires_grad_(True)
    s = pr.gauss_sum_autograd(qd, kd, vd, 1.0)
    (s * _dev(w)).sum().backward()
    torch.cuda.synchronize()
    want = _oracle_backward(q, k, v, w, 1.0)
    for key, t in (("x", qd), ("y", kd), ("b", vd)):
        assert t.grad.dtype == torch.float16
        # the fp16 cast of the gradient adds one more rounding of 2^-11 relative
        assert_normalised(t.grad.float().cpu().numpy(), want[key][0], want[key][1], 2 * TOL_F16, f"autograd {key}")


# ------------------------------------------------------------------ float32 backward entry
@pytest.mark.parametrize("M,N,D,C,sigma", [(1, 1, 3, 1, 0.1), (700, 2000, 2, 3, 0.2), (2049, 1537, 3, 1, 0.05),
                                           (513, 4097, 8, 8, 0.5)])
def test_gauss_sum_backward_f32(M, N, D, C, sigma):
    import pairwise_reductions_amd as pr
    _announce("backward_f32", M=M, N=N, D=D, C=C, sigma=sigma)
    x, y, b = _rand(M + 3 * N, M, N, D, C)
    g = workloads.upstream_gradient(M, C, seed=M)
    sig = float(np.float32(sigma))
    got = pr.gauss_sum_backward(_dev(x), _dev(y), _dev(b), _dev(g), sig)
    wx, nx = oracle.gauss_sum_grad_x(x, y, b, g, sig, workers=8)
    wy, ny = oracle.gauss_sum_grad_y(x, y, b, g, sig, workers=8)
    wb, nb = oracle.gauss_sum_grad_b(x, y, g, sig, workers=8)
    assert_normalised(_host(got["x"]), wx, nx, TOL_F32, "backward f32 x")
    assert_normalised(_host(got["y"]), wy, ny, TOL_F32, "backward f32 y")
    assert_normalised(_host(got["b"]), wb, nb, TOL_F32, "backward f32 b")


# ------------------------------------------------------------------ scaled Gauss sum
SCALED_SHAPES = [(1, 1, 3, 1, 0.1), (257, 1000, 3, 2, 0.1), (1025, 513, 1, 1, 0.05), (3000, 70_001, 3, 4, 0.02)]


@pytest.mark.parametrize("M,N,D,C,sigma", SCALED_SHAPES)
def test_gauss_sum_scaled_f32(M, N, D, C, sigma):
    import pairwise_reductions_amd as pr
    _announce("scaled_f32", M=M, N=N, D=D, C=C, sigma=sigma)
    x, y, b = _rand(M * 5 + N, M, N, D, C)
    rng = np.random.default_rng(M + N)
    r = rng.standard_normal(M).astype(np.float32)
    c = rng.standard_normal(N).astype(np.float32)
    sig = float(np.float32(sigma))
    for rs, cs in ((r, c), (r, None), (None, c), (None, None)):
        got = _host(pr.gauss_sum_scaled(_dev(x), _dev(y), _dev(b), sig,
                                        row_scale=None if rs is None else _dev(rs),
                                        col_scale=None if cs is None else _dev(cs)))
        want, norm = oracle.gauss_sum_scaled(x, y, b, sig, row_scale=rs, col_scale=cs, workers=8)
        assert_normalised(got, want, norm, TOL_F32, "scaled f32")


@pytest.mark.parametrize("B,M,N,D,C,sigma", [(2, 300, 1000, 32, 32, 0.7), (1, 513, 2049, 64, 3, 1.0),
                                             (3, 100, 4000, 16, 1, 1.0)])
def test_gauss_sum_scaled_fp16(B, M, N, D, C, sigma):
    import pairwise_reductions_amd as pr
    _announce("scaled_fp16", B=B, M=M, N=N, D=D, C=C, sigma=sigma)
    q, k, v = _highd_inputs(B + M + N, B, M, N, D, C)
    rng = np.random.default_rng(M * N)
    r = rng.standard_normal((B, M)).astype(np.float32)
    c = (rng.standard_normal((B, N)) * 100.0).astype(np.float32)
    sig = float(np.float32(sigma))
    got = _host(pr.gauss_sum_scaled(_dev(q), _dev(k), _dev(v), sig, row_scale=_dev(r), col_scale=_dev(c)))
    for t in range(B):
        want, norm = oracle.gauss_sum_scaled(q[t], k[t], v[t], sig, row_scale=r[t], col_scale=c[t], workers=8)
        assert_normalised(got[t], want, norm, TOL_F16, "scaled fp16")


# ------------------------------------------------------------------ diffusion scaling
@pytest.mark.parametrize("N,D,sigma,alpha", [(1, 3, 0.1, 0.5), (1000, 3, 0.1, 0.5), (4097, 2, 0.05, 1.0),
                                             (20_000, 3, 0.05, 0.0)])
def test_diffusion_scaling_f32(N, D, sigma, alpha):
    import pairwise_reductions_amd as pr
    _announce("diffusion_f32", N=N, D=D, sigma=sigma, alpha=alpha)
    x, _, _ = _rand(N + D, N, 1, D, 1)
    sig = float(np.float32(sigma))
    s, q, d = (_host(t) for t in pr.diffusion_scaling(_dev(x), sig, alpha))
    ws, wq, wd = oracle.diffusion_scaling(x, sig, alpha, workers=8)
    for got, want, name in ((q, wq, "q"), (d, wd, "d"), (s, ws, "s")):
        rel = np.max(np.abs(got - want) / np.abs(want))
        assert rel <= 2e-4, f"diffusion f32 {name}: {rel:.3e}"


@pytest.mark.parametrize("B,N,D,sigma,alpha", [(2, 1000, 32, 1.0, 0.5), (1, 3000, 64, 1.5, 1.0)])
def test_diffusion_scaling_fp16(B, N, D, sigma, alpha):
    import pairwise_reductions_amd as pr
    _announce("diffusion_fp16", B=B, N=N, D=D, sigma=sigma, alpha=alpha)
    x, _, _ = _highd_inputs(N + B, B, N, 1, D, 1)
    sig = float(np.float32(sigma))
    s, q, d = (_host(t) for t in pr.diffusion_scaling(_dev(x), sig, alpha))
    for t in range(B):
        ws, wq, wd = oracle.diffusion_scaling(x[t], sig, alpha, workers=8)
        for got, want, name in ((q[t], wq, "q"), (d[t], wd, "d"), (s[t], ws, "s")):
            rel = np.max(np.abs(got - want) / np.abs(want))
            assert rel <= 4e-3, f"diffusion fp16 {name}: {rel:.3e}"


def test_diffusion_operator_eigenvector():
    """diag(s) K diag(s) applied through the scaled Gauss sum maps sqrt(d) to itself."""
    import pairwise_reductions_amd as pr
    _announce("diffusion_eigen")
    x, _, _ = _rand(7, 5000, 1, 3, 1)
    sig = 0.05
    s, q, d = pr.diffusion_scaling(_dev(x), sig, 0.5)
    v = d.sqrt().reshape(-1, 1).contiguous()
    out = _host(pr.gauss_sum_scaled(_dev(x), _dev(x), v, sig, row_scale=s, col_scale=s))
    want = _host(v)
    assert np.max(np.abs(out - want) / want) <= 3e-4


# ------------------------------------------------------------------ weighted argKmin
WARGK_SHAPES = [(1, 1, 3, 1), (257, 1000, 3, 10), (1025, 513, 1, 4), (700, 2000, 2, 16), (300, 5000, 8, 64),
                (2000, 70_001, 3, 1), (4097, 20_000, 3, 32), (350, 1999, 7, 4)]


def _grid(rng, shape, bits=24):
    return (rng.integers(0, 2 ** bits, size=shape) * 2.0 ** -bits).astype(np.float32)


@pytest.mark.parametrize("M,N,D,K", WARGK_SHAPES)
def test_argkmin_weighted_shapes(M, N, D, K):
    """Indices bit-exact, keys within 1e-6 relative (they are float64 keys rounded to float32)."""
    import pairwise_reductions_amd as pr
    _announce("argkmin_weighted", M=M, N=N, D=D, K=K)
    rng = np.random.default_rng(M * 3 + N)
    x, y = _grid(rng, (M, D)), _grid(rng, (N, D))
    w = (rng.integers(-2 ** 20, 2 ** 20, size=N) * 2.0 ** -24).astype(np.float32)   # |w| < 1/16
    idx, dist = pr.argkmin_weighted(_dev(x), _dev(y), _dev(w), K, with_dist=True)
    want_i, want_k = oracle.argkmin_weighted(x, y, w, K, workers=8)
    assert np.array_equal(_host(idx), want_i), "weighted argkmin indices"
    got_k = _host(dist).astype(np.float64)
    assert np.all(np.abs(got_k - want_k) <= 1e-6 * np.maximum(np.abs(want_k), 1e-30) + 1e-45)


def test_argkmin_weighted_ties_and_large_weights():
    """Planted equal keys (duplicate columns with equal weights, and distance differences the
    weights cancel) resolve to the lower index; weights far larger than the distances, of both
    signs, keep the ranking exact (the screening bound covers |w|)."""
    import pairwise_reductions_amd as pr
    _announce("argkmin_weighted_ties")
    rng = np.random.default_rng(55)
    M, N = 600, 3000
    x = _grid(rng, (M, 3), bits=8)
    y = _grid(rng, (N, 3), bits=8)
    w = (rng.integers(-4, 5, size=N) * 2.0 ** -8).astype(np.float32)
    y[100:200] = y[0:100]
    w[100:200] = w[0:100]
    idx = pr.argkmin_weighted(_dev(x), _dev(y), _dev(w), 8)
    want, _ = oracle.argkmin_weighted(x, y, w, 8, workers=8)
    assert np.array_equal(_host(idx), want)
    w2 = (rng.integers(-2 ** 20, 2 ** 20, size=N) * 2.0 ** -4).astype(np.float32)    # |w| up to 65536
    idx2 = pr.argkmin_weighted(_dev(x), _dev(y), _dev(w2), 5)
    want2, _ = oracle.argkmin_weighted(x, y, w2, 5, workers=8)
    assert np.array_equal(_host(idx2), want2)


# ------------------------------------------------- bf16 and float32 inputs, matrix-core path
TYPED_SHAPES = [
    # (B, M, N, D, C, sigma)
    (1, 1, 1, 32, 1, 1.0), (2, 300, 1000, 32, 32, 0.7), (1, 513, 2049, 64, 3, 1.0), (3, 129, 777, 128, 64, 1.5),
    (2, 400, 1500, 16, 17, 1.0), (1, 1000, 4096, 96, 8, 1.2),
]


def _typed_inputs(seed, B, M, N, D, C, dtype, shift=0.0):
    """Points ~ N(0, I/D) (+ shift) and weights ~ N(0, 1), rounded to `dtype`; returns the
    device tensors and their exact float64 values for the oracle."""
    import torch
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn((B, M, D), generator=g, dtype=torch.float64) / D ** 0.5 + shift).to(dtype)
    k = (torch.randn((B, N, D), generator=g, dtype=torch.float64) / D ** 0.5).to(dtype)
    v = torch.randn((B, N, C), generator=g, dtype=torch.float64).to(dtype)
    host = [t.to(torch.float64).numpy() for t in (q, k, v)]
    return (q.cuda(), k.cuda(), v.cuda()), host


@pytest.mark.parametrize("B,M,N,D,C,sigma", TYPED_SHAPES)
def test_gauss_sum_bf16_shapes(B, M, N, D, C, sigma):
    import torch
    import pairwise_reductions_amd as pr
    _announce("gauss_sum_bf16", B=B, M=M, N=N, D=D, C=C, sigma=sigma)
    (q, k, v), (qh, kh, vh) = _typed_inputs(B * 31 + M + D, B, M, N, D, C, torch.bfloat16)
    sig = float(np.float32(sigma))
    got = _host(pr.gauss_sum(q, k, v, sig))
    want, norm = oracle.gauss_sum_batched(qh, kh, vh, 1.0 / (sig * sig), workers=8)
    assert_normalised(got, want, norm, TOL_F16, "bf16")


@pytest.mark.parametrize("B,M,N,D,C,sigma", TYPED_SHAPES)
def test_gauss_sum_f32_matrix_core_shapes(B, M, N, D, C, sigma):
    """float32 inputs on the matrix cores (hi + lo fp16 parts, three products each) meet the
    float32 tolerance."""
    import torch
    import pairwise_reductions_amd as pr
    _announce("gauss_sum_f32_mfma", B=B, M=M, N=N, D=D, C=C, sigma=sigma)
    (q, k, v), (qh, kh, vh) = _typed_inputs(B * 37 + M + D, B, M, N, D, C, torch.float32)
    sig = float(np.float32(sigma))
    got = _host(pr.gauss_sum(q, k, v, sig))
    want, norm = oracle.gauss_sum_batched(qh, kh, vh, 1.0 / (sig * sig), workers=8)
    assert_normalised(got, want, norm, TOL_F32, "f32 matrix-core")


# Feature widths that are not a multiple of 16: the points are copied, zero-padded, into the
# workspace first; float32 with 9 <= D <= 15 takes the matrix-core path this way too.
ODD_WIDTHS = [
    # (dtype name, B, M, N, D, C, sigma)
    ("float32", 1, 700, 2000, 9, 1, 0.6), ("float32", 2, 513, 1500, 12, 3, 0.8), ("float32", 1, 300, 1000, 15, 2, 0.7),
    ("float32", 2, 400, 1200, 20, 4, 1.0), ("float32", 1, 257, 999, 50, 8, 1.2), ("float32", 1, 200, 777, 100, 1, 1.5),
    ("float16", 2, 700, 2000, 9, 1, 0.6), ("float16", 1, 513, 1500, 12, 32, 0.8), ("float16", 3, 400, 1200, 20, 4, 1.0),
    ("float16", 1, 257, 999, 50, 17, 1.2), ("float16", 2, 200, 777, 100, 64, 1.5), ("float16", 1, 300, 900, 3, 2, 0.3),
    ("bfloat16", 1, 700, 2000, 9, 1, 0.6), ("bfloat16", 2, 400, 1200, 20, 4, 1.0), ("bfloat16", 1, 257, 999, 100, 8, 1.5),
    # 32x32 forward tiles (D <= 32, 17 <= C <= 32): ragged rows and keys, several stages and splits
    ("float16", 3, 1025, 777, 32, 31, 0.9), ("bfloat16", 1, 513, 1500, 24, 20, 1.1), ("float16", 2, 100, 9000, 7, 24, 0.7),
]


@pytest.mark.parametrize("dname,B,M,N,D,C,sigma", ODD_WIDTHS)
def test_gauss_sum_any_feature_width(dname, B, M, N, D, C, sigma):
    import torch
    import pairwise_reductions_amd as pr
    _announce("gauss_sum_width", dtype=dname, B=B, M=M, N=N, D=D, C=C, sigma=sigma)
    dtype = getattr(torch, dname)
    (q, k, v), (qh, kh, vh) = _typed_inputs(B * 53 + M + D, B, M, N, D, C, dtype)
    sig = float(np.float32(sigma))
    got = _host(pr.gauss_sum(q, k, v, sig))
    want, norm = oracle.gauss_sum_batched(qh, kh, vh, 1.0 / (sig * sig), workers=8)
    assert_normalised(got, want, norm, TOL_F32 if dname == "float32" else TOL_F16, f"width {D} {dname}")


@pytest.mark.parametrize("B,M,N,D,C,sigma", [(1, 700, 2000, 20, 1, 1.0), (2, 300, 1000, 50, 3, 1.2),
                                             (1, 400, 900, 9, 17, 0.8), (2, 257, 600, 100, 2, 1.5)])
def test_gauss_sum_backward_fp16_any_feature_width(B, M, N, D, C, sigma):
    import pairwise_reductions_amd as pr
    _announce("backward_fp16_width", B=B, M=M, N=N, D=D, C=C, sigma=sigma)
    q, k, v = _highd_inputs(B * 9 + M * 5 + N + D, B, M, N, D, C)
    g = workloads.upstream_gradient(M, C, seed=M + D, B=B)
    sig = float(np.float32(sigma))
    got = pr.gauss_sum_backward(_dev(q), _dev(k), _dev(v), _dev(g), sig)
    want = _oracle_backward(q, k, v, g, sig)
    for key in ("x", "y", "b"):
        assert_normalised(_host(got[key]), want[key][0], want[key][1], TOL_F16, f"backward width {D} {key}")


def test_gauss_sum_f32_bf16_far_rows_and_scaled():
    """Rows far from every key (the running shift), and the scaled form, for both input types."""
    import torch
    import pairwise_reductions_amd as pr
    _announce("typed_far_scaled")
    for dtype, tol in ((torch.float32, TOL_F32), (torch.bfloat16, TOL_F16)):
        (q, k, v), (qh, kh, vh) = _typed_inputs(61, 2, 500, 2000, 32, 4, dtype, shift=1.0)
        got = _host(pr.gauss_sum(q, k, v, 1.0))
        want, norm = oracle.gauss_sum_batched(qh, kh, vh, 1.0, workers=8)
        assert_normalised(got, want, norm, tol, f"far {dtype}")
        rng = np.random.default_rng(62)
        r = rng.standard_normal((2, 500)).astype(np.float32)
        c = rng.standard_normal((2, 2000)).astype(np.float32)
        got = _host(pr.gauss_sum_scaled(q, k, v, 1.0, row_scale=_dev(r), col_scale=_dev(c)))
        for t in range(2):
            want, norm = oracle.gauss_sum_scaled(qh[t], kh[t], vh[t], 1.0, row_scale=r[t], col_scale=c[t], workers=8)
            assert_normalised(got[t], want, norm, tol, f"scaled {dtype}")


def test_diffusion_scaling_f32_matrix_core():
    import torch
    import pairwise_reductions_amd as pr
    _announce("diffusion_f32_mfma")
    (x, _, _), (xh, _, _) = _typed_inputs(63, 2, 1500, 1, 32, 1, torch.float32)
    s, q, d = (_host(t) for t in pr.diffusion_scaling(x, 1.0, 0.5))
    for t in range(2):
        ws, wq, wd = oracle.diffusion_scaling(xh[t], 1.0, 0.5, workers=8)
        for got, want, name in ((q[t], wq, "q"), (d[t], wd, "d"), (s[t], ws, "s")):
            rel = np.max(np.abs(got - want) / np.abs(want))
            assert rel <= 2e-4, f"diffusion f32 matrix-core {name}: {rel:.3e}"


# ------------------------------------------------------------------ edge cases of the extensions
def test_extension_edge_cases():
    """Empty sides, all-zero weights and scales, and sigma -> infinity for the backward, the
    scaled sum, the diffusion passes and the weighted argKmin."""
    import torch
    import pairwise_reductions_amd as pr
    _announce("extension_edges")
    # fp16 backward: N = 0 gives zero x-gradients; M = 0 gives zero y- and b-gradients
    q, k, v = _highd_inputs(71, 2, 100, 300, 32, 3)
    g = workloads.upstream_gradient(100, 3, seed=72, B=2)
    got = pr.gauss_sum_backward(_dev(q), _dev(k[:, :0].copy()), _dev(v[:, :0].copy()), _dev(g), 1.0, need=("x",))
    assert np.all(_host(got["x"]) == 0.0)
    got = pr.gauss_sum_backward(_dev(q[:, :0].copy()), _dev(k), _dev(v), _dev(g[:, :0].copy()), 1.0, need=("y", "b"))
    assert np.all(_host(got["y"]) == 0.0) and np.all(_host(got["b"]) == 0.0)
    # all-zero upstream gradient and all-zero weights: every gradient is exactly zero
    zg = np.zeros_like(g)
    got = pr.gauss_sum_backward(_dev(q), _dev(k), _dev(v), _dev(zg), 1.0)
    for key in ("x", "y", "b"):
        assert np.all(_host(got[key]) == 0.0), key
    got = pr.gauss_sum_backward(_dev(q), _dev(k), _dev(np.zeros_like(v)), _dev(g), 1.0, need=("x", "y"))
    assert np.all(_host(got["x"]) == 0.0) and np.all(_host(got["y"]) == 0.0)
    # float32 backward with M = 1 = N and x = y: the x-gradient is exactly zero
    x1 = np.array([[0.25, 0.5, 0.75]], np.float32)
    got = pr.gauss_sum_backward(_dev(x1), _dev(x1), _dev(np.ones((1, 1), np.float32)), _dev(np.ones((1, 1), np.float32)),
                                0.1, need=("x",))
    assert np.all(_host(got["x"]) == 0.0)
    # scaled sum: a zero column scale zeroes the output, a zero row scale too, on both paths
    x, y, b = _rand(73, 300, 900, 3, 2)
    out = _host(pr.gauss_sum_scaled(_dev(x), _dev(y), _dev(b), 0.1, col_scale=_dev(np.zeros(900, np.float32))))
    assert np.all(out == 0.0)
    out = _host(pr.gauss_sum_scaled(_dev(q), _dev(k), _dev(v), 1.0, row_scale=_dev(np.zeros((2, 100), np.float32))))
    assert np.all(out == 0.0)
    out = _host(pr.gauss_sum_scaled(_dev(q), _dev(k), _dev(v), 1.0, col_scale=_dev(np.zeros((2, 300), np.float32))))
    assert np.all(out == 0.0)
    # diffusion: sigma -> infinity gives s = 1/sqrt(N) for any alpha; one point gives s = 1
    xs, _, _ = _rand(74, 1000, 1, 3, 1)
    s, qd, dd = (_host(t) for t in pr.diffusion_scaling(_dev(xs), 1e30, 0.5))
    assert np.allclose(qd, 1000.0, rtol=1e-5) and np.allclose(s, 1.0 / np.sqrt(1000.0), rtol=1e-5)
    s1, _, _ = (_host(t) for t in pr.diffusion_scaling(_dev(xs[:1]), 0.1, 1.0))
    assert np.allclose(s1, 1.0, rtol=1e-6)
    # weighted argKmin with K = N returns a full ordering; M = 0 is a no-op
    xw, yw, _ = _rand(75, 50, 20, 2, 1)
    w = np.random.default_rng(76).standard_normal(20).astype(np.float32)
    idx = _host(pr.argkmin_weighted(_dev(xw), _dev(yw), _dev(w), 20))
    want, _ = oracle.argkmin_weighted(xw, yw, w, 20)
    assert np.array_equal(idx, want)
    pr.argkmin_weighted(_dev(xw[:0]), _dev(yw), _dev(w), 3)
    torch.cuda.synchronize()


def test_extension_determinism():
    """Two runs of each extension give bit-identical outputs."""
    import pairwise_reductions_amd as pr
    _announce("extension_determinism")
    q, k, v = _highd_inputs(81, 2, 700, 3000, 32, 2)
    g = workloads.upstream_gradient(700, 2, seed=82, B=2)
    a = pr.gauss_sum_backward(_dev(q), _dev(k), _dev(v), _dev(g), 1.0)
    b = pr.gauss_sum_backward(_dev(q), _dev(k), _dev(v), _dev(g), 1.0)
    for key in a:
        assert np.array_equal(_host(a[key]), _host(b[key])), key
    x, _, _ = _rand(83, 5000, 1, 3, 1)
    s1 = _host(pr.diffusion_scaling(_dev(x), 0.05, 0.5)[0])
    s2 = _host(pr.diffusion_scaling(_dev(x), 0.05, 0.5)[0])
    assert np.array_equal(s1, s2)
