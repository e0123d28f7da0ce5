"""Parity of the HIP path (through the C ABI) with the float64 oracle on seeded inputs.

Tolerances: Gauss sums and gradients within 1e-4 of the oracle relative to the row normaliser
sum_j |k_ij b_j| (resp. sum_j |k_ij (g_i.b_j)(x_i - y_j)| / sigma^2); log-sum-exp within 1e-4
absolute; argKmin indices bit-exact and distances within 1e-6 relative.
"""
import numpy as np
import pytest

import oracle
from pairwise_reductions_amd import workloads

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_LSE = 1e-4


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


def _announce(name, **kw):
    print(f"[case] {name} " + " ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def lse_bound(want):
    """1e-4 absolute, or one float32 ulp of |lse| where that is larger (|lse| >= 2048: there
    the correctly rounded float32 output alone may be 1.2e-4 or more away from the exact
    value)."""
    return np.maximum(TOL_LSE, np.spacing(np.abs(want).astype(np.float32)).astype(np.float64))


def assert_normalised(got, want, norm, tol, what=""):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - want)
    pos = norm > 0
    if np.any(pos):
        rel = err[pos] / norm[pos]
        worst = float(rel.max())
        assert worst <= tol, f"{what}: max normalised error {worst:.3e} > {tol:.1e}"
    assert np.all(np.abs(got[~pos]) <= np.finfo(np.float32).tiny), f"{what}: nonzero where the normaliser is 0"


def _rand(seed, M, N, D, C, lo=0.0, hi=1.0):
    rng = np.random.default_rng(seed)
    x = rng.uniform(lo, hi, (M, D)).astype(np.float32)
    y = rng.uniform(lo, hi, (N, D)).astype(np.float32)
    b = rng.standard_normal((N, C)).astype(np.float32)
    return x, y, b


GAUSS_SHAPES = [
    # (M, N, D, C, sigma): single tile, ragged row/column tails, every D and several C, the
    # column-split path (small M, large N) and the unsplit path (large M)
    (1, 1, 3, 1, 0.1), (1, 37, 3, 1, 0.3), (257, 1000, 3, 1, 0.1), (1025, 513, 1, 1, 0.05),
    (700, 2000, 2, 3, 0.2), (513, 1500, 8, 8, 0.5), (2000, 300, 5, 4, 0.3), (300, 4099, 4, 2, 0.07),
    (100, 100_003, 3, 2, 0.02), (50_001, 777, 3, 1, 0.1), (1500, 1500, 6, 5, 0.4), (999, 2500, 7, 7, 0.6),
    # 32x32 tiles with 2-4 channels (one 32-row tile per wave), ragged tails and column splits
    (4000, 5001, 3, 4, 0.05), (33, 40_000, 1, 3, 0.1), (1999, 3333, 2, 2, 0.08),
]


@pytest.mark.parametrize("M,N,D,C,sigma", GAUSS_SHAPES)
def test_gauss_sum_shapes(M, N, D, C, sigma):
    import pairwise_reductions_amd as pr
    _announce("gauss_sum", M=M, N=N, D=D, C=C, sigma=sigma)
    x, y, b = _rand(M * 7 + N, M, N, D, C)
    sig = float(np.float32(sigma))
    got = _host(pr.gauss_sum(_dev(x), _dev(y), _dev(b), sig))
    want, norm = oracle.gauss_sum(x, y, b, sig, workers=8)
    assert_normalised(got, want, norm, TOL_F32, "gauss_sum")


# The float32 low-D sum computes its exponent on the matrix cores when the exponent scale
# 2 c2 h^2 (h: half-width of the points' bounding box, c2 = log2(e) / (2 sigma^2)) is small
# enough for the low part of the split exponent to stay below 32 (2 c2 h^2 <= 2^13 at D = 3,
# <= 2^10 at D = 8), and falls back to the float64 sweep otherwise. These cases sit on both
# sides of that line, plus spreads that move h: an offset cube, a symmetric box, an outlier.
EXPONENT_REGIMES = [
    # (D, sigma, lo, hi, outlier)
    (3, 0.3, 0.0, 1.0, False), (3, 0.01, 0.0, 1.0, False), (3, 0.0067, 0.0, 1.0, False),
    (3, 0.006, 0.0, 1.0, False), (3, 0.001, 0.0, 1.0, False), (3, 0.05, 1000.0, 1001.0, False),
    (3, 0.5, -5.0, 5.0, False), (3, 0.05, 0.0, 1.0, True), (1, 0.004, 0.0, 1.0, False),
    (8, 0.5, 0.0, 1.0, False), (8, 0.03, 0.0, 1.0, False), (8, 0.015, 0.0, 1.0, False),
    (6, 0.2, -1.0, 1.0, False), (7, 0.3, 0.0, 1.0, False),
]


@pytest.mark.parametrize("D,sigma,lo,hi,outlier", EXPONENT_REGIMES)
def test_gauss_sum_exponent_regimes(D, sigma, lo, hi, outlier):
    import pairwise_reductions_amd as pr
    _announce("gauss_sum_regime", D=D, sigma=sigma, lo=lo, hi=hi, outlier=outlier)
    M, N, C = 700, 3001, 2
    x, y, b = _rand(int(sigma * 1e4) + 31 * D, M, N, D, C, lo, hi)
    # every row gets a column within about sigma, so no row's sum underflows float32
    rng = np.random.default_rng(D)
    y[:M] = x + (0.5 * sigma * rng.standard_normal((M, D))).astype(np.float32)
    if outlier:
        y[M + 17] = 1000.0
    sig = float(np.float32(sigma))
    got = _host(pr.gauss_sum(_dev(x), _dev(y), _dev(b), sig))
    want, norm = oracle.gauss_sum(x, y, b, sig, workers=8)
    assert_normalised(got, want, norm, TOL_F32, "gauss_sum regime")


# Points set aside: when the points' bounding box is too wide for the matrix cores but a box of
# the largest admissible half-width around their mean holds all but at most 256 rows and 256
# columns, those are summed separately (set-aside columns added to every row in index order,
# set-aside rows over all columns) and the rest stays on the matrix cores. More than 256 on
# either side sends the call to the float64 sweep. Every case must match the oracle.
SET_ASIDE_CASES = [
    # (name, D, C, sigma, rows set aside, columns set aside, scaled)
    ("one far column", 3, 1, 0.05, [], [17], False),
    ("one far row", 3, 1, 0.05, [5], [], False),
    ("far row next to far column", 3, 2, 0.05, [17], [17], False),
    ("scattered rows and columns", 3, 3, 0.02, [0, 3, 99, 698, 699], [1, 2, 700, 3000], False),
    ("scaled, D = 5", 5, 2, 0.1, [9, 10], [11, 2999], True),
    ("256 rows and 256 columns", 3, 1, 0.05, list(range(0, 700, 3))[:256], list(range(1, 3001, 11))[:256], False),
    ("more than 256 columns", 3, 1, 0.05, [], list(range(0, 3001, 9))[:300], False),
    ("D = 1", 1, 1, 0.004, [1], [2], False),
]


@pytest.mark.parametrize("name,D,C,sigma,rows,cols,scaled", SET_ASIDE_CASES, ids=[c[0] for c in SET_ASIDE_CASES])
def test_gauss_sum_set_aside_points(name, D, C, sigma, rows, cols, scaled):
    import pairwise_reductions_amd as pr
    _announce("gauss_sum_set_aside", case=name, D=D, C=C, sigma=sigma)
    M, N = 700, 3001
    x, y, b = _rand(len(rows) * 7 + len(cols) + D, M, N, D, C)
    rng = np.random.default_rng(D + len(cols))
    y[:M] = x + (0.5 * sigma * rng.standard_normal((M, D))).astype(np.float32)
    far = (1000.0 + 3.0 * np.arange(max(len(rows), len(cols)))).astype(np.float32)
    for k, i in enumerate(rows):
        x[i] = far[k] + 0.25 * sigma * k / max(len(rows), 1)
    for k, j in enumerate(cols):
        y[j] = far[k]
    sig = float(np.float32(sigma))
    if scaled:
        r = rng.uniform(0.5, 2.0, M).astype(np.float32)
        c = rng.uniform(-1.0, 1.0, N).astype(np.float32)
        got = _host(pr.gauss_sum_scaled(_dev(x), _dev(y), _dev(b), sig, row_scale=_dev(r), col_scale=_dev(c)))
        want, norm = oracle.gauss_sum_scaled(x, y, b, sig, row_scale=r, col_scale=c, workers=8)
    else:
        got = _host(pr.gauss_sum(_dev(x), _dev(y), _dev(b), sig))
        want, norm = oracle.gauss_sum(x, y, b, sig, workers=8)
    assert_normalised(got, want, norm, TOL_F32, f"set aside: {name}")
    if not scaled:
        again = _host(pr.gauss_sum(_dev(x), _dev(y), _dev(b), sig))
        assert np.array_equal(got, again), "set-aside results must be reproducible"


@pytest.mark.parametrize("D,sigma,lo,hi,outlier", EXPONENT_REGIMES)
def test_lse_exponent_regimes(D, sigma, lo, hi, outlier):
    import pairwise_reductions_amd as pr
    _announce("lse_regime", D=D, sigma=sigma, lo=lo, hi=hi, outlier=outlier)
    M, N = 700, 3001
    x, y, _ = _rand(int(sigma * 1e4) + 37 * D, M, N, D, 1, lo, hi)
    rng = np.random.default_rng(D + 1)
    y[:M] = x + (0.5 * sigma * rng.standard_normal((M, D))).astype(np.float32)
    if outlier:
        y[M + 17] = 1000.0
    sig = float(np.float32(sigma))
    got = _host(pr.lse(_dev(x), _dev(y), sig)).astype(np.float64)
    want = oracle.logsumexp_reduction(x, y, sig, workers=8)
    err = np.abs(got - want)
    assert np.all(err <= lse_bound(want)), f"lse regime: max error {err.max():.3e}"


def test_gauss_sum_workload_10k_all_rows():
    import pairwise_reductions_amd as pr
    inp = workloads.make_inputs("gauss_sum_10k")
    _announce("gauss_sum_10k", M=inp["M"], N=inp["N"])
    sig = float(inp["sigma"])
    got = _host(pr.gauss_sum(_dev(inp["x"]), _dev(inp["y"]), _dev(inp["b"]), sig))
    want, norm = oracle.gauss_sum(inp["x"], inp["y"], inp["b"], sig, workers=8)
    assert_normalised(got, want, norm, TOL_F32, "gauss_sum_10k")


def test_gauss_sum_edge_cases():
    import torch
    import pairwise_reductions_amd as pr
    _announce("gauss_sum_edges")
    x, y, b = _rand(3, 64, 10, 3, 2)
    # N = 0 writes zeros
    out = pr.gauss_sum(_dev(x), _dev(y[:0]), _dev(b[:0]), 0.1)
    assert np.all(_host(out) == 0.0)
    # M = 0 is a no-op (the output keeps its contents)
    sentinel = torch.full((0, 2), 7.0, device="cuda")
    pr.gauss_sum(_dev(x[:0]), _dev(y), _dev(b), 0.1, out=sentinel)
    # x_i = y_j with every other column far away: the result is b_j (the far terms underflow to
    # exactly 0; the coincident term is exp of an exponent computed to about 1e-6, well inside
    # the 1e-4 bar)
    y2 = np.array([[0, 0, 0], [50, 0, 0], [0, 60, 0]], np.float32)
    b2 = np.array([[0.75], [2.0], [-4.0]], np.float32)
    got = _host(pr.gauss_sum(_dev(y2[[1, 0, 2]]), _dev(y2), _dev(b2), 0.5))
    assert np.allclose(got[:, 0], [2.0, 0.75, -4.0], rtol=1e-5, atol=0)
    # sigma -> infinity: s_i = sum_j b_j
    x3, y3, b3 = _rand(5, 300, 700, 3, 1)
    got = _host(pr.gauss_sum(_dev(x3), _dev(y3), _dev(b3), 1e30))
    assert np.allclose(got[:, 0], b3.astype(np.float64).sum(), rtol=0, atol=1e-4 * np.abs(b3).sum())


def test_gauss_sum_deterministic():
    import pairwise_reductions_amd as pr
    _announce("gauss_sum_determinism")
    x, y, b = _rand(11, 3000, 20_000, 3, 1)
    xd, yd, bd = _dev(x), _dev(y), _dev(b)
    a = _host(pr.gauss_sum(xd, yd, bd, 0.05))
    for _ in range(3):
        assert np.array_equal(a, _host(pr.gauss_sum(xd, yd, bd, 0.05)))


LSE_SHAPES = [(1, 1, 3, 0.1), (257, 1000, 3, 0.1), (1025, 513, 1, 0.05), (700, 2000, 2, 0.2),
              (513, 1500, 8, 0.5), (100, 100_003, 3, 0.02), (50_001, 777, 3, 0.1), (333, 7, 3, 0.01)]


@pytest.mark.parametrize("M,N,D,sigma", LSE_SHAPES)
def test_lse_shapes(M, N, D, sigma):
    import pairwise_reductions_amd as pr
    _announce("lse", M=M, N=N, D=D, sigma=sigma)
    x, y, _ = _rand(M * 3 + N, M, N, D, 1)
    sig = float(np.float32(sigma))
    got = _host(pr.lse(_dev(x), _dev(y), sig))
    want = oracle.logsumexp_reduction(x, y, sig, workers=8)
    assert np.all(np.abs(got - want) <= lse_bound(want))


def test_lse_far_rows_and_empty():
    import pairwise_reductions_amd as pr
    _announce("lse_far_and_empty")
    rng = np.random.default_rng(21)
    y = rng.random((5000, 3)).astype(np.float32)
    # rows far from every column: a plain sum of exponentials underflows, the reduction not
    x = (rng.random((300, 3)) + np.array([3.0, 0.0, 0.0])).astype(np.float32)
    got = _host(pr.lse(_dev(x), _dev(y), 0.05))
    want = oracle.logsumexp_reduction(x, y, float(np.float32(0.05)))
    assert np.all(np.isfinite(got))
    assert np.all(np.abs(got - want) <= lse_bound(want))
    got = _host(pr.lse(_dev(x), _dev(y[:0]), 0.1))
    assert np.all(np.isneginf(got))


def test_lse_some_far_rows_among_near_ones():
    """Rows far from every column scattered among ordinary rows, over several column splits: the
    far ones (log-sum-exp below 64 ln 2) are recomputed after the matrix-core sweep, the others
    keep its result."""
    import pairwise_reductions_amd as pr
    _announce("lse_mixed_far")
    rng = np.random.default_rng(23)
    y = rng.random((40_000, 3)).astype(np.float32)
    x = rng.random((3000, 3)).astype(np.float32)
    x[::7] += np.float32(2.5)          # every seventh row far outside the columns' cube
    x[5::97] = np.float32(1.3)         # a few just outside it (sums near 2^-64)
    for sigma in (0.05, 0.1):
        sig = float(np.float32(sigma))
        got = _host(pr.lse(_dev(x), _dev(y), sig)).astype(np.float64)
        want = oracle.logsumexp_reduction(x, y, sig, workers=8)
        err = np.abs(got - want)
        assert np.all(err <= lse_bound(want)), f"sigma {sigma}: max error {err.max():.3e}"
        idx, flse = pr.argkmin_lse(_dev(x), _dev(y), 4, sig)
        err = np.abs(_host(flse).astype(np.float64) - want)
        assert np.all(err <= lse_bound(want)), f"argkmin_lse sigma {sigma}: max error {err.max():.3e}"


ARGK_SHAPES = [(1, 1, 3, 1), (257, 1000, 3, 10), (1025, 513, 1, 4), (700, 2000, 2, 16),
               (513, 1500, 8, 32), (100, 100_003, 3, 10), (50_001, 777, 3, 10), (300, 64, 3, 64),
               (200, 5000, 3, 64), (333, 20, 5, 20), (1000, 3000, 3, 3),
               # two rows per lane with two-column tiles (D > 4), odd column counts
               (513, 1501, 8, 10), (401, 2999, 5, 8), (129, 4097, 6, 2)]


@pytest.mark.parametrize("M,N,D,K", ARGK_SHAPES)
def test_argkmin_shapes(M, N, D, K):
    import pairwise_reductions_amd as pr
    _announce("argkmin", M=M, N=N, D=D, K=K)
    rng = np.random.default_rng(M + N + K)
    x = workloads.grid24(rng, (M, D))
    y = workloads.grid24(rng, (N, D))
    idx, dist = pr.argkmin(_dev(x), _dev(y), K, with_dist=True)
    idx, dist = _host(idx), _host(dist)
    want_idx, want_d2 = oracle.argkmin(x, y, K, workers=8)
    assert np.array_equal(idx.astype(np.int64), want_idx)
    assert np.allclose(dist, want_d2, rtol=1e-6, atol=0)


# From 16384 rows on, the argKmin sweeps take their rows in spatial order (a counting sort by
# grid cell); every row's result must still be the oracle's, bit for bit.
ORDERED_ARGK_SHAPES = [(16384, 2000, 3, 10), (20000, 3001, 1, 4), (20001, 2500, 2, 1), (17000, 4000, 5, 16),
                       (30000, 1500, 8, 32), (16500, 999, 3, 64)]


@pytest.mark.parametrize("M,N,D,K", ORDERED_ARGK_SHAPES)
def test_argkmin_spatially_ordered_rows(M, N, D, K):
    import pairwise_reductions_amd as pr
    _announce("argkmin_ordered", M=M, N=N, D=D, K=K)
    rng = np.random.default_rng(M + 3 * N + K)
    x = workloads.grid24(rng, (M, D))
    y = workloads.grid24(rng, (N, D))
    x[::7] = (x[::7] * 0.01).astype(np.float32)   # a dense corner: many rows in few cells
    idx, dist = pr.argkmin(_dev(x), _dev(y), K, with_dist=True)
    want_idx, want_d2 = oracle.argkmin(x, y, K, workers=8)
    assert np.array_equal(_host(idx).astype(np.int64), want_idx)
    assert np.allclose(_host(dist), want_d2, rtol=1e-6, atol=0)
    w = rng.uniform(-0.01, 0.01, N).astype(np.float32)
    widx, wkeys = pr.argkmin_weighted(_dev(x), _dev(y), _dev(w), K, with_dist=True)
    want_widx, _ = oracle.argkmin_weighted(x, y, w, K, workers=8)
    assert np.array_equal(_host(widx).astype(np.int64), want_widx)
    if D <= 3:
        sig = float(np.float32(0.1))
        fidx, flse = pr.argkmin_lse(_dev(x), _dev(y), K, sig)
        assert np.array_equal(_host(fidx).astype(np.int64), want_idx)
        want_lse = oracle.logsumexp_reduction(x, y, sig, workers=8)
        assert np.all(np.abs(_host(flse) - want_lse) <= lse_bound(want_lse))


def test_argkmin_spatially_ordered_rows_ties():
    """Many rows (spatial order and starting thresholds) on a coarse grid with planted duplicate
    columns: equal keys still resolve to the lower column index, with and without weights."""
    import pairwise_reductions_amd as pr
    _announce("argkmin_ordered_ties")
    rng = np.random.default_rng(17)
    M, N = 20_000, 3000
    x = (rng.integers(0, 8, size=(M, 3)) / 8.0).astype(np.float32)
    y = (rng.integers(0, 8, size=(N, 3)) / 8.0).astype(np.float32)
    y[100:200] = y[0]
    w = (rng.integers(-2, 3, size=N) / 64.0).astype(np.float32)
    w[100:200] = w[0]
    for K in (1, 10, 33, 64):
        idx = _host(pr.argkmin(_dev(x), _dev(y), K)).astype(np.int64)
        want, _ = oracle.argkmin(x, y, K, workers=8)
        assert np.array_equal(idx, want), K
        widx = _host(pr.argkmin_weighted(_dev(x), _dev(y), _dev(w), K)).astype(np.int64)
        wwant, _ = oracle.argkmin_weighted(x, y, w, K, workers=8)
        assert np.array_equal(widx, wwant), K


def test_argkmin_ties_lowest_index():
    import pairwise_reductions_amd as pr
    _announce("argkmin_ties")
    rng = np.random.default_rng(5)
    # a coarse grid makes many exactly equal distances; duplicates are planted on purpose
    x = (rng.integers(0, 8, size=(2000, 3)) / 8.0).astype(np.float32)
    y = (rng.integers(0, 8, size=(3000, 3)) / 8.0).astype(np.float32)
    y[100:200] = y[0]
    for K in (1, 5, 10, 33):
        idx = _host(pr.argkmin(_dev(x), _dev(y), K)).astype(np.int64)
        want, _ = oracle.argkmin(x, y, K, workers=8)
        assert np.array_equal(idx, want), K


GRAD_SHAPES = [(1, 1, 3, 1, 0.1), (257, 1000, 3, 1, 0.1), (1025, 513, 1, 1, 0.05), (700, 2000, 2, 3, 0.2),
               (513, 1500, 8, 8, 0.5), (100, 100_003, 3, 2, 0.05), (20_001, 777, 3, 1, 0.1)]


@pytest.mark.parametrize("M,N,D,C,sigma", GRAD_SHAPES)
def test_grad_x_shapes(M, N, D, C, sigma):
    import pairwise_reductions_amd as pr
    _announce("grad_x", M=M, N=N, D=D, C=C, sigma=sigma)
    x, y, b = _rand(M * 5 + N, M, N, D, C)
    g = np.random.default_rng(M).standard_normal((M, C)).astype(np.float32)
    sig = float(np.float32(sigma))
    got = _host(pr.gauss_sum_grad_x(_dev(x), _dev(y), _dev(b), _dev(g), sig))
    want, norm = oracle.gauss_sum_grad_x(x, y, b, g, sig, workers=8)
    assert_normalised(got, want, norm, TOL_F32, "grad_x")


@pytest.mark.parametrize("D,sigma,lo,hi,outlier", EXPONENT_REGIMES)
def test_grad_xy_exponent_regimes(D, sigma, lo, hi, outlier):
    """One-channel gradients on both sides of the matrix-core / float32 decision. Every x has a
    y within about sigma and every y an x (both gradients then have rows whose kernel values
    stay in float32 range; a row with none underflows to 0 by reading 10)."""
    import pairwise_reductions_amd as pr
    _announce("grad_regime", D=D, sigma=sigma, lo=lo, hi=hi, outlier=outlier)
    M = N = 1501
    x, y, b = _rand(int(sigma * 1e4) + 41 * D, M, N, D, 1, lo, hi)
    rng = np.random.default_rng(D + 2)
    y[:] = x[rng.permutation(M)] + (0.5 * sigma * rng.standard_normal((N, D))).astype(np.float32)
    if outlier:
        y[17] = 1000.0
        x[17] = 1000.02
    g = rng.standard_normal((M, 1)).astype(np.float32)
    sig = float(np.float32(sigma))
    got = _host(pr.gauss_sum_grad_x(_dev(x), _dev(y), _dev(b), _dev(g), sig))
    want, norm = oracle.gauss_sum_grad_x(x, y, b, g, sig, workers=8)
    assert_normalised(got, want, norm, TOL_F32, "grad_x regime")
    got = _host(pr.gauss_sum_grad_y(_dev(x), _dev(y), _dev(b), _dev(g), sig))
    want, norm = oracle.gauss_sum_grad_y(x, y, b, g, sig, workers=8)
    assert_normalised(got, want, norm, TOL_F32, "grad_y regime")


@pytest.mark.parametrize("extreme", [False, True])
def test_grad_xy_weight_signs_zeros_and_range(extreme):
    """One-channel gradients with weights of both signs, exact zeros and magnitudes over 2^+-20.
    The matrix-core sweep carries log2 |b_j| in the exponent and the sign of b_j in the column
    record; with one weight of 1e-12 (|log2| near 40, beyond what the exponent pieces carry)
    the call takes the float32 sweep instead. Both must match the oracle, for the x-gradient
    (weights b) and the y-gradient (the roles exchanged: the upstream g weighs the columns)."""
    import pairwise_reductions_amd as pr
    _announce("grad_weight_range", extreme=extreme)
    M, N, D, sig = 1200, 1700, 3, float(np.float32(0.1))
    x, y, _ = _rand(9101, M, N, D, 1)
    rng = np.random.default_rng(9102)
    b = (rng.standard_normal((N, 1)) * np.exp2(rng.integers(-20, 21, (N, 1)))).astype(np.float32)
    b[::7] = 0.0
    g = (rng.standard_normal((M, 1)) * np.exp2(rng.integers(-20, 21, (M, 1)))).astype(np.float32)
    g[::5] = 0.0
    if extreme:
        b[5] = 1e-12
        g[3] = -1e-12
    got = _host(pr.gauss_sum_grad_x(_dev(x), _dev(y), _dev(b), _dev(g), sig))
    want, norm = oracle.gauss_sum_grad_x(x, y, b, g, sig, workers=8)
    assert_normalised(got, want, norm, TOL_F32, "grad_x weights")
    got = _host(pr.gauss_sum_grad_y(_dev(x), _dev(y), _dev(b), _dev(g), sig))
    want, norm = oracle.gauss_sum_grad_y(x, y, b, g, sig, workers=8)
    assert_normalised(got, want, norm, TOL_F32, "grad_y weights")


def test_grad_x_of_squared_loss_mixture():
    """The KeOps example's loss sum_i a_i^2 on the 8-cluster mixture: the upstream gradient
    is g = 2 s with s the oracle's forward, rounded to float32 for both sides."""
    import pairwise_reductions_amd as pr
    inp = workloads.make_inputs("gauss_sum_grad_x_100k_mixture", M=4000, N=6000)
    _announce("grad_x_loss_mixture", M=4000, N=6000)
    sig = float(inp["sigma"])
    s, _ = oracle.gauss_sum(inp["x"], inp["y"], inp["b"], sig, workers=8)
    g = (2.0 * s).astype(np.float32)
    got = _host(pr.gauss_sum_grad_x(_dev(inp["x"]), _dev(inp["y"]), _dev(inp["b"]), _dev(g), sig))
    want, norm = oracle.gauss_sum_grad_x(inp["x"], inp["y"], inp["b"], g, sig, workers=8)
    assert_normalised(got, want, norm, TOL_F32, "grad_x loss")


# ------------------------------------------------------------------ fp16 matrix-core path
TOL_F16 = 2e-3

HIGHD_SHAPES = [
    # (B, M, N, D, C, sigma)
    (1, 1, 1, 32, 32, 1.0), (1, 100, 77, 32, 32, 1.0), (2, 300, 1000, 32, 32, 0.7),
    (4, 513, 2049, 32, 32, 1.0), (1, 1024, 4096, 64, 32, 1.5), (1, 257, 300, 32, 64, 1.0),
    (2, 700, 5000, 64, 64, 2.0), (3, 4097, 8191, 32, 32, 1.0),
    # channel counts that are not multiples of 16 (padded inside the library), as in the flash
    # page's C = 1 figures
    (4, 1000, 3000, 32, 1, 1.0), (2, 513, 2000, 32, 3, 0.8), (1, 300, 1000, 64, 17, 1.0), (2, 200, 700, 32, 48, 1.0),
]


def _highd_inputs(seed, B, M, N, D, C, shift=0.0):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((B, M, D)) / np.sqrt(D) + shift).astype(np.float16)
    k = (rng.standard_normal((B, N, D)) / np.sqrt(D)).astype(np.float16)
    v = rng.standard_normal((B, N, C)).astype(np.float16)
    return q, k, v


def _check_highd(q, k, v, sigma):
    import pairwise_reductions_amd as pr
    sig = float(np.float32(sigma))
    got = _host(pr.gauss_sum(_dev(q), _dev(k), _dev(v), sig))
    tau = 1.0 / (sig * sig)
    want, norm = oracle.gauss_sum_batched(q, k, v, tau, workers=8)
    assert_normalised(got, want, norm, TOL_F16, "gauss_sum fp16")


@pytest.mark.parametrize("B,M,N,D,C,sigma", HIGHD_SHAPES)
def test_gauss_sum_fp16_shapes(B, M, N, D, C, sigma):
    _announce("gauss_sum_fp16", B=B, M=M, N=N, D=D, C=C, sigma=sigma)
    q, k, v = _highd_inputs(B * 13 + M + N, B, M, N, D, C)
    _check_highd(q, k, v, sigma)


def test_gauss_sum_fp16_far_rows_and_rescale():
    """Rows far from every key (all kernel values below the fp16 normal range without the
    running shift), and keys ordered far-to-near so the shift must rise mid-sweep."""
    _announce("gauss_sum_fp16_far")
    q, k, v = _highd_inputs(77, 2, 600, 3000, 32, 32, shift=1.0)
    _check_highd(q, k, v, 1.0)
    rng = np.random.default_rng(78)
    qn = (rng.standard_normal((1, 300, 32)) / np.sqrt(32)).astype(np.float16)
    kn = (rng.standard_normal((1, 4000, 32)) / np.sqrt(32)).astype(np.float16)
    d2 = ((qn[0, :1].astype(np.float64) - kn[0].astype(np.float64)) ** 2).sum(axis=1)
    kn = kn[:, np.argsort(-d2)]          # farthest keys first for row 0
    vn = rng.standard_normal((1, 4000, 32)).astype(np.float16)
    _check_highd(qn, kn, vn, 0.25)


def test_all_ops_deterministic():
    import pairwise_reductions_amd as pr
    _announce("determinism")
    rng = np.random.default_rng(9)
    x = workloads.grid24(rng, (5000, 3))
    y = workloads.grid24(rng, (70000, 3))
    b = rng.standard_normal((70000, 2)).astype(np.float32)
    g = rng.standard_normal((5000, 2)).astype(np.float32)
    xd, yd, bd, gd = _dev(x), _dev(y), _dev(b), _dev(g)
    runs = [(_host(pr.lse(xd, yd, 0.05)), _host(pr.argkmin(xd, yd, 7)),
             _host(pr.gauss_sum_grad_x(xd, yd, bd, gd, 0.05))) for _ in range(2)]
    for a, c in zip(runs[0], runs[1]):
        assert np.array_equal(a, c)
    q, k, v = _highd_inputs(10, 2, 1000, 3000, 32, 32)
    qd, kd, vd = _dev(q), _dev(k), _dev(v)
    assert np.array_equal(_host(pr.gauss_sum(qd, kd, vd, 1.0)), _host(pr.gauss_sum(qd, kd, vd, 1.0)))


# ------------------------------------------------ gradients with respect to y and b
GRADYB_SHAPES = [(1, 1, 3, 1, 0.1), (1000, 257, 3, 1, 0.1), (513, 1025, 1, 2, 0.05), (2000, 700, 2, 3, 0.2),
                 (1500, 513, 8, 8, 0.5), (100_003, 100, 3, 2, 0.05), (777, 20_001, 3, 1, 0.1)]


@pytest.mark.parametrize("M,N,D,C,sigma", GRADYB_SHAPES)
def test_grad_y_and_b_shapes(M, N, D, C, sigma):
    import pairwise_reductions_amd as pr
    _announce("grad_y_b", M=M, N=N, D=D, C=C, sigma=sigma)
    x, y, b = _rand(M * 11 + N, M, N, D, C)
    g = np.random.default_rng(N).standard_normal((M, C)).astype(np.float32)
    sig = float(np.float32(sigma))
    xd, yd, bd, gd = _dev(x), _dev(y), _dev(b), _dev(g)
    gy = _host(pr.gauss_sum_grad_y(xd, yd, bd, gd, sig))
    gb = _host(pr.gauss_sum_grad_b(xd, yd, gd, sig))
    want_y, norm_y = oracle.gauss_sum_grad_y(x, y, b, g, sig, workers=8)
    want_b, norm_b = oracle.gauss_sum_grad_b(x, y, g, sig, workers=8)
    assert_normalised(gy, want_y, norm_y, TOL_F32, "grad_y")
    assert_normalised(gb, want_b, norm_b, TOL_F32, "grad_b")


def test_autograd_function_all_gradients():
    """loss = sum_i s_i . w_i through the autograd wrapper: forward and the three gradients
    against the oracle with the upstream gradient g = w."""
    import torch
    import pairwise_reductions_amd as pr
    _announce("autograd")
    inp = workloads.make_inputs("gauss_sum_grad_x_100k_mixture", M=3000, N=5000)
    sig = float(inp["sigma"])
    w = workloads.upstream_gradient(3000, 1, seed=5)
    x = _dev(inp["x"]).requires_grad_(True)
    y = _dev(inp["y"]).requires_grad_(True)
    b = _dev(inp["b"]).requires_grad_(True)
    s = pr.gauss_sum_autograd(x, y, b, sig)
    (s * _dev(w)).sum().backward()
    torch.cuda.synchronize()
    want_s, norm_s = oracle.gauss_sum(inp["x"], inp["y"], inp["b"], sig, workers=8)
    assert_normalised(s.detach().cpu().numpy(), want_s, norm_s, TOL_F32, "autograd forward")
    gx, nx = oracle.gauss_sum_grad_x(inp["x"], inp["y"], inp["b"], w, sig, workers=8)
    gy, ny = oracle.gauss_sum_grad_y(inp["x"], inp["y"], inp["b"], w, sig, workers=8)
    gb, nb = oracle.gauss_sum_grad_b(inp["x"], inp["y"], w, sig, workers=8)
    assert_normalised(x.grad.cpu().numpy(), gx, nx, TOL_F32, "autograd x")
    assert_normalised(y.grad.cpu().numpy(), gy, ny, TOL_F32, "autograd y")
    assert_normalised(b.grad.cpu().numpy(), gb, nb, TOL_F32, "autograd b")


# --------------------------------------------------- fused argKmin + log-sum-exp
@pytest.mark.parametrize("M,N,D,K", ARGK_SHAPES)
def test_argkmin_lse_shapes(M, N, D, K):
    import pairwise_reductions_amd as pr
    _announce("argkmin_lse", M=M, N=N, D=D, K=K)
    rng = np.random.default_rng(M + 2 * N + K)
    x = workloads.grid24(rng, (M, D))
    y = workloads.grid24(rng, (N, D))
    sig = float(np.float32(0.1))
    idx, dist, lse = pr.argkmin_lse(_dev(x), _dev(y), K, sig, with_dist=True)
    idx, dist, lse = _host(idx), _host(dist), _host(lse)
    want_idx, want_d2 = oracle.argkmin(x, y, K, workers=8)
    assert np.array_equal(idx.astype(np.int64), want_idx)
    assert np.allclose(dist, want_d2, rtol=1e-6, atol=0)
    want_lse = oracle.logsumexp_reduction(x, y, sig, workers=8)
    assert np.all(np.abs(lse - want_lse) <= lse_bound(want_lse))


@pytest.mark.parametrize("D,sigma,lo,hi,outlier", EXPONENT_REGIMES)
def test_argkmin_lse_exponent_regimes(D, sigma, lo, hi, outlier):
    """argKmin + LSE on both sides of the matrix-core decision: the matrix-core log-sum-exp
    beside the plain argKmin sweep where the decision admits the inputs, the fused float64
    sweep where it declines."""
    import pairwise_reductions_amd as pr
    _announce("argkmin_lse_regime", D=D, sigma=sigma, lo=lo, hi=hi, outlier=outlier)
    M, N, K = 700, 3001, 10
    x, y, _ = _rand(int(sigma * 1e4) + 43 * D, M, N, D, 1, lo, hi)
    rng = np.random.default_rng(D + 3)
    y[:M] = x + (0.5 * sigma * rng.standard_normal((M, D))).astype(np.float32)
    if outlier:
        y[M + 17] = 1000.0
    sig = float(np.float32(sigma))
    idx, dist, lse = pr.argkmin_lse(_dev(x), _dev(y), K, sig, with_dist=True)
    idx, dist, lse = _host(idx), _host(dist), _host(lse).astype(np.float64)
    want_idx, want_d2 = oracle.argkmin(x, y, K, workers=8)
    assert np.array_equal(idx.astype(np.int64), want_idx)
    assert np.allclose(dist, want_d2, rtol=1e-6, atol=0)
    want_lse = oracle.logsumexp_reduction(x, y, sig, workers=8)
    err = np.abs(lse - want_lse)
    assert np.all(err <= lse_bound(want_lse)), f"argkmin_lse regime: max LSE error {err.max():.3e}"


# From 16384 rows on, argKmin without weights at D <= 3, K <= 16 screens on the matrix cores in
# the frame of the points' bounding box (fp16 pieces, a proven margin, exact float64 keys for
# the kept columns). Frames that stress it: a narrow box far from the origin, one far outlier
# that makes the box huge (so the margin admits nearly every column), plain float32 values,
# coarse grids with many equal keys, every D and K bucket it takes.
SCREEN_CASES = [
    # (name, M, N, D, K)
    ("far narrow box, coarse grid", 20_000, 3000, 3, 10),
    ("one far outlier", 17_000, 1500, 3, 4),
    ("plain float32 normals", 20_000, 4000, 3, 16),
    ("D = 2, coarse grid", 18_000, 2500, 2, 8),
    ("D = 1, duplicates", 16_384, 2000, 1, 2),
    ("K = 1", 16_500, 3333, 3, 1),
]


@pytest.mark.parametrize("name,M,N,D,K", SCREEN_CASES, ids=[c[0] for c in SCREEN_CASES])
def test_argkmin_matrix_core_screen_frames(name, M, N, D, K):
    import pairwise_reductions_amd as pr
    _announce("argkmin_screen", case=name, M=M, N=N, D=D, K=K)
    rng = np.random.default_rng(M + N + D + K)
    if name.startswith("far"):
        x = (1000.0 + rng.integers(0, 16, size=(M, D)) / 16.0).astype(np.float32)
        y = (1000.0 + rng.integers(0, 16, size=(N, D)) / 16.0).astype(np.float32)
    elif name.startswith("one far"):
        x = workloads.grid24(rng, (M, D))
        y = workloads.grid24(rng, (N, D))
        y[N // 2] = 1.0e6
    elif name.startswith("plain"):
        x = (rng.standard_normal((M, D)) * 3.0).astype(np.float32)
        y = (rng.standard_normal((N, D)) * 3.0).astype(np.float32)
    elif name.startswith("D = 2"):
        x = (rng.integers(0, 12, size=(M, D)) / 12.0).astype(np.float32)
        y = (rng.integers(0, 12, size=(N, D)) / 12.0).astype(np.float32)
    elif name.startswith("D = 1"):
        x = workloads.grid24(rng, (M, D))
        y = workloads.grid24(rng, (N, D))
        y[300:400] = y[7]
    else:
        x = workloads.grid24(rng, (M, D))
        y = workloads.grid24(rng, (N, D))
    idx, dist = pr.argkmin(_dev(x), _dev(y), K, with_dist=True)
    want_idx, want_d2 = oracle.argkmin(x, y, K, workers=8)
    assert np.array_equal(_host(idx).astype(np.int64), want_idx)
    assert np.allclose(_host(dist), want_d2, rtol=1e-6, atol=0)
    sig = float(np.float32(0.1))
    fidx = _host(pr.argkmin_lse(_dev(x), _dev(y), K, sig)[0]).astype(np.int64)
    assert np.array_equal(fidx, want_idx)


def test_argkmin_screening_far_from_origin_and_unaligned_values():
    """The screening bound grows with |x|^2 + max|y|^2: points near 1000 on a coarse grid
    (many exact ties) and plain float32 values (keys not exact) must still give the oracle's
    indices bit for bit, ties to the lower index."""
    import pairwise_reductions_amd as pr
    _announce("argkmin_screening")
    rng = np.random.default_rng(31)
    x = (1000.0 + rng.integers(0, 16, size=(3000, 3)) / 16.0).astype(np.float32)
    y = (1000.0 + rng.integers(0, 16, size=(9000, 3)) / 16.0).astype(np.float32)
    for K in (1, 10, 32):
        idx = _host(pr.argkmin(_dev(x), _dev(y), K)).astype(np.int64)
        want, _ = oracle.argkmin(x, y, K, workers=8)
        assert np.array_equal(idx, want), K
    x2 = (rng.standard_normal((2000, 5)) * 3.0).astype(np.float32)
    y2 = (rng.standard_normal((7000, 5)) * 3.0).astype(np.float32)
    y2[500:600] = y2[0]
    idx, lse = pr.argkmin_lse(_dev(x2), _dev(y2), 12, 0.7)
    want, _ = oracle.argkmin(x2, y2, 12, workers=8)
    assert np.array_equal(_host(idx).astype(np.int64), want)
    want_lse = oracle.logsumexp_reduction(x2, y2, float(np.float32(0.7)), workers=8)
    assert np.all(np.abs(_host(lse) - want_lse) <= lse_bound(want_lse))


