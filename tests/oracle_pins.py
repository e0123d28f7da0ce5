"""Pins for the CPU oracle: checks against facts other than the oracle itself.

Each check takes the oracle module as ``o`` so that tests/test_oracle_mutations.py can run
the same checks against deliberately broken copies of the oracle and confirm each plausible
mistake is caught. Checks raise AssertionError on failure.

What pins what (page citations are by title and section):
  * closed forms: the Gaussian lattice sum equals the Gaussian integral (2 pi sigma^2)^(D/2)
    up to exponentially small terms (Poisson summation), the self term exp(0) = 1, a
    hand-computed exp(-2);
  * independent library routes: scikit-learn's rbf_kernel, scipy's cdist and logsumexp,
    scipy's cKDTree, PyTorch's scaled_dot_product_attention (the two augmentations of
    "Fast Gauss Sums via Flash Attention", Algorithms 1 and 2) and torch.autograd for the
    gradient of the loss sum_i a_i^2 from the KeOps LazyTensor example;
  * exact arithmetic: argKmin against a full sort of exact rational squared distances;
  * limits and invariants: sigma -> infinity, coincident columns, translation invariance,
    central finite differences of the (separately pinned) forward;
  * spectral facts of the diffusion operator ("FlashDiffusion", section 2.2): the
    normalised operator has eigenvalue 1 with eigenvector sqrt(d) and no larger one, and
    its Markov form has unit row sums.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np


def _rng(seed=0):
    return np.random.default_rng(seed)


def _grid_points(rng, shape, bits=12):
    return (rng.integers(0, 2 ** bits, size=shape) * 2.0 ** -bits).astype(np.float32)


# ----------------------------------------------------------------------------- gauss sum

def check_gauss_sigma_infinity(o):
    """sigma -> infinity: every kernel value is exactly 1, so s_i = sum_j b_j."""
    rng = _rng(1)
    x = rng.random((7, 3)).astype(np.float32)
    y = rng.random((11, 3)).astype(np.float32)
    b = rng.standard_normal((11, 2)).astype(np.float32)
    s, n = o.gauss_sum(x, y, b, 1e30)
    want = b.astype(np.float64).sum(axis=0)
    assert np.allclose(s, np.broadcast_to(want, s.shape), rtol=0, atol=1e-12)
    assert np.allclose(n, np.abs(b).astype(np.float64).sum(axis=0), rtol=0, atol=1e-12)


def check_gauss_hand_values(o):
    """Hand-computed kernel values: |x-y|^2 = 1 with sigma = 1/2 gives exp(-2); x = y gives 1."""
    x = np.array([[1.0, 0.0, 0.0], [0.0, 0.0, 0.0]], dtype=np.float32)
    y = np.array([[0.0, 0.0, 0.0]], dtype=np.float32)
    b = np.array([[3.0]], dtype=np.float32)
    s, _ = o.gauss_sum(x, y, b, 0.5)
    assert abs(s[0, 0] - 3.0 * math.exp(-2.0)) <= 1e-15
    assert s[1, 0] == 3.0
    # |x - y|^2 = 0.25 + 4 = 4.25 with sigma = 2: exp(-4.25/8)
    x2 = np.array([[0.5, 2.0]], dtype=np.float32)
    y2 = np.array([[0.0, 0.0]], dtype=np.float32)
    s2, _ = o.gauss_sum(x2, y2, np.array([[1.0]], dtype=np.float32), 2.0)
    assert abs(s2[0, 0] - math.exp(-4.25 / 8.0)) <= 1e-15


def check_gauss_coincident_columns(o):
    """All y_j equal to y0 and all b_j equal to b0: s_i = N exp(-|x_i-y0|^2/(2 sigma^2)) b0,
    written here through the one-dimensional factorisation of the exponential."""
    rng = _rng(2)
    N = 13
    x = rng.random((5, 3)).astype(np.float32)
    y0 = np.array([0.25, 0.5, 0.75], dtype=np.float32)
    y = np.tile(y0, (N, 1))
    b = np.full((N, 1), -1.5, dtype=np.float32)
    sigma = 0.3
    s, _ = o.gauss_sum(x, y, b, sigma)
    for i in range(5):
        k = 1.0
        for d in range(3):
            k *= math.exp(-((float(x[i, d]) - float(y0[d])) ** 2) / (2 * sigma * sigma))
        assert abs(s[i, 0] - N * k * -1.5) <= 1e-13 * N


def check_gauss_self_term(o):
    """x_i = y_j and every other column far away (its kernel underflows to 0): s_i = b_j."""
    y = np.array([[0.0, 0.0, 0.0], [50.0, 0.0, 0.0], [0.0, 60.0, 0.0]], dtype=np.float32)
    b = np.array([[0.75], [2.0], [-4.0]], dtype=np.float32)
    x = y[[1, 0, 2]]
    s, n = o.gauss_sum(x, y, b, 0.5)
    assert s[0, 0] == 2.0 and s[1, 0] == 0.75 and s[2, 0] == -4.0
    assert n[2, 0] == 4.0


def check_gauss_lattice_integral(o):
    """Closed form: columns on a cubic lattice of spacing h = sigma/2 with weights h^D sum to
    the Gaussian integral (2 pi sigma^2)^(D/2); by Poisson summation the relative error is
    about 2 exp(-2 pi^2 sigma^2 / h^2) = 2 exp(-8 pi^2) ~ 1e-34, and truncating the lattice
    at 12 sigma costs exp(-72)."""
    for D, sigma in ((1, 0.37), (2, 0.2), (3, 0.1)):
        h = sigma / 2
        ticks = np.arange(-24, 25) * h
        mesh = np.meshgrid(*([ticks] * D), indexing="ij")
        y = np.stack([m.ravel() for m in mesh], axis=1)
        b = np.full((y.shape[0], 1), h ** D)
        x = np.array([[0.3 * h] * D, [-0.45 * h] * D, [0.0] * D])
        s, _ = o.gauss_sum(x, y, b, sigma)
        want = (2 * math.pi * sigma * sigma) ** (D / 2)
        assert np.allclose(s[:, 0], want, rtol=1e-11, atol=0), (D, s[:, 0], want)


def check_gauss_vs_sklearn(o):
    """Independent library route: sklearn's rbf_kernel(X, Y, gamma) = exp(-gamma |x-y|^2)."""
    from sklearn.metrics.pairwise import rbf_kernel
    rng = _rng(3)
    x = rng.random((37, 3)).astype(np.float32)
    y = rng.random((53, 3)).astype(np.float32)
    b = rng.standard_normal((53, 3)).astype(np.float32)
    for sigma in (0.05, 0.3, 2.0):
        s, n = o.gauss_sum(x, y, b, sigma)
        K = rbf_kernel(x.astype(np.float64), y.astype(np.float64), gamma=1.0 / (2 * sigma * sigma))
        assert np.allclose(s, K @ b.astype(np.float64), rtol=1e-10, atol=1e-13)
        assert np.allclose(n, K @ np.abs(b.astype(np.float64)), rtol=1e-10, atol=1e-13)


def check_keops_example_convention(o):
    """The KeOps LazyTensor example uses K_ij = exp(-D_ij) with D_ij the squared distance,
    i.e. sigma = 1/sqrt(2); a_i = sum_j K_ij. Compared with scipy's cdist."""
    from scipy.spatial.distance import cdist
    rng = _rng(4)
    x = rng.standard_normal((20, 3)).astype(np.float32)
    y = rng.standard_normal((30, 3)).astype(np.float32)
    Dij = cdist(x.astype(np.float64), y.astype(np.float64), "sqeuclidean")
    s, _ = o.gauss_sum(x, y, np.ones((30, 1), np.float32), 1.0 / math.sqrt(2.0))
    assert np.allclose(s[:, 0], np.exp(-Dij).sum(axis=1), rtol=1e-12, atol=0)


def check_gauss_permutations(o):
    """Permuting rows permutes outputs; permuting columns with their weights changes nothing;
    the result is linear in b; and sum_i s_i(x, y) = sum_j s_j(y, x) for unit weights."""
    rng = _rng(5)
    x = rng.random((9, 2)).astype(np.float32)
    y = rng.random((14, 2)).astype(np.float32)
    b1 = rng.standard_normal((14, 1)).astype(np.float32)
    b2 = rng.standard_normal((14, 1)).astype(np.float32)
    sig = 0.2
    s1, _ = o.gauss_sum(x, y, b1, sig)
    pr = rng.permutation(9)
    pc = rng.permutation(14)
    sp, _ = o.gauss_sum(x[pr], y[pc], b1[pc], sig)
    assert np.allclose(sp, s1[pr], rtol=1e-13, atol=1e-15)
    s2, _ = o.gauss_sum(x, y, b2, sig)
    s12, _ = o.gauss_sum(x, y, 2.0 * b1.astype(np.float64) - 3.0 * b2.astype(np.float64), sig)
    assert np.allclose(s12, 2 * s1 - 3 * s2, rtol=1e-12, atol=1e-13)
    a, _ = o.gauss_sum(x, y, np.ones((14, 1), np.float32), sig)
    c, _ = o.gauss_sum(y, x, np.ones((9, 1), np.float32), sig)
    assert abs(a.sum() - c.sum()) <= 1e-12 * a.sum()


# ---------------------------------------------------------------------------- batched

def _rux_inputs(seed=6, B=2, M=12, N=17, D=5, C=3):
    rng = _rng(seed)
    q = (rng.standard_normal((B, M, D)) / math.sqrt(D)).astype(np.float16)
    k = (rng.standard_normal((B, N, D)) / math.sqrt(D)).astype(np.float16)
    v = rng.standard_normal((B, N, C)).astype(np.float16)
    return q, k, v


def check_batched_rux_reweight(o):
    """"Fast Gauss Sums via Flash Attention", Algorithm 2 (reweight): pad q, k, v, add the
    extra key e_{D+2} with value kappa e_{C+1}, run softmax attention with scale tau, and
    s = kappa * alpha / beta. Attention here is torch's scaled_dot_product_attention."""
    import torch
    q, k, v = _rux_inputs()
    B, M, D = q.shape
    N, C = k.shape[1], v.shape[2]
    for tau in (1.0, 2.5):
        s, _ = o.gauss_sum_batched(q, k, v, tau)
        qt = torch.from_numpy(q.astype(np.float64))
        kt = torch.from_numpy(k.astype(np.float64))
        vt = torch.from_numpy(v.astype(np.float64))
        kappa = math.sqrt(N + 1)
        qa = torch.cat([qt, torch.ones(B, M, 1, dtype=torch.float64),
                        0.5 * (qt * qt).sum(-1, keepdim=True)], dim=-1)
        ka = torch.cat([kt, -0.5 * (kt * kt).sum(-1, keepdim=True),
                        torch.zeros(B, N, 1, dtype=torch.float64)], dim=-1)
        k0 = torch.zeros(B, 1, D + 2, dtype=torch.float64)
        k0[..., D + 1] = 1.0
        ka = torch.cat([k0, ka], dim=1)
        va = torch.cat([vt, torch.zeros(B, N, 1, dtype=torch.float64)], dim=-1)
        v0 = torch.zeros(B, 1, C + 1, dtype=torch.float64)
        v0[..., C] = kappa
        va = torch.cat([v0, va], dim=1)
        out = torch.nn.functional.scaled_dot_product_attention(qa, ka, va, scale=tau)
        alpha, beta = out[..., :C], out[..., C:]
        want = (kappa * alpha / beta).numpy()
        assert np.allclose(s, want, rtol=1e-10, atol=1e-12)


def check_batched_rux_prescale(o):
    """"Fast Gauss Sums via Flash Attention", Algorithm 1 (prescale): v~ = v exp(-tau/2 |k|^2),
    s = att(q, k, v~) exp(lse(q, k)) exp(-tau/2 |q|^2), with att the softmax attention with
    scale tau (torch SDPA) and lse the log-sum-exp of tau q.k (torch.logsumexp)."""
    import torch
    q, k, v = _rux_inputs(seed=7)
    tau = 1.7
    s, _ = o.gauss_sum_batched(q, k, v, tau)
    qt = torch.from_numpy(q.astype(np.float64))
    kt = torch.from_numpy(k.astype(np.float64))
    vt = torch.from_numpy(v.astype(np.float64))
    vs = vt * torch.exp(-0.5 * tau * (kt * kt).sum(-1, keepdim=True))
    att = torch.nn.functional.scaled_dot_product_attention(qt, kt, vs, scale=tau)
    lse = torch.logsumexp(tau * qt @ kt.transpose(-1, -2), dim=-1, keepdim=True)
    want = (att * torch.exp(lse) * torch.exp(-0.5 * tau * (qt * qt).sum(-1, keepdim=True))).numpy()
    assert np.allclose(s, want, rtol=1e-10, atol=1e-12)


def check_batched_independent(o):
    """Each batch entry is its own problem: batch t equals gauss_sum with sigma = 1/sqrt(tau)."""
    q, k, v = _rux_inputs(seed=8, B=3)
    tau = 4.0
    s, n = o.gauss_sum_batched(q, k, v, tau)
    for t in range(3):
        st, nt = o.gauss_sum(q[t], k[t], v[t], 0.5)
        assert np.allclose(s[t], st, rtol=1e-13, atol=1e-15)
        assert np.allclose(n[t], nt, rtol=1e-13, atol=1e-15)


# -------------------------------------------------------------------------------- lse

def check_lse_vs_scipy(o):
    """scipy.special.logsumexp over f = -cdist^2/(2 sigma^2)."""
    from scipy.spatial.distance import cdist
    from scipy.special import logsumexp
    rng = _rng(9)
    x = rng.random((23, 3)).astype(np.float32)
    y = rng.random((41, 3)).astype(np.float32)
    for sigma in (0.01, 0.1, 1.0):
        f = -cdist(x.astype(np.float64), y.astype(np.float64), "sqeuclidean") / (2 * sigma * sigma)
        got = o.logsumexp_reduction(x, y, sigma)
        assert np.allclose(got, logsumexp(f, axis=1), rtol=1e-13, atol=1e-12)


def check_lse_identical_columns(o):
    """N identical columns: lse_i = log N - |x_i - y0|^2 / (2 sigma^2)."""
    x = np.array([[0.1, 0.2, 0.3], [2.0, -1.0, 0.5]], dtype=np.float32)
    y0 = np.array([0.5, 0.5, 0.5], dtype=np.float32)
    N = 1000
    y = np.tile(y0, (N, 1))
    sigma = 0.05
    got = o.logsumexp_reduction(x, y, sigma)
    for i in range(2):
        d2 = sum((float(x[i, d]) - float(y0[d])) ** 2 for d in range(3))
        want = math.log(N) - d2 / (2 * sigma * sigma)
        assert abs(got[i] - want) <= 1e-12 * max(1.0, abs(want))


def check_lse_far_cloud(o):
    """A column cloud far from the row: the plain sum of exponentials underflows to 0 but the
    reduction stays finite; for a single far column it is exactly -d^2/(2 sigma^2)."""
    x = np.array([[0.0, 0.0, 0.0]], dtype=np.float32)
    y = np.array([[30.0, 40.0, 0.0]], dtype=np.float32)  # distance 50
    sigma = 0.1
    got = o.logsumexp_reduction(x, y, sigma)
    assert got[0] == -2500.0 / (2 * 0.1 * 0.1) or abs(got[0] + 125000.0) <= 1e-9
    y2 = np.array([[30.0, 40.0, 0.0], [30.0, 40.0, 0.0]], dtype=np.float32)
    got2 = o.logsumexp_reduction(x, y2, sigma)
    assert abs(got2[0] - (math.log(2.0) - 125000.0)) <= 1e-9


def check_lse_lattice(o):
    """Closed form via the lattice integral: lse = log((2 pi sigma^2)^(3/2) / h^3)."""
    sigma = 0.1
    h = sigma / 2
    ticks = np.arange(-24, 25) * h
    mesh = np.meshgrid(ticks, ticks, ticks, indexing="ij")
    y = np.stack([m.ravel() for m in mesh], axis=1)
    x = np.array([[0.2 * h, -0.1 * h, 0.4 * h]])
    got = o.logsumexp_reduction(x, y, sigma)
    want = math.log((2 * math.pi * sigma * sigma) ** 1.5 / h ** 3)
    assert abs(got[0] - want) <= 1e-12


def check_lse_empty(o):
    x = np.zeros((3, 3), np.float32)
    y = np.zeros((0, 3), np.float32)
    got = o.logsumexp_reduction(x, y, 0.1)
    assert got.shape == (3,) and np.all(np.isneginf(got))


def check_lse_consistent_with_sum(o):
    """Where nothing underflows, lse_i = log(sum_j k_ij) = log of the unit-weight Gauss sum."""
    rng = _rng(10)
    x = rng.random((15, 3)).astype(np.float32)
    y = rng.random((25, 3)).astype(np.float32)
    s, _ = o.gauss_sum(x, y, np.ones((25, 1), np.float32), 0.5)
    got = o.logsumexp_reduction(x, y, 0.5)
    assert np.allclose(got, np.log(s[:, 0]), rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------- argkmin

def _exact_rank(x, y, K):
    """Exact squared distances of the float32 values as rationals, sorted by (d2, j)."""
    out = []
    for i in range(x.shape[0]):
        keys = []
        for j in range(y.shape[0]):
            d2 = sum((Fraction(float(x[i, d])) - Fraction(float(y[j, d]))) ** 2 for d in range(x.shape[1]))
            keys.append((d2, j))
        keys.sort()
        out.append([j for _, j in keys[:K]])
    return np.array(out)


def check_argkmin_exact_bruteforce(o):
    """Full sort of exact rational squared distances, with planted duplicate columns and an
    equidistant configuration so that ties must resolve to the lower index."""
    rng = _rng(11)
    x = _grid_points(rng, (9, 3))
    y = _grid_points(rng, (30, 3))
    y[7] = y[3]
    y[20] = y[3]          # triple duplicate
    y[12] = x[0]          # exact hit
    y[25] = y[12]         # duplicate of the hit
    # columns at equal distance 0.25 from x[1] in different directions
    for j, dvec in zip((2, 5, 9), ((0.25, 0, 0), (0, -0.25, 0), (0, 0, 0.25))):
        y[j] = x[1] + np.array(dvec, dtype=np.float32)
    for K in (1, 4, 30):
        idx, d2 = o.argkmin(x, y, K)
        assert np.array_equal(idx, _exact_rank(x, y, K))
        for i in range(x.shape[0]):
            for r in range(K):
                j = idx[i, r]
                exact = sum((Fraction(float(x[i, d])) - Fraction(float(y[j, d]))) ** 2 for d in range(3))
                assert Fraction(d2[i, r]) == exact


def check_argkmin_k1_is_argmin(o):
    """K = 1 is the argmin with the first occurrence on ties (numpy.argmin on scipy's cdist)."""
    from scipy.spatial.distance import cdist
    rng = _rng(12)
    x = _grid_points(rng, (40, 3), bits=4)
    y = _grid_points(rng, (70, 3), bits=4)    # coarse grid: many exact ties
    idx, _ = o.argkmin(x, y, 1)
    Dm = cdist(x.astype(np.float64), y.astype(np.float64), "sqeuclidean")
    assert np.array_equal(idx[:, 0], np.argmin(Dm, axis=1))


def check_argkmin_vs_kdtree(o):
    """Distances of the K nearest columns agree with scipy's cKDTree (its tie order unused)."""
    from scipy.spatial import cKDTree
    rng = _rng(13)
    x = rng.random((50, 3)).astype(np.float32)
    y = rng.random((400, 3)).astype(np.float32)
    K = 8
    _, d2 = o.argkmin(x, y, K)
    dd, _ = cKDTree(y.astype(np.float64)).query(x.astype(np.float64), k=K)
    assert np.allclose(np.sqrt(d2), dd, rtol=1e-12, atol=1e-14)


def check_keys_exact_flag(o):
    rng = _rng(14)
    x = (rng.integers(0, 2 ** 24, size=(5, 3)) * 2.0 ** -24).astype(np.float32)
    assert o.keys_are_exact(x, x)
    z = rng.standard_normal((5, 3)).astype(np.float32) * 1000
    assert not o.keys_are_exact(z, np.array([[1e-30, 0, 0]], np.float32))


# ------------------------------------------------------------------------------- grad

def check_grad_vs_autograd(o):
    """torch.autograd on the dense float64 formula, loss = sum_i a_i^2 (the KeOps LazyTensor
    example), so the upstream gradient is g = 2 a."""
    import torch
    rng = _rng(15)
    for (M, N, D, C, sigma) in ((11, 19, 3, 1, 0.3), (7, 9, 2, 3, 0.8)):
        x = rng.random((M, D)).astype(np.float32)
        y = rng.random((N, D)).astype(np.float32)
        b = rng.standard_normal((N, C)).astype(np.float32)
        xt = torch.tensor(x.astype(np.float64), requires_grad=True)
        yt = torch.from_numpy(y.astype(np.float64))
        bt = torch.from_numpy(b.astype(np.float64))
        Dij = ((xt[:, None, :] - yt[None, :, :]) ** 2).sum(-1)
        a = torch.exp(-Dij / (2 * sigma * sigma)) @ bt
        (gx,) = torch.autograd.grad((a ** 2).sum(), [xt])
        g = 2.0 * a.detach().numpy()
        got, _ = o.gauss_sum_grad_x(x, y, b, g, sigma)
        assert np.allclose(got, gx.numpy(), rtol=1e-11, atol=1e-12)


def check_grad_finite_differences(o):
    """Central differences of the forward reduction in float64 (step 1e-6)."""
    rng = _rng(16)
    x = rng.random((4, 3))
    y = rng.random((12, 3))
    b = rng.standard_normal((12, 2))
    g = rng.standard_normal((4, 2))
    sigma = 0.4
    got, _ = o.gauss_sum_grad_x(x, y, b, g, sigma)
    h = 1e-6
    for i in range(4):
        for d in range(3):
            xp = x.copy(); xp[i, d] += h
            xm = x.copy(); xm[i, d] -= h
            sp, _ = o.gauss_sum(xp, y, b, sigma)
            sm, _ = o.gauss_sum(xm, y, b, sigma)
            fd = float((g[i] * (sp[i] - sm[i])).sum() / (2 * h))
            assert abs(fd - got[i, d]) <= 1e-7 * max(1.0, abs(fd))


def check_grad_limits(o):
    """x = y for a single pair gives exactly 0; for sigma -> infinity every kernel value is
    1, so sigma^2 grad_i -> -sum_j (g_i . b_j)(x_i - y_j); translation invariance."""
    z = np.array([[0.3, 0.1, 0.9]])
    got, _ = o.gauss_sum_grad_x(z, z, np.array([[2.0]]), np.array([[1.5]]), 0.2)
    assert np.all(got == 0.0)
    rng = _rng(17)
    x = rng.random((5, 3))
    y = rng.random((8, 3))
    b = rng.standard_normal((8, 1))
    g = rng.standard_normal((5, 1))
    big = 1e8
    got, _ = o.gauss_sum_grad_x(x, y, b, g, big)
    want = -((g @ b.T)[:, :, None] * (x[:, None, :] - y[None, :, :])).sum(axis=1)
    assert np.allclose(got * big * big, want, rtol=1e-6, atol=1e-9)
    shift = np.array([5.0, -3.0, 2.0])
    g1, _ = o.gauss_sum_grad_x(x, y, b, g, 0.3)
    g2, _ = o.gauss_sum_grad_x(x + shift, y + shift, b, g, 0.3)
    assert np.allclose(g1, g2, rtol=1e-9, atol=1e-12)


def check_grad_yb_vs_autograd(o):
    """torch.autograd of sum_i (a_i . w_i) for a fixed w on the dense float64 formula gives
    the gradients with respect to y and b for the upstream gradient g = w."""
    import torch
    rng = _rng(18)
    for (M, N, D, C, sigma) in ((13, 9, 3, 1, 0.35), (6, 11, 2, 3, 0.9)):
        x = rng.random((M, D)).astype(np.float32)
        y = rng.random((N, D)).astype(np.float32)
        b = rng.standard_normal((N, C)).astype(np.float32)
        w = rng.standard_normal((M, C))
        xt = torch.from_numpy(x.astype(np.float64))
        yt = torch.tensor(y.astype(np.float64), requires_grad=True)
        bt = torch.tensor(b.astype(np.float64), requires_grad=True)
        Dij = ((xt[:, None, :] - yt[None, :, :]) ** 2).sum(-1)
        a = torch.exp(-Dij / (2 * sigma * sigma)) @ bt
        gy, gb = torch.autograd.grad((a * torch.from_numpy(w)).sum(), [yt, bt])
        got_y, _ = o.gauss_sum_grad_y(x, y, b, w, sigma)
        got_b, _ = o.gauss_sum_grad_b(x, y, w, sigma)
        assert np.allclose(got_y, gy.numpy(), rtol=1e-11, atol=1e-12)
        assert np.allclose(got_b, gb.numpy(), rtol=1e-11, atol=1e-12)


def check_grad_y_finite_differences_and_limits(o):
    """Central differences in y of the forward; sigma -> infinity makes grad_b_j = sum_i g_i;
    moving every point by the same vector leaves both gradients unchanged."""
    rng = _rng(19)
    x = rng.random((7, 3))
    y = rng.random((5, 3))
    b = rng.standard_normal((5, 2))
    g = rng.standard_normal((7, 2))
    sigma = 0.45
    got, _ = o.gauss_sum_grad_y(x, y, b, g, sigma)
    h = 1e-6
    for j in range(5):
        for d in range(3):
            yp = y.copy(); yp[j, d] += h
            ym = y.copy(); ym[j, d] -= h
            sp, _ = o.gauss_sum(x, yp, b, sigma)
            sm, _ = o.gauss_sum(x, ym, b, sigma)
            fd = float((g * (sp - sm)).sum() / (2 * h))
            assert abs(fd - got[j, d]) <= 1e-7 * max(1.0, abs(fd))
    gb, _ = o.gauss_sum_grad_b(x, y, g, 1e30)
    assert np.allclose(gb, np.broadcast_to(g.sum(axis=0), gb.shape), rtol=0, atol=1e-12)
    shift = np.array([-2.0, 7.0, 0.5])
    a1, _ = o.gauss_sum_grad_y(x, y, b, g, sigma)
    a2, _ = o.gauss_sum_grad_y(x + shift, y + shift, b, g, sigma)
    assert np.allclose(a1, a2, rtol=1e-9, atol=1e-12)


def check_argkmin_weighted_exact(o):
    """Weighted keys d2 - w as exact rationals (grid points, weights on a dyadic grid, so the
    float64 difference is exact), sorted by (key, j); planted equal keys (a column twice with
    the same weight, and two columns whose distance difference the weights cancel) resolve to
    the lower index."""
    rng = _rng(28)
    x = _grid_points(rng, (8, 3))
    y = _grid_points(rng, (25, 3))
    w = (rng.integers(-2 ** 10, 2 ** 10, size=25) * 2.0 ** -12).astype(np.float32)
    y[9] = y[4]
    w[9] = w[4]
    # column 15 at distance^2 0.25 from x[2] with weight 0.25 - 0.0625 ties column 16 at 0.0625, weight 0
    y[15] = x[2] + np.array([0.5, 0, 0], dtype=np.float32)
    w[15] = np.float32(0.1875)
    y[16] = x[2] + np.array([0, 0.25, 0], dtype=np.float32)
    w[16] = np.float32(0.0)
    for K in (1, 3, 25):
        idx, keys = o.argkmin_weighted(x, y, w, K)
        for i in range(x.shape[0]):
            exact = []
            for j in range(25):
                d2 = sum((Fraction(float(x[i, d])) - Fraction(float(y[j, d]))) ** 2 for d in range(3))
                exact.append((d2 - Fraction(float(w[j])), j))
            exact.sort()
            assert list(idx[i]) == [j for _, j in exact[:K]]
            assert all(Fraction(keys[i, r]) == exact[r][0] for r in range(K))


def check_argkmin_weighted_reductions(o):
    """w = 0 is plain argKmin; a constant weight changes no index and shifts every key; with
    w_j = 2 sigma^2 ln b_j the K = 1 column is the argmax of b_j exp(-d2/(2 sigma^2))
    (numpy exp, well-separated maxima)."""
    rng = _rng(29)
    x = rng.random((30, 3))
    y = rng.random((40, 3))
    i0, k0 = o.argkmin(x, y, 5)
    i1, k1 = o.argkmin_weighted(x, y, np.zeros(40), 5)
    assert np.array_equal(i0, i1) and np.array_equal(k0, k1)
    i2, k2 = o.argkmin_weighted(x, y, np.full(40, 0.375), 5)
    assert np.array_equal(i0, i2) and np.allclose(k2, k0 - 0.375, rtol=0, atol=1e-15)
    sigma = 0.2
    b = rng.random(40) + 0.1
    idx, _ = o.argkmin_weighted(x, y, 2 * sigma * sigma * np.log(b), 1)
    vals = b[None, :] * np.exp(-((x[:, None, :] - y[None, :, :]) ** 2).sum(-1) / (2 * sigma * sigma))
    top2 = np.sort(vals, axis=1)[:, -2:]
    sep = top2[:, 1] > top2[:, 0] * (1 + 1e-9)
    assert np.array_equal(idx[sep, 0], np.argmax(vals, axis=1)[sep])


# ------------------------------------------------------------- batched backward (fp16 path)

def check_batched_backward_vs_attention_autograd(o):
    """torch.autograd through "Fast Gauss Sums via Flash Attention", Algorithm 1 (prescale:
    s = att_tau(q, k, v~) e^{lse_tau(q, k~)} e^{-tau/2 |q|^2} with v~ = v e^{-tau/2 |k|^2}),
    evaluated with scaled_dot_product_attention and logsumexp in float64, gives the
    gradients of sum_m (s_m . w_m) with respect to q, k and v."""
    import torch
    q, k, v = _rux_inputs(seed=21, B=2, M=9, N=11, D=4, C=3)
    w = _rng(22).standard_normal((2, 9, 3))
    for sigma in (0.8, 1.7):
        tau = 1.0 / (sigma * sigma)
        qt = torch.tensor(q.astype(np.float64), requires_grad=True)
        kt = torch.tensor(k.astype(np.float64), requires_grad=True)
        vt = torch.tensor(v.astype(np.float64), requires_grad=True)
        kk = (kt * kt).sum(-1)
        vtil = vt * torch.exp(-0.5 * tau * kk)[..., None]
        att = torch.nn.functional.scaled_dot_product_attention(qt, kt, vtil, scale=tau)
        # att uses softmax over tau q.k; undo its normalisation with the log-sum-exp
        lse = torch.logsumexp(tau * qt @ kt.transpose(-1, -2), dim=-1)
        s = att * torch.exp(lse - 0.5 * tau * (qt * qt).sum(-1))[..., None]
        gq, gk, gv = torch.autograd.grad((s * torch.from_numpy(w)).sum(), [qt, kt, vt])
        got = o.gauss_sum_batched_backward(q, k, v, w, sigma)
        assert np.allclose(got["x"][0], gq.numpy(), rtol=1e-9, atol=1e-12)
        assert np.allclose(got["y"][0], gk.numpy(), rtol=1e-9, atol=1e-12)
        assert np.allclose(got["b"][0], gv.numpy(), rtol=1e-9, atol=1e-12)


# ------------------------------------------------------------ scaled operator, diffusion

def _rbf(x, y, sigma):
    from sklearn.metrics.pairwise import rbf_kernel
    return rbf_kernel(np.asarray(x, np.float64), np.asarray(y, np.float64), gamma=1.0 / (2.0 * sigma * sigma))


def check_scaled_vs_dense_diagonals(o):
    """"FlashDiffusion", section 2.2: diag(r) K diag(c) V with the kernel matrix from
    scikit-learn's rbf_kernel and explicit diagonal matrices; signed scales."""
    rng = _rng(23)
    x = rng.random((10, 3))
    y = rng.random((14, 3))
    b = rng.standard_normal((14, 2))
    r = rng.standard_normal(10)
    c = rng.standard_normal(14)
    sigma = 0.4
    K = _rbf(x, y, sigma)
    want = np.diag(r) @ K @ np.diag(c) @ b
    got, n = o.gauss_sum_scaled(x, y, b, sigma, row_scale=r, col_scale=c)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-14)
    assert np.allclose(n, np.abs(np.diag(r) @ K) @ np.abs(np.diag(c) @ b), rtol=1e-12, atol=1e-14)
    only_r, _ = o.gauss_sum_scaled(x, y, b, sigma, row_scale=r)
    assert np.allclose(only_r, np.diag(r) @ K @ b, rtol=1e-12, atol=1e-14)
    only_c, _ = o.gauss_sum_scaled(x, y, b, sigma, col_scale=c)
    assert np.allclose(only_c, K @ np.diag(c) @ b, rtol=1e-12, atol=1e-14)


def check_scaled_single_column(o):
    """A column scale that keeps one column j0 gives r_i k(x_i, y_j0) c_j0 b_j0 (math.exp)."""
    rng = _rng(24)
    x = rng.random((5, 2))
    y = rng.random((6, 2))
    b = rng.standard_normal((6, 1))
    r = rng.random(5) + 0.5
    c = np.zeros(6)
    c[3] = -1.75
    sigma = 0.6
    got, _ = o.gauss_sum_scaled(x, y, b, sigma, row_scale=r, col_scale=c)
    for i in range(5):
        d2 = sum((x[i, d] - y[3, d]) ** 2 for d in range(2))
        want = r[i] * math.exp(-d2 / (2 * sigma * sigma)) * c[3] * b[3, 0]
        assert abs(got[i, 0] - want) <= 1e-14 * max(1.0, abs(want))


def check_diffusion_dense_formula(o):
    """The alpha-normalised symmetric diffusion matrix built densely: q = K 1,
    K_a = diag(q^-a) K diag(q^-a), d = K_a 1, s = q^-a d^-1/2 (kernel from scikit-learn)."""
    rng = _rng(25)
    x = rng.random((12, 3))
    sigma = 0.3
    K = _rbf(x, x, sigma)
    q = K.sum(axis=1)
    for alpha in (0.0, 0.5, 1.0):
        Ka = np.diag(q ** -alpha) @ K @ np.diag(q ** -alpha)
        d = Ka.sum(axis=1)
        s, qo, do = o.diffusion_scaling(x, sigma, alpha)
        assert np.allclose(qo, q, rtol=1e-12)
        assert np.allclose(do, d, rtol=1e-12)
        assert np.allclose(s, q ** -alpha / np.sqrt(d), rtol=1e-12)


def check_diffusion_spectrum(o):
    """A = diag(s) K diag(s) has the eigenvector sqrt(d) with eigenvalue 1, its largest
    (A is similar to the row-stochastic D^-1 K_alpha), and D^-1 K_alpha has unit row sums."""
    rng = _rng(26)
    x = rng.random((15, 2))
    sigma = 0.25
    K = _rbf(x, x, sigma)
    for alpha in (0.5, 1.0):
        s, q, d = o.diffusion_scaling(x, sigma, alpha)
        A = np.diag(s) @ K @ np.diag(s)
        assert np.allclose(A @ np.sqrt(d), np.sqrt(d), rtol=1e-11)
        ev = np.linalg.eigvalsh(A)
        assert abs(ev[-1] - 1.0) < 1e-11 and ev[0] > -1.0 - 1e-11
        p = q ** -alpha
        P = np.diag(1.0 / d) @ np.diag(p) @ K @ np.diag(p)
        assert np.allclose(P.sum(axis=1), 1.0, rtol=1e-12)


def check_diffusion_sigma_infinity(o):
    """sigma -> infinity: K is all ones, q = N, d = N^(1 - 2 alpha) and s = 1/sqrt(N)."""
    x = _rng(27).random((9, 3))
    for alpha in (0.0, 0.5, 1.0, 2.0):
        s, q, d = o.diffusion_scaling(x, 1e30, alpha)
        assert np.allclose(q, 9.0, rtol=1e-14)
        assert np.allclose(d, 9.0 ** (1 - 2 * alpha), rtol=1e-13)
        assert np.allclose(s, 1.0 / 3.0, rtol=1e-13)


GAUSS_CHECKS = [check_gauss_sigma_infinity, check_gauss_hand_values, check_gauss_coincident_columns,
                check_gauss_self_term, check_gauss_lattice_integral, check_gauss_vs_sklearn,
                check_keops_example_convention, check_gauss_permutations]
BATCHED_CHECKS = [check_batched_rux_reweight, check_batched_rux_prescale, check_batched_independent]
LSE_CHECKS = [check_lse_vs_scipy, check_lse_identical_columns, check_lse_far_cloud, check_lse_lattice,
              check_lse_empty, check_lse_consistent_with_sum]
ARGK_CHECKS = [check_argkmin_exact_bruteforce, check_argkmin_k1_is_argmin, check_argkmin_vs_kdtree,
               check_keys_exact_flag]
WARGK_CHECKS = [check_argkmin_weighted_exact, check_argkmin_weighted_reductions]
GRAD_CHECKS = [check_grad_vs_autograd, check_grad_finite_differences, check_grad_limits]
GRADYB_CHECKS = [check_grad_yb_vs_autograd, check_grad_y_finite_differences_and_limits]
BATCHED_GRAD_CHECKS = [check_batched_backward_vs_attention_autograd]
SCALED_CHECKS = [check_scaled_vs_dense_diagonals, check_scaled_single_column]
DIFFUSION_CHECKS = [check_diffusion_dense_formula, check_diffusion_spectrum, check_diffusion_sigma_infinity]
ALL_CHECKS = (GAUSS_CHECKS + BATCHED_CHECKS + LSE_CHECKS + ARGK_CHECKS + GRAD_CHECKS + GRADYB_CHECKS +
              BATCHED_GRAD_CHECKS + SCALED_CHECKS + DIFFUSION_CHECKS + WARGK_CHECKS)
