"""Whole-workload parity: the full-size workloads, run on the device in the launch
configuration the benchmark times, compared with the float64 oracle on every row (the
100k-point workloads and the batched fp16 one) or on 16,384 seeded rows plus the first and
last 64 (the 1M-point Gauss sum, whose 1e12 pairs the oracle cannot cover in a test).

The device results of one workload are computed once per session and cached; the oracle's
share is cut into row parts so that each test ends within tens of seconds on the host
cores. Tolerances are those of test_parity_gpu (argKmin indices bit-exact).
"""
import functools
import os

import numpy as np
import pytest

import oracle
from pairwise_reductions_amd import workloads
from test_parity_gpu import TOL_F16, TOL_F32, _announce, _dev, _host, assert_normalised, lse_bound

pytestmark = [pytest.mark.gpu, pytest.mark.full]

WORKERS = max(1, min(16, os.cpu_count() or 1))


def _parts(M, n):
    edges = np.linspace(0, M, n + 1).astype(np.int64)
    return [np.arange(edges[k], edges[k + 1]) for k in range(n)]


# ------------------------------------------- argKmin K = 10 + LSE, 100k x 100k, D = 3
@functools.lru_cache(maxsize=1)
def _argkmin_lse_device():
    import pairwise_reductions_amd as pr
    inp = workloads.make_inputs("argkmin_lse_100k")
    _announce("argkmin_lse_100k device", M=inp["M"], N=inp["N"], K=inp["K"])
    sig = float(inp["sigma"])
    xd, yd = _dev(inp["x"]), _dev(inp["y"])
    idx, dist = pr.argkmin(xd, yd, inp["K"], with_dist=True)
    lse = pr.lse(xd, yd, sig)
    fidx, fdist, flse = pr.argkmin_lse(xd, yd, inp["K"], sig, with_dist=True)
    out = {k: _host(v) for k, v in dict(idx=idx, dist=dist, lse=lse, fidx=fidx, fdist=fdist, flse=flse).items()}
    return inp, out


ARGK_PARTS = 4


@pytest.mark.parametrize("part", range(ARGK_PARTS))
def test_argkmin_lse_workload_100k_every_row(part):
    """Every row of the 100k x 100k, K = 10 workload through both entry points (argKmin +
    LSE as two calls, and the combined call): indices bit for bit, distances to 1e-6
    relative, the log-sum-exp within the LSE bound."""
    inp, got = _argkmin_lse_device()
    M, K = inp["M"], inp["K"]
    rows = _parts(M, ARGK_PARTS)[part]
    _announce("argkmin_lse_100k every row", part=part, rows=f"{rows[0]}..{rows[-1]}")
    assert oracle.keys_are_exact(inp["x"], inp["y"])
    want_idx, want_d2 = oracle.argkmin(inp["x"][rows], inp["y"], K, workers=WORKERS)
    want_lse = oracle.logsumexp_reduction(inp["x"][rows], inp["y"], float(inp["sigma"]), workers=WORKERS)
    for tag in ("", "f"):
        idx = got[tag + "idx"][rows].astype(np.int64)
        bad = np.flatnonzero(np.any(idx != want_idx, axis=1))
        assert bad.size == 0, f"{tag}argkmin: {bad.size} rows differ, first row {rows[bad[0]] if bad.size else -1}"
        assert np.allclose(got[tag + "dist"][rows], want_d2, rtol=1e-6, atol=0), f"{tag}argkmin distances"
        err = np.abs(got[tag + "lse"][rows].astype(np.float64) - want_lse)
        assert np.all(err <= lse_bound(want_lse)), f"{tag}lse: max error {err.max():.3e}"


# ------------------------------------------- forward + grad_x, 100k x 100k mixture
@functools.lru_cache(maxsize=1)
def _mixture_device():
    import pairwise_reductions_amd as pr
    inp = workloads.make_inputs("gauss_sum_grad_x_100k_mixture")
    _announce("mixture_100k device", M=inp["M"], N=inp["N"])
    sig = float(inp["sigma"])
    g = workloads.upstream_gradient(inp["M"], inp["C"])
    xd, yd, bd = _dev(inp["x"]), _dev(inp["y"]), _dev(inp["b"])
    s = _host(pr.gauss_sum(xd, yd, bd, sig))
    grad = _host(pr.gauss_sum_grad_x(xd, yd, bd, _dev(g), sig))
    return inp, g, s, grad


MIX_PARTS = 3


@pytest.mark.parametrize("part", range(MIX_PARTS))
def test_gauss_sum_grad_x_workload_100k_mixture_every_row(part):
    inp, g, s, grad = _mixture_device()
    rows = _parts(inp["M"], MIX_PARTS)[part]
    _announce("mixture_100k every row", part=part, rows=f"{rows[0]}..{rows[-1]}")
    sig = float(inp["sigma"])
    want_s, norm_s = oracle.gauss_sum(inp["x"][rows], inp["y"], inp["b"], sig, workers=WORKERS)
    assert_normalised(s[rows], want_s, norm_s, TOL_F32, "forward 100k")
    want_g, norm_g = oracle.gauss_sum_grad_x(inp["x"][rows], inp["y"], inp["b"], g[rows], sig, workers=WORKERS)
    assert_normalised(grad[rows], want_g, norm_g, TOL_F32, "grad_x 100k")


# ------------------------------------------- batched fp16, B = 4, 16384^2, D = C = 32
@functools.lru_cache(maxsize=1)
def _fp16_device():
    import pairwise_reductions_amd as pr
    inp = workloads.make_inputs("batched_gauss_sum_fp16")
    _announce("batched_fp16 device", B=inp["B"], M=inp["M"], N=inp["N"])
    got = _host(pr.gauss_sum(_dev(inp["x"]), _dev(inp["y"]), _dev(inp["b"]), float(inp["sigma"])))
    return inp, got


@pytest.mark.parametrize("batch", range(4))
def test_gauss_sum_fp16_workload_every_row(batch):
    inp, got = _fp16_device()
    _announce("batched_fp16 every row", batch=batch)
    t = slice(batch, batch + 1)
    want, norm = oracle.gauss_sum_batched(inp["x"][t], inp["y"][t], inp["b"][t], 1.0, workers=WORKERS)
    assert_normalised(got[t], want, norm, TOL_F16, f"fp16 workload batch {batch}")


# ------------------------------------------- Gauss sum 1M x 1M, sigma = 0.01
@functools.lru_cache(maxsize=1)
def _gauss_1m_device():
    import pairwise_reductions_amd as pr
    inp = workloads.make_inputs("gauss_sum_1m")
    _announce("gauss_sum_1m device", M=inp["M"], N=inp["N"])
    got = _host(pr.gauss_sum(_dev(inp["x"]), _dev(inp["y"]), _dev(inp["b"]), float(inp["sigma"])))
    rows = workloads.sample_rows(inp["M"], 16384, seed=1, edge=64)
    return inp, got, rows


G1M_PARTS = 4


@pytest.mark.parametrize("part", range(G1M_PARTS))
def test_gauss_sum_workload_1m_16k_rows(part):
    """16,384 seeded rows plus the first and last 64 of the 1M x 1M sum, each against all
    1e6 columns."""
    inp, got, rows = _gauss_1m_device()
    sel = np.array_split(rows, G1M_PARTS)[part]
    _announce("gauss_sum_1m rows", part=part, count=sel.size)
    want, norm = oracle.gauss_sum(inp["x"][sel], inp["y"], inp["b"], float(inp["sigma"]), workers=WORKERS)
    assert_normalised(got[sel], want, norm, TOL_F32, "gauss_sum_1m")


def test_gauss_sum_workload_1m_with_outliers():
    """The 1M x 1M workload with one far row and one far column (a point near (1000, 1000,
    1000) on each side): they are set aside and the rest stays on the matrix cores. Checked on
    1,024 seeded rows, the first and last 64 and the far row, against all columns."""
    import pairwise_reductions_amd as pr
    inp = workloads.make_inputs("gauss_sum_1m")
    x, y = inp["x"].copy(), inp["y"].copy()
    x[123_457] = 1000.0
    y[876_543] = np.float32(1000.001)
    _announce("gauss_sum_1m_outliers", M=inp["M"], N=inp["N"])
    sig = float(inp["sigma"])
    got = _host(pr.gauss_sum(_dev(x), _dev(y), _dev(inp["b"]), sig))
    rows = np.union1d(workloads.sample_rows(inp["M"], 1024, seed=7), [123_457])
    want, norm = oracle.gauss_sum(x[rows], y, inp["b"], sig, workers=WORKERS)
    assert_normalised(got[rows], want, norm, TOL_F32, "gauss_sum_1m with outliers")
