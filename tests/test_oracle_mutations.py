"""Plant plausible mistakes in a copy of the oracle and check that a pin catches each one.

Each mutation replaces one exact snippet of oracle/reductions.py in a private copy that is
executed as a separate module; the real oracle is untouched.
"""
import os
import types

import pytest

import oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "reductions.py")

MUTATIONS = [
    # (name, original snippet, mutated snippet, pin group)
    ("dropped factor 2 in 2 sigma^2", "two_sigma2 = 2.0 * float(sigma) * float(sigma)\n    absb",
     "two_sigma2 = float(sigma) * float(sigma)\n    absb", pins.GAUSS_CHECKS),
    ("wrong exponent sign", "k = np.exp(-d2 / two_sigma2)", "k = np.exp(d2 / two_sigma2)", pins.GAUSS_CHECKS),
    ("wrong coordinate index", "diff = xr[:, d][:, None] - y[:, d][None, :]",
     "diff = xr[:, d][:, None] - y[:, 0][None, :]", pins.GAUSS_CHECKS),
    ("difference not squared", "d2 += diff * diff", "d2 += np.abs(diff)", pins.GAUSS_CHECKS),
    ("sum instead of difference", "diff = xr[:, d][:, None] - y[:, d][None, :]",
     "diff = xr[:, d][:, None] + y[:, d][None, :]", pins.GAUSS_CHECKS),
    ("weights replaced by |b|", "s[sl] = k @ b", "s[sl] = k @ absb", pins.GAUSS_CHECKS),
    ("batched: tau instead of tau/2", "half_tau = 0.5 * float(tau)", "half_tau = float(tau)", pins.BATCHED_CHECKS),
    ("batched: weights of another batch", "kt, vt, absv = k[t], v[t], np.abs(v[t])",
     "kt, vt, absv = k[t], v[0], np.abs(v[t])", pins.BATCHED_CHECKS),
    ("lse: dropped max term", "out[sl] = m + np.log(", "out[sl] = np.log(", pins.LSE_CHECKS),
    ("lse: max shift not subtracted", "np.exp(f - m[:, None])", "np.exp(f)", pins.LSE_CHECKS),
    ("lse: sigma^2 instead of 2 sigma^2",
     "two_sigma2 = 2.0 * float(sigma) * float(sigma)\n\n    def block(sl):\n        f =",
     "two_sigma2 = float(sigma) * float(sigma)\n\n    def block(sl):\n        f =", pins.LSE_CHECKS),
    ("argkmin: descending order", 'order = np.argsort(d2, axis=1, kind="stable")[:, :K]',
     'order = np.argsort(-d2, axis=1, kind="stable")[:, :K]', pins.ARGK_CHECKS),
    ("argkmin: ties to the higher index", 'order = np.argsort(d2, axis=1, kind="stable")[:, :K]',
     'order = (d2.shape[1] - 1 - np.argsort(d2[:, ::-1], axis=1, kind="stable"))[:, :K]', pins.ARGK_CHECKS),
    ("argkmin: off-by-one slice", 'order = np.argsort(d2, axis=1, kind="stable")[:, :K]',
     'order = np.argsort(d2, axis=1, kind="stable")[:, 1:K + 1]', pins.ARGK_CHECKS),
    ("grad: wrong sign", "grad[sl, d] = -term.sum(axis=1) / sigma2", "grad[sl, d] = term.sum(axis=1) / sigma2",
     pins.GRAD_CHECKS),
    ("grad: dropped upstream factor", "w = k * (g[sl] @ b.T)", "w = k * b.T.sum(axis=0)", pins.GRAD_CHECKS),
    ("grad: y - x instead of x - y", "diff = x[sl, d][:, None] - y[:, d][None, :]",
     "diff = y[:, d][None, :] - x[sl, d][:, None]", pins.GRAD_CHECKS),
    ("grad: missing 1/sigma^2", "grad[sl, d] = -term.sum(axis=1) / sigma2", "grad[sl, d] = -term.sum(axis=1)",
     pins.GRAD_CHECKS),
    ("grad_y: wrong sign", "grad[sl, d] = term.sum(axis=1) / sigma2", "grad[sl, d] = -term.sum(axis=1) / sigma2",
     pins.GRADYB_CHECKS),
    ("grad_y: transposed weights", "w = k * (b[sl] @ g.T)", "w = k * (b[sl] @ g.T).sum(axis=0)",
     pins.GRADYB_CHECKS),
    ("grad_b: |g| instead of g", "grad[sl] = k @ g", "grad[sl] = k @ absg", pins.GRADYB_CHECKS),
    ("grad_b: sigma^2 instead of 2 sigma^2",
     "two_sigma2 = 2.0 * float(sigma) * float(sigma)\n    absg",
     "two_sigma2 = float(sigma) * float(sigma)\n    absg", pins.GRADYB_CHECKS),
    ("scaled: column scale added, not multiplied", "b = _f64(col_scale)[:, None] * b",
     "b = _f64(col_scale)[:, None] + b", pins.SCALED_CHECKS),
    ("scaled: row scale divides", "s = r * s", "s = s / r", pins.SCALED_CHECKS),
    ("diffusion: q^alpha instead of q^-alpha", "p = q ** (-float(alpha))", "p = q ** float(alpha)",
     pins.DIFFUSION_CHECKS),
    ("diffusion: left factor of d dropped", "d = p * gauss_sum(x, x, p, sigma, workers)[0][:, 0]",
     "d = gauss_sum(x, x, p, sigma, workers)[0][:, 0]", pins.DIFFUSION_CHECKS),
    ("diffusion: d^-1 instead of d^-1/2", "return p / np.sqrt(d), q, d", "return p / d, q, d", pins.DIFFUSION_CHECKS),
    ("batched backward: first batch's upstream gradient everywhere",
     'parts["x"].append(gauss_sum_grad_x(x[t], y[t], b[t], g[t], sigma, workers))',
     'parts["x"].append(gauss_sum_grad_x(x[t], y[t], b[t], g[0], sigma, workers))', pins.BATCHED_GRAD_CHECKS),
    ("weighted argkmin: weight added", "kk = squared_distances(x[sl], y) - w[None, :]",
     "kk = squared_distances(x[sl], y) + w[None, :]", pins.WARGK_CHECKS),
    ("weighted argkmin: unstable sort", 'order = np.argsort(kk, axis=1, kind="stable")[:, :K]',
     'order = (kk.shape[1] - 1 - np.argsort(kk[:, ::-1], axis=1, kind="stable"))[:, :K]', pins.WARGK_CHECKS),
]


def _mutated_module(orig, new):
    with open(SRC) as f:
        text = f.read()
    assert text.count(orig) == 1, f"snippet must occur exactly once: {orig!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(text.replace(orig, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,orig,new,checks", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(name, orig, new, checks):
    mutant = _mutated_module(orig, new)
    caught = []
    for check in checks:
        try:
            check(mutant)
        except Exception as exc:  # an assertion or a crash both count as caught
            caught.append((check.__name__, type(exc).__name__))
    assert caught, f"no pin caught the planted mistake: {name}"
