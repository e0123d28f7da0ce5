"""The CPU oracle against its pins (closed forms, independent libraries, exact arithmetic)."""
import numpy as np
import pytest

import oracle
import oracle_pins as pins
from pairwise_reductions_amd import workloads


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(oracle)


def test_config_grid_keys_are_exact():
    """The argKmin workload draws points on the 2^-24 grid in [0,1)^3, so float64 squared
    distances are exact and the oracle's ranking is the true ranking."""
    inp = workloads.make_inputs("argkmin_lse_100k", M=2000, N=3000)
    assert oracle.keys_are_exact(inp["x"], inp["y"])


def test_parallel_equals_serial():
    inp = workloads.make_inputs("gauss_sum_10k", M=700, N=9000)
    s1, n1 = oracle.gauss_sum(inp["x"], inp["y"], inp["b"], float(inp["sigma"]))
    s2, n2 = oracle.gauss_sum(inp["x"], inp["y"], inp["b"], float(inp["sigma"]), workers=4)
    assert np.array_equal(s1, s2) and np.array_equal(n1, n2)


def test_workload_generators_are_deterministic():
    a = workloads.make_inputs("gauss_sum_grad_x_100k_mixture", M=100, N=120)
    b = workloads.make_inputs("gauss_sum_grad_x_100k_mixture", M=100, N=120)
    for key in ("x", "y", "b"):
        assert a[key].dtype == np.float32 and np.array_equal(a[key], b[key])
    c = workloads.make_inputs("batched_gauss_sum_fp16", M=64, N=80)
    assert c["x"].shape == (4, 64, 32) and c["x"].dtype == np.float16
    assert c["b"].shape == (4, 80, 32)
    u = workloads.make_inputs("gauss_sum_1m", M=1000, N=1000)
    assert np.all((u["x"] >= 0) & (u["x"] < 1))
    assert np.all(u["x"].astype(np.float64) * 2 ** 24 == np.round(u["x"].astype(np.float64) * 2 ** 24))
