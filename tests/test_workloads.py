"""Pins for the seeded input generator: measured gate density against its closed form."""
import numpy as np
import pytest
from scipy.special import ndtr

from activation_sparse_feedforward_amd import workloads as W
from oracle import twell_oracle as O


def _expected_density(inp):
    """Closed form given the drawn (rounded) inputs: g[t,j] = x0_t w0_j + sum_{k>=1} x_tk w_jk
    with x_tk ~ N(0,1) independent of the weights, so P(g > 0) = Phi(x0_t w0_j / ||w_j,1:||)."""
    x0 = inp["x"][:, 0].astype(np.float64)
    w = inp["w_gate_t"].astype(np.float64)
    s = np.sqrt(np.sum(w[:, 1:] ** 2, axis=1))
    return ndtr(np.outer(x0, w[:, 0] / s))


@pytest.mark.parametrize("cfg,kw", [
    (1, {}),
    (2, {"T": 256}),
    (3, {"T": 64}),
    (5, {"T": 64, "rho": 0.02}),
    (4, {"T": 512}),
])
def test_generator_density_within_5_sigma(cfg, kw):
    w = W.workload(cfg, **kw)
    inp = W.make_inputs(w)
    g = inp["x"].astype(np.float64) @ inp["w_gate_t"].astype(np.float64).T
    p = _expected_density(inp)
    nnz = int(np.count_nonzero(g > 0))
    mean, var = p.sum(), (p * (1 - p)).sum()
    assert abs(nnz - mean) <= 5 * np.sqrt(var) + 1, (nnz, mean, np.sqrt(var))
    # and the target density (before rounding) is what the recipe says
    if w.density == "uniform":
        assert abs(mean / p.size - w.rho) < 0.03 * w.rho


def test_generator_is_deterministic_and_rounded():
    w = W.workload(2, T=16)
    a, b = W.make_inputs(w), W.make_inputs(w)
    for k in ("x", "w_gate_t", "w_up_t", "w_down"):
        np.testing.assert_array_equal(a[k], b[k])
        np.testing.assert_array_equal(W.bf16_bits_to_f32(a[k + "_raw"]), a[k])
        np.testing.assert_array_equal(O.round_to_storage(a[k], "bf16"), a[k].astype(np.float64))
    # a smaller T is a prefix of the larger draw for x
    big = W.make_inputs(W.workload(2, T=32))
    np.testing.assert_array_equal(big["x"][:16, 1:], a["x"][:, 1:])


def test_lognormal_tail_recipe():
    w = W.workload(4, T=20000)
    rho = W.row_densities(w)
    tail = rho >= 0.05
    assert 0.015 < tail.mean() < 0.025
    assert abs(np.median(rho[~tail]) - 0.005) < 0.0005
