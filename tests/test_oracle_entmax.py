"""Pins of the oracle's alpha-entmax against what the pages and the mathematics fix.

DashAttention paper (arXiv 2605.18753v1): §2 Eq. 2 (thresholded form, sparsemax at alpha = 2,
softmax as alpha -> 1, sparsity rising with alpha) and App. A Eq. 11-13 (variational form with
the Tsallis entropy, threshold by sort for alpha in {1.5, 2} or by bisection).
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.optimize import minimize

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def tsallis_objective(p, z, alpha):
    """p^T z + H_alpha(p), the variational form of alpha-entmax (App. A, Eq. 11-12)."""
    return float(p @ z + (np.sum(p - p ** alpha)) / (alpha * (alpha - 1.0)))


def entmax_by_optimizer(z, alpha):
    """argmax over the simplex of p^T z + H_alpha(p), by a general constrained optimizer."""
    m = z.size
    cons = ({"type": "eq", "fun": lambda p: np.sum(p) - 1.0, "jac": lambda p: np.ones(m)},)
    best = None
    for start in (np.full(m, 1.0 / m), np.eye(m)[int(np.argmax(z))] * 0.9 + 0.1 / m):
        res = minimize(lambda p: -tsallis_objective(np.clip(p, 0, None), z, alpha), start,
                       method="SLSQP", bounds=[(0.0, 1.0)] * m, constraints=cons,
                       options=dict(ftol=1e-15, maxiter=2000))
        p = np.clip(res.x, 0, None)
        p /= p.sum()
        if best is None or tsallis_objective(p, z, alpha) > tsallis_objective(best, z, alpha):
            best = p
    return best


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
@pytest.mark.parametrize("seed", range(4))
def test_entmax_is_the_variational_argmax(orc, alpha, seed):
    """Eq. 13 (threshold form) must solve Eq. 11 (max of p^T z + Tsallis entropy)."""
    rng = np.random.default_rng(100 + seed)
    z = rng.normal(size=7) * rng.uniform(0.5, 4.0)
    p = orc.entmax((alpha - 1.0) * z, alpha)
    q = entmax_by_optimizer(z, alpha)
    # the oracle's point is at least as good as anything the optimizer finds ...
    assert tsallis_objective(p, z, alpha) >= tsallis_objective(q, z, alpha) - 1e-10
    # ... and it is the same point (the objective is strictly concave)
    assert np.max(np.abs(p - q)) < 2e-4


def test_sparsemax_textbook_example(orc):
    """alpha = 2 is sparsemax: the Euclidean projection of z onto the simplex (App. A).
    For z = (1, 0.5, 0) the projection is (0.75, 0.25, 0): with support {1, 2},
    tau = (1 + 0.5 - 1) / 2 = 0.25 and 0 <= tau."""
    p = orc.entmax(np.array([1.0, 0.5, 0.0]), 2.0)
    np.testing.assert_allclose(p, [0.75, 0.25, 0.0], atol=1e-15)


@pytest.mark.parametrize("seed", range(5))
def test_sparsemax_is_euclidean_projection(orc, seed):
    """Brute force over every support set of a small vector: the projection onto the simplex is
    the feasible candidate (z_S - t, t fixed by the sum) closest to z."""
    rng = np.random.default_rng(seed)
    z = rng.normal(size=6) * 0.7
    best, best_d = None, math.inf
    m = z.size
    for mask in range(1, 1 << m):
        s = [i for i in range(m) if mask >> i & 1]
        t = (z[s].sum() - 1.0) / len(s)
        p = np.zeros(m)
        p[s] = z[s] - t
        if np.all(p >= -1e-15):
            d = np.sum((p - z) ** 2)
            if d < best_d:
                best, best_d = p, d
    np.testing.assert_allclose(orc.entmax(z, 2.0), best, atol=1e-12)


def test_two_element_entmax15_closed_form(orc):
    """alpha = 1.5 with two entries a > b and a - b < 1: both stay in the support and
    (a - tau)^2 + (b - tau)^2 = 1 gives a - tau = (delta + sqrt(2 - delta^2)) / 2."""
    for a, b in [(0.3, 0.1), (0.0, -0.9), (2.0, 2.0)]:
        delta = a - b
        s = (delta + math.sqrt(2 - delta * delta)) / 2
        p = orc.entmax(np.array([a, b]), 1.5)
        np.testing.assert_allclose(p, [s * s, (s - delta) ** 2], atol=1e-13)
    # a gap of at least 1 leaves only the larger entry
    np.testing.assert_allclose(orc.entmax(np.array([1.5, 0.5]), 1.5), [1.0, 0.0], atol=0)


def test_softmax_limit(orc):
    """alpha -> 1 recovers softmax (Eq. 2 and App. A 'Special cases')."""
    rng = np.random.default_rng(7)
    for _ in range(5):
        z = rng.normal(size=40) * 2.0
        eps = 1e-5
        p = orc.entmax(eps * z, 1.0 + eps)
        sm = np.exp(z - z.max())
        sm /= sm.sum()
        assert np.max(np.abs(p - sm)) <= 1e-4


@pytest.mark.parametrize("alpha", [1.25, 1.5, 2.0])
def test_normalisation_support_and_uniqueness(orc, alpha):
    """Sum of probabilities is 1; zero exactly where x <= tau (Eq. 2); sort and bisection agree."""
    rng = np.random.default_rng(11)
    for _ in range(20):
        m = int(rng.integers(1, 300))
        x = (alpha - 1.0) * rng.normal(size=m) * rng.uniform(0.1, 20.0)
        tau = orc.entmax_tau(x, alpha)
        p = orc.entmax(x, alpha)
        assert abs(p.sum() - 1.0) <= 1e-12
        np.testing.assert_array_equal(p > 0, x > tau)
        tb = orc.entmax_tau(x, alpha, method="bisect")
        assert abs(tau - tb) <= 1e-12
        # bracket [max - 1, max - m^(1 - alpha)]
        assert x.max() - 1.0 - 1e-15 <= tau <= x.max() - m ** (1.0 - alpha) + 1e-15


def test_sort_and_bisection_agree(orc):
    rng = np.random.default_rng(12)
    for alpha in (1.5, 2.0):
        for _ in range(50):
            x = rng.normal(size=int(rng.integers(1, 600))) * rng.uniform(0.01, 10.0)
            assert abs(orc.entmax_tau(x, alpha, "sort") - orc.entmax_tau(x, alpha, "bisect")) <= 1e-12


def test_sparsity_rises_with_alpha(orc):
    """Support size never grows as alpha increases on the same scores (§2)."""
    rng = np.random.default_rng(13)
    alphas = [1.05, 1.25, 1.5, 1.75, 2.0]
    for _ in range(30):
        z = rng.normal(size=64) * rng.uniform(0.5, 5.0)
        sizes = [int((orc.entmax((a - 1.0) * z, a) > 0).sum()) for a in alphas]
        assert all(s1 >= s2 for s1, s2 in zip(sizes, sizes[1:])), sizes


def test_golden_entmax_fixture(orc):
    """Closed-form values stored under tests/golden (each case cites its derivation)."""
    with open(os.path.join(GOLDEN, "entmax_closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        p = orc.entmax(np.array(c["x"]), c["alpha"])
        np.testing.assert_allclose(p, c["p"], atol=c["atol"], err_msg=c["why"])
