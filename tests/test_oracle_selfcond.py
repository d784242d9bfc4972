"""Pins of the self-conditioning oracle (oracle/selfcond.py)."""
import math

import numpy as np
import pytest

from oracle import selfcond as SC


def test_one_hot_row_selects_the_embedding_row():
    V, d = 64, 5
    rng = np.random.default_rng(1)
    E = rng.normal(size=(V, d))
    z = np.full((3, V), -1e6)
    targets = [0, 17, 63]
    for r, t in enumerate(targets):
        z[r, t] = 0.0
    assert np.array_equal(SC.self_condition(z, 0.8, E), E[targets])


def test_uniform_row_averages_the_embedding():
    V, d = 50, 4
    E = np.random.default_rng(2).normal(size=(V, d))
    s = SC.self_condition(np.zeros((2, V)), 0.4, E)
    assert np.allclose(s, E.mean(axis=0), rtol=1e-14, atol=1e-15)


def test_ones_column_is_total_probability():
    V = 300
    z = np.random.default_rng(3).normal(size=(4, V)) * 3
    s = SC.self_condition(z, 0.7, np.ones((V, 1)))
    assert np.allclose(s, 1.0, rtol=0, atol=1e-14)


def test_set_indicators_match_brute_force_probability_sums():
    # tiny case: probabilities summed by plain loops over exp(z/T)
    V, T = 7, 0.6
    z = np.array([[0.3, -1.2, 2.0, 0.0, 0.5, -0.7, 1.1]])
    sets = [{0, 2}, {1, 3, 5}, {6}, set(range(V))]
    E = np.array([[1.0 if v in S else 0.0 for S in sets] for v in range(V)])
    w = [math.exp(zv / T) for zv in z[0]]
    tot = sum(w)
    want = [sum(w[v] for v in S) / tot for S in sets]
    assert np.allclose(SC.self_condition(z, T, E)[0], want, rtol=1e-14, atol=0)


def test_index_column_gives_the_truncated_geometric_mean():
    # z_v = -a v: p(v) = (1 - q) q^v / (1 - q^V) with q = exp(-a/T); its mean
    # is q/(1-q) - V q^V / (1 - q^V)
    V, a, T = 1000, 0.05, 0.8
    q = math.exp(-a / T)
    mean = q / (1 - q) - V * q ** V / (1 - q ** V)
    z = -a * np.arange(V, dtype=np.float64)[None, :]
    got = SC.self_condition(z, T, np.arange(V, dtype=np.float64)[:, None])[0, 0]
    assert got == pytest.approx(mean, rel=1e-12)


def test_linear_in_the_embedding_and_invariant_to_logit_shifts():
    V, d = 40, 3
    rng = np.random.default_rng(5)
    z = rng.normal(size=(2, V))
    E1, E2 = rng.normal(size=(V, d)), rng.normal(size=(V, d))
    s = SC.self_condition(z, 0.5, 2 * E1 - E2)
    assert np.allclose(s, 2 * SC.self_condition(z, 0.5, E1) - SC.self_condition(z, 0.5, E2),
                       rtol=1e-12, atol=1e-13)
    assert np.allclose(SC.self_condition(z + 7.5, 0.5, E1), SC.self_condition(z, 0.5, E1),
                       rtol=1e-12, atol=1e-13)
    assert np.all(SC.magnitude(z, 0.5, E1) >= np.abs(SC.self_condition(z, 0.5, E1)) - 1e-15)
