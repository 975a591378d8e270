"""Pins of the oracle's momentum EMA and MuonH hyperball update
(ai.thesatyajit.com, "Marin 535B-A23B", section "A sphere for every matrix") by closed forms and
invariants, none of which retype the oracle's formulas."""

import numpy as np
import pytest

import oracle


def test_momentum_geometric_sum_and_edges():
    """From zero with a constant G, t steps give (1 - mu^t) G; mu = 0 copies G."""
    rng = np.random.default_rng(1)
    G = rng.standard_normal((5, 7))
    M = np.zeros_like(G)
    for t in range(1, 6):
        M = oracle.momentum_ema(M, G, 0.9)
        np.testing.assert_allclose(M, (1 - 0.9 ** t) * G, rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(oracle.momentum_ema(M, G, 0.0), G)


def test_norm_is_preserved():
    rng = np.random.default_rng(2)
    for lr in (1e-3, 0.05, 0.7, 3.0):
        W, U = rng.standard_normal((20, 12)), rng.standard_normal((20, 12))
        Wn, info = oracle.hyperball_update(W, U, lr)
        assert np.linalg.norm(Wn) == pytest.approx(np.linalg.norm(W), rel=1e-14)
        assert info["w_norm"] == pytest.approx(np.linalg.norm(W), rel=1e-15)


def test_parallel_and_orthogonal_updates():
    """U along W: W' = (1 - lr) W, rescaled back to W itself.  U orthogonal to
    W with ||U|| = ||W||: ||W'||^2 = (1 + lr^2) ||W||^2, so
    W_new = (W - lr U) / sqrt(1 + lr^2)."""
    W = np.array([[3.0, 0.0], [0.0, 4.0]])
    Wn, info = oracle.hyperball_update(W, 2.0 * W, 0.25)
    np.testing.assert_allclose(Wn, W, rtol=1e-15)
    assert info["new_norm"] == pytest.approx(0.75 * 5.0, rel=1e-15)
    U = np.array([[0.0, 4.0], [-3.0, 0.0]])  # <W, U> = 0, ||U|| = ||W|| = 5
    Wn, _ = oracle.hyperball_update(W, U, 0.5)
    np.testing.assert_allclose(Wn, (W - 0.5 * U) / np.sqrt(1.25), rtol=1e-15)
    # the step is lr times W's norm, whatever U's scale
    np.testing.assert_allclose(oracle.hyperball_update(W, 1e6 * U, 0.5)[0], Wn, rtol=1e-14)


def test_floors():
    """Zero update: nothing moves.  Zero weight: stays zero (the 1e-10 floors)."""
    W = np.arange(6.0).reshape(2, 3)
    np.testing.assert_array_equal(oracle.hyperball_update(W, np.zeros_like(W), 0.1)[0], W)
    Wn, info = oracle.hyperball_update(np.zeros((2, 3)), np.ones((2, 3)), 0.1)
    assert not Wn.any() and info["w_norm"] == 0.0
