"""Pins of the comparison every parity test goes through.

oracle.relative_frobenius(x, ref) = ||x - ref||_F / ||ref||_F is the
relative Frobenius difference the EMA-Gram page reports between two update
directions (marin.community, "Sharding EMA-Gram eigensolves", section
"Results").  Each value below is worked out by hand from small integer
matrices, not by calling a norm routine, so a checker that returns 0, drops
the square root, divides by the wrong norm or ignores the sign of the
difference fails here.  The shared parity helpers (tests/parity.py) are
then fed planted wrong results and must reject every one.
"""

import numpy as np
import pytest

import oracle
import parity


# ------------------------------------------------------ hand-computed values
def test_double_of_reference_is_one():
    """||2A - A|| / ||A|| = 1 exactly."""
    A = np.array([[1.0, -2.0], [3.0, 4.0]])
    assert oracle.relative_frobenius(2.0 * A, A) == 1.0


def test_known_difference():
    """A = diag(3, 4): ||A||_F = 5.  E has one entry 1: ||E||_F = 1, so the
    ratio is 1/5; E' = [[0, 3], [4, 0]] (||E'||_F = 5) gives 1."""
    A = np.diag([3.0, 4.0])
    E = np.array([[0.0, 1.0], [0.0, 0.0]])
    assert oracle.relative_frobenius(A + E, A) == pytest.approx(0.2, rel=1e-15)
    assert oracle.relative_frobenius(A - E, A) == pytest.approx(0.2, rel=1e-15)
    E2 = np.array([[0.0, 3.0], [4.0, 0.0]])
    assert oracle.relative_frobenius(A + E2, A) == pytest.approx(1.0, rel=1e-15)


def test_square_root_of_sum_of_squares():
    """Difference entries (1, 2, 2) over a reference with entries (2, 4, 4):
    sqrt(9)/sqrt(36) = 1/2 (a checker without the square root gives 1/4)."""
    ref = np.array([[2.0, 4.0, 4.0]])
    x = ref + np.array([[1.0, 2.0, -2.0]])
    assert oracle.relative_frobenius(x, ref) == pytest.approx(0.5, rel=1e-15)


def test_denominator_is_the_reference():
    """x = [[0, 0]], ref = [[3, 4]]: ||x - ref|| = 5, ||ref|| = 5 -> 1; with
    the arguments swapped the reference is zero and the value is ||x|| = 5."""
    x = np.zeros((1, 2))
    ref = np.array([[3.0, 4.0]])
    assert oracle.relative_frobenius(x, ref) == pytest.approx(1.0, rel=1e-15)
    assert oracle.relative_frobenius(ref, x) == pytest.approx(5.0, rel=1e-15)


def test_zero_reference_branch():
    """A zero reference gives the absolute norm of x: 0 for x = 0, 13 for
    x with entries (5, 12)."""
    z = np.zeros((2, 2))
    assert oracle.relative_frobenius(z, z) == 0.0
    assert oracle.relative_frobenius(np.array([[5.0, 0.0], [0.0, 12.0]]), z) == pytest.approx(13.0, rel=1e-15)


def test_scale_invariance():
    """Scaling both arguments by a power of two leaves the value unchanged
    bit for bit; scaling only x moves it."""
    rng = np.random.default_rng(11)
    ref = rng.standard_normal((7, 5))
    x = ref + 1e-3 * rng.standard_normal((7, 5))
    e = oracle.relative_frobenius(x, ref)
    assert oracle.relative_frobenius(2.0 ** 40 * x, 2.0 ** 40 * ref) == e
    assert oracle.relative_frobenius(2.0 ** -40 * x, 2.0 ** -40 * ref) == e
    assert oracle.relative_frobenius(2.0 * x, ref) > 0.9


def test_values_that_must_be_rejected():
    """Relative perturbations of 2e-4 and 2e-3 exceed the root (1e-4) and
    update (1e-3) tolerances; 5e-5 and 5e-4 pass them."""
    ref = np.arange(1.0, 13.0).reshape(3, 4)
    assert oracle.relative_frobenius(ref * (1 + 2e-4), ref) == pytest.approx(2e-4, rel=1e-9)
    assert not oracle.relative_frobenius(ref * (1 + 2e-4), ref) <= parity.ROOT_TOL
    assert not oracle.relative_frobenius(ref * (1 + 2e-3), ref) <= parity.UPDATE_TOL
    assert oracle.relative_frobenius(ref * (1 + 5e-5), ref) <= parity.ROOT_TOL
    assert oracle.relative_frobenius(ref * (1 + 5e-4), ref) <= parity.UPDATE_TOL


def test_nan_is_never_within_tolerance():
    """A NaN anywhere in x gives a NaN difference, which no tolerance accepts."""
    ref = np.eye(3)
    x = np.eye(3)
    x[1, 2] = np.nan
    assert not oracle.relative_frobenius(x, ref) <= 1.0


# ------------------------------------------ planted results in the helpers
def _toy_reference():
    """The oracle's step 3 on a seeded 24 x 40 weight: roots, update, state."""
    rng = np.random.default_rng(12)
    grads = [rng.standard_normal((24, 40)).astype(np.float32) for _ in range(3)]
    *_, last = oracle.run_sequence(grads, 0.95, 1e-6)
    _, L, R, XL, XR, U, flags = last
    assert flags == 0
    return L, R, XL, XR, U


def test_helpers_accept_float32_rounding_of_the_reference():
    L, R, XL, XR, U = _toy_reference()
    parity.assert_root(XL.astype(np.float32), XL, "XL")
    parity.assert_root(XR.astype(np.float32), XR, "XR")
    parity.assert_update(U.astype(np.float32), U, "U")
    parity.assert_state(L.copy(), L, 1e-12, "L")


PLANTED_ROOTS = {
    # a root within tolerance that is not exactly symmetric
    "asymmetric": lambda X: X + np.where(np.arange(X.size).reshape(X.shape) == 1, 1e-5 * np.abs(X).max(), 0),
    "power -1/2 instead of -1/4": lambda X: np.linalg.matrix_power(X, 2),
    "one entry off by 1e-3": lambda X: X + np.where(np.arange(X.size).reshape(X.shape) == 5, 1e-3 * np.abs(X).max(), 0),
    "scaled by 1 + 2e-4": lambda X: X * (1 + 2e-4),
    "identity": lambda X: np.eye(X.shape[0]),
    "a NaN": lambda X: np.where(np.arange(X.size).reshape(X.shape) == 0, np.nan, X),
}


@pytest.mark.parametrize("name", sorted(PLANTED_ROOTS))
def test_assert_root_rejects(name):
    _, _, XL, XR, _ = _toy_reference()
    for X in (XL, XR):
        bad = PLANTED_ROOTS[name](X.copy()).astype(np.float32)
        with pytest.raises(AssertionError):
            parity.assert_root(bad, X, name)


def test_assert_update_rejects_planted_results():
    L, R, XL, XR, U = _toy_reference()
    G = np.linalg.solve(XL, np.linalg.solve(XR.T, U.T).T)  # the gradient behind U
    planted = {
        "powers +1/4 instead of -1/4": np.linalg.inv(XL) @ G @ np.linalg.inv(XR),
        "powers -1/2 instead of -1/4": XL @ XL @ G @ XR @ XR,
        "left root only": XL @ G,
        "right root only": G @ XR,
        "gradient itself": G,
        "sign flip": -U,
        "scaled by 1 + 2e-3": U * (1 + 2e-3),
        "zero": np.zeros_like(U),
    }
    for name, bad in planted.items():
        with pytest.raises(AssertionError):
            parity.assert_update(bad.astype(np.float32), U, name)


def test_assert_state_rejects_planted_results():
    L, R, *_ = _toy_reference()
    planted = {
        "float32 rounding at the float64 tolerance": L.astype(np.float32).astype(np.float64),
        "asymmetric": L + np.triu(np.full_like(L, 1e-12 * np.abs(L).max()), 1),
        "beta and 1 - beta swapped": L * 19.0,
    }
    for name, bad in planted.items():
        with pytest.raises(AssertionError):
            parity.assert_state(bad, L, 1e-12, name)
