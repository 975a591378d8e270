"""Planted mistakes in the oracle, each of which the oracle's pins must catch.

Every mutation below replaces one oracle function, for the duration of one
test, with a version carrying a plausible mistake: swapped EMA weights, a
dropped factor, the wrong power, the regulariser added before the rescale,
a transposed reconstruction, a one-sided apply, another normalisation, an
unsymmetrised input, or a broken comparison.  The pins of
test_oracle_pins.py and test_oracle_checker_pins.py then run against the
mutated oracle, and at least one of them has to fail.  All of this is on the
CPU and touches nothing outside the oracle module's namespace.
"""

import numpy as np
import pytest

import oracle
import oracle.step as step
import test_oracle_checker_pins as CP
import test_oracle_pins as P

_orig_root = step.inv_quarter_root
_orig_gram_ema = step.gram_ema_update
_orig_apply = step.precondition_apply
_orig_rf = step.relative_frobenius


def _ema_swapped(L, R, G, beta):
    # beta on the new Gram, 1 - beta on the old state
    return _orig_gram_ema(L, R, G, 1.0 - beta)


def _ema_no_weight(L, R, G, beta):
    # old state decayed, new Gram added without its (1 - beta) factor
    b = float(beta)
    return b * np.asarray(L, float) + step.left_gram(G), b * np.asarray(R, float) + step.right_gram(G)


def _root_power_half(A, eps, normalize="trace"):
    X, info = _orig_root(A, eps, normalize)
    return X @ X, info


def _root_eps_before_rescale(A, eps, normalize="trace"):
    # (A + eps I) / s instead of A / s + eps I
    if normalize == "trace":
        tr = float(np.trace(np.asarray(A, float)))
        if tr != 0.0 and np.isfinite(tr):
            return _orig_root(A, eps / tr, normalize)
    return _orig_root(A, eps, normalize)


def _root_transposed_reconstruction(A, eps, normalize="trace"):
    X, info = _orig_root(A, eps, normalize)
    if info["flags"]:
        return X, info
    Ahat, _ = step.rescale(0.5 * (np.asarray(A, float) + np.asarray(A, float).T), normalize)
    w, V = np.linalg.eigh(Ahat)
    return (V.T * (w + eps) ** -0.25) @ V, info


def _root_frobenius_normalised(A, eps, normalize="trace"):
    if normalize == "trace":
        A = np.asarray(A, float)
        nf = float(np.linalg.norm(A))
        if nf > 0.0 and np.isfinite(nf):
            X, info = _orig_root(A / nf, eps, "none")
            info = dict(info, scale=nf)
            return X, info
    return _orig_root(A, eps, normalize)


def _root_unsymmetrised(A, eps, normalize="trace"):
    # eigh reads only one triangle: feeding it the raw lower triangle
    A = np.asarray(A, float)
    low = np.tril(A) + np.tril(A, -1).T
    return _orig_root(low, eps, normalize)


def _apply_left_only(XL, G, XR, alpha=1.0):
    return float(alpha) * (np.asarray(XL, float) @ np.asarray(G, float))


def _rf_zero(x, ref):
    return 0.0


def _rf_squared(x, ref):
    return _orig_rf(x, ref) ** 2


def _rf_wrong_denominator(x, ref):
    x = np.asarray(x, float)
    den = np.linalg.norm(x)
    return float(np.linalg.norm(x - np.asarray(ref, float)) / den) if den else 0.0


MUTATIONS = {
    "EMA weights swapped": ("gram_ema_update", _ema_swapped),
    "EMA without the (1 - beta) factor": ("gram_ema_update", _ema_no_weight),
    "power -1/2 instead of -1/4": ("inv_quarter_root", _root_power_half),
    "eps added before the rescale": ("inv_quarter_root", _root_eps_before_rescale),
    "transposed reconstruction V^T f V": ("inv_quarter_root", _root_transposed_reconstruction),
    "Frobenius normalisation instead of trace": ("inv_quarter_root", _root_frobenius_normalised),
    "input not symmetrised": ("inv_quarter_root", _root_unsymmetrised),
    "apply drops the right root": ("precondition_apply", _apply_left_only),
    "comparison returns 0": ("relative_frobenius", _rf_zero),
    "comparison squared": ("relative_frobenius", _rf_squared),
    "comparison divides by ||x||": ("relative_frobenius", _rf_wrong_denominator),
}

# The pins, with fixed arguments (the slow 50-digit whole-step pin is left out).
PINS = [
    P.test_gram_products_by_loops,
    P.test_ema_weights_by_loops,
    lambda: P.test_diagonal_closed_form_multistep(4, 6),
    lambda: P.test_2x2_closed_form(3.0, 1.0, 2.0, 1e-6),
    lambda: P.test_2x2_closed_form(0.1, -0.4, 2.5, 1e-2),
    lambda: P.test_4x4_root_bruteforce_mpmath(0),
    lambda: P.test_step1_svd_form(6, 9, 0.95),
    P.test_inverse_root_invariants,
    P.test_second_method_coupled_newton_fp64,
    P.test_permutation_equivariance,
    P.test_input_symmetric_part,
    P.test_flags,
    CP.test_double_of_reference_is_one,
    CP.test_known_difference,
    CP.test_square_root_of_sum_of_squares,
    CP.test_denominator_is_the_reference,
    CP.test_values_that_must_be_rejected,
]


def _failing_pins():
    failed = 0
    for pin in PINS:
        try:
            pin()
        except Exception:  # an assertion, or a shape error from a wrong operand
            failed += 1
    return failed


def test_pins_pass_on_the_oracle_as_written():
    assert _failing_pins() == 0


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_fails_a_pin(monkeypatch, name):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(step, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    assert _failing_pins() >= 1, f"no pin catches: {name}"
