"""Comparisons shared by the parity tests (HIP path against the fp64 oracle).

Tolerances: relative Frobenius error <= 1e-4 on every root and <= 1e-3 on
every update direction, the comparison the EMA-Gram page uses between update
directions (marin.community, "Sharding EMA-Gram eigensolves", section
"Results").  Roots and Gram states must also be exactly symmetric and
finite.  Each helper raises AssertionError with the context on failure; the
CPU suite feeds them planted wrong results.
"""

import numpy as np

import oracle

ROOT_TOL = 1e-4
UPDATE_TOL = 1e-3


def _host(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.asarray(a, dtype=np.float64)


def assert_close(got, ref, tol, ctx=""):
    """relative_frobenius(got, ref) <= tol with every element finite; returns the error."""
    g = _host(got)
    assert g.shape == np.shape(ref), (ctx, g.shape, np.shape(ref))
    assert np.isfinite(g).all(), f"{ctx}: non-finite elements"
    err = oracle.relative_frobenius(g, ref)
    assert err <= tol, (ctx, err, tol)
    return err


def assert_symmetric(got, ctx=""):
    g = _host(got)
    assert np.array_equal(g, g.T), f"{ctx}: not exactly symmetric"


def assert_root(got, ref, ctx="", tol=ROOT_TOL):
    """An inverse root: exactly symmetric, finite, within tol of the oracle."""
    assert_symmetric(got, ctx)
    return assert_close(got, ref, tol, ctx)


def assert_update(got, ref, ctx="", tol=UPDATE_TOL):
    """An update direction: finite, within tol of the oracle."""
    return assert_close(got, ref, tol, ctx)


def assert_state(got, ref, tol, ctx=""):
    """A Gram state: exactly symmetric, finite, within tol of the oracle."""
    assert_symmetric(got, ctx)
    return assert_close(got, ref, tol, ctx)
