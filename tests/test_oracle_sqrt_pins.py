"""Pins of the oracle's inverse square root W = (Â + eps I)^(-1/2) (the root
tilderesearch, "Online KL Shampoo", computes by its scaled CANS coupled
iteration, sections 2.2-2.4 and appendix D) against things other than
itself: closed forms, 50-digit brute force, the inverse-root equation, a
second fp64 method written here, and the page's printed CANS table (its
coefficients reproduce its printed ceilings and reach S^(-1/2) through the
scalar recurrence the iteration applies to every eigenvalue)."""

import json
import os

import mpmath
import numpy as np
import pytest

import oracle
from matrix_roots_amd import workloads

HERE = os.path.dirname(os.path.abspath(__file__))


def _cans_table():
    with open(os.path.join(HERE, "golden", "okls_cans_table.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("a,b,c,eps", [(3.0, 1.0, 2.0, 1e-6), (0.1, -0.4, 2.5, 1e-2),
                                       (1.0, 0.0, 4.0, 0.0), (2.0, 1.9, 2.0, 1e-8)])
def test_2x2_closed_form(a, b, c, eps):
    """W = sum_k (l_k + eps)^(-1/2) P_k with the spectral projectors of [[a,b],[b,c]]."""
    A = np.array([[a, b], [b, c]])
    mid, rad = (a + c) / 2.0, np.hypot((a - c) / 2.0, b)
    lp, lm = mid + rad, mid - rad
    I = np.eye(2)
    if rad == 0.0:
        Wexp = (lp + eps) ** -0.5 * I
    else:
        Pp = (A - lm * I) / (lp - lm)
        Pm = (A - lp * I) / (lm - lp)
        Wexp = (lp + eps) ** -0.5 * Pp + (lm + eps) ** -0.5 * Pm
    W, info = oracle.inv_sqrt_root(A, eps, normalize="none")
    assert info["flags"] == 0
    np.testing.assert_allclose(W, Wexp, rtol=1e-13, atol=1e-14)


def test_diagonal_closed_form():
    a = np.array([4.0, 1.0, 0.25, 9.0, 0.0])
    for normalize, s in (("none", 1.0), ("trace", a.sum())):
        W, info = oracle.inv_sqrt_root(np.diag(a), 1e-3, normalize)
        np.testing.assert_allclose(W, np.diag((a / s + 1e-3) ** -0.5), rtol=1e-14, atol=0)
        assert info["scale"] == pytest.approx(s, rel=1e-15)


def _mp_isqrt(A, eps):
    mpmath.mp.dps = 50
    d = A.shape[0]
    M = mpmath.matrix([[mpmath.mpf(float(A[i, j])) for j in range(d)] for i in range(d)])
    E, Q = mpmath.mp.eigsy(M)
    f = [(E[k] + mpmath.mpf(eps)) ** mpmath.mpf(-0.5) for k in range(d)]
    return np.array([[float(sum(Q[i, k] * f[k] * Q[j, k] for k in range(d))) for j in range(d)]
                     for i in range(d)])


@pytest.mark.parametrize("seed", [0, 1])
def test_4x4_bruteforce_mpmath(seed):
    rng = np.random.default_rng(20 + seed)
    B = rng.standard_normal((4, 4))
    A = B @ B.T + np.diag([0.0, 0.0, 1e-3, 0.0])
    for eps in (1e-6, 1e-2):
        W, _ = oracle.inv_sqrt_root(A, eps, "none")
        assert oracle.relative_frobenius(W, _mp_isqrt(A, eps)) < 1e-13


def test_inverse_root_equation_and_quarter_root_square():
    rng = workloads.rng_for(98, 0)
    A = workloads.spd_loguniform(40, rng, -4.0, 0.0).astype(np.float64)
    for normalize in ("none", "trace"):
        for eps in (0.0, 1e-6, 1e-2):
            W, info = oracle.inv_sqrt_root(A, eps, normalize)
            S = A / info["scale"] + eps * np.eye(40)
            assert np.array_equal(W, W.T)
            assert np.linalg.norm(W @ S @ W - np.eye(40)) < 1e-9
            if eps > 0.0:
                X, _ = oracle.inv_quarter_root(A, eps, normalize)
                assert oracle.relative_frobenius(W, X @ X) < 1e-12


def _coupled_ns(S, iters=80):
    """Classical coupled Newton-Schulz for S^(-1/2) in fp64 (Y -> S^(1/2)/sqrt(c),
    Z -> (S/c)^(-1/2) with Q = (3I - ZY)/2), from Y = S/c, Z = I,
    c = ||S||_F; written here, independent of the HIP path."""
    d = S.shape[0]
    c = np.linalg.norm(S)
    Y, Z, I = S / c, np.eye(d), np.eye(d)
    for _ in range(iters):
        Q = 0.5 * (3.0 * I - Z @ Y)
        Y, Z = Y @ Q, Q @ Z
    return Z / np.sqrt(c)


def test_second_method_coupled_newton_schulz():
    rng = workloads.rng_for(97, 0)
    A = workloads.spd_loguniform(48, rng, -3.0, 0.0).astype(np.float64)
    for eps in (0.0, 1e-4):
        W, _ = oracle.inv_sqrt_root(A, eps, "none")
        assert oracle.relative_frobenius(W, _coupled_ns(A + eps * np.eye(48))) < 1e-9


def test_flags():
    d = 6
    W, info = oracle.inv_sqrt_root(np.zeros((d, d)), 1e-4, "trace")
    assert info["flags"] == oracle.FLAG_ZERO_TRACE
    np.testing.assert_array_equal(W, 100.0 * np.eye(d))
    A = np.diag([1.0, 2.0, -0.5, 1.0, 1.0, 1.0])
    W, info = oracle.inv_sqrt_root(A, 1e-2, "none")
    assert info["flags"] == oracle.FLAG_NOT_PD and np.isnan(W).all()
    B = np.eye(d)
    B[1, 2] = np.inf
    W, info = oracle.inv_sqrt_root(B, 1e-2, "none")
    assert info["flags"] == oracle.FLAG_NONFINITE and np.isnan(W).all()


# ------------------------------------------------- the page's CANS table
def _scalar_run(y0, coeffs):
    y, z = np.array(y0, dtype=np.float64), np.ones_like(y0, dtype=np.float64)
    ys, zs, ps = [y.copy()], [z.copy()], []
    for a, b in coeffs:
        p = z * y
        ps.append(p)
        q = a + b * p
        y, z = y * q, z * q
        ys.append(y.copy())
        zs.append(z.copy())
    ps.append(z * y)
    return ys, zs, ps


def test_cans_table_reproduces_printed_ceilings():
    """Suprema over y0 in (0, 1] of z_k and p_k = z_k y_k equal the page's
    printed Z ceilings (five digits) and P ceilings (three digits, printed
    truncated: 1.15 for a supremum of 1.1595); the printed Y ceilings bound
    y_k.  A mistyped coefficient moves these."""
    t = _cans_table()
    y0 = np.concatenate([np.logspace(-14, 0, 100001), np.linspace(0.0, 1.0, 100001)[1:]])
    ys, zs, ps = _scalar_run(y0, t["coefficients"])
    for k in range(t["steps"] + 1):
        assert zs[k].max() == pytest.approx(t["z_ceilings"][k], rel=2e-4), k
        assert ps[k].max() == pytest.approx(t["p_ceilings"][k], rel=1e-2), k
        assert ys[k].max() <= t["y_ceilings"][k] * 1.005, k


def test_cans_composed_map_reaches_inverse_sqrt():
    """After the ten steps z_10(y0) * sqrt(y0) = 1 to within 3e-5 on
    [1e-6, 0.99] (the range the page's figures use), and fails far below it."""
    t = _cans_table()
    y0 = np.logspace(-6, np.log10(0.99), 20001)
    _, zs, _ = _scalar_run(y0, t["coefficients"])
    err = np.abs(zs[-1] * np.sqrt(y0) - 1.0)
    assert err.max() < 3e-5, err.max()
    _, zlow, _ = _scalar_run(np.array([1e-9]), t["coefficients"])
    assert abs(zlow[-1][0] * np.sqrt(1e-9) - 1.0) > 0.5
