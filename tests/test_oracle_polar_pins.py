"""Pins of the oracle's CANS polar orthogonalisation (U phi(Sigma/sqrt(L))
V^T, the ten CANS steps of tilderesearch, "Online KL Shampoo", section 2.3,
acting on singular values) against things other than itself: the direct
matrix iteration X <- a X + b X X^T X in fp64 written here, the SVD polar
factor for spectra in the polynomials' range, closed forms for diagonal and
rank-1 inputs, and invariances."""

import json
import os

import numpy as np
import pytest

import oracle
from matrix_roots_amd import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))


def _coeffs():
    with open(os.path.join(HERE, "golden", "okls_cans_table.json")) as f:
        return json.load(f)["coefficients"]


def _direct_iteration(G):
    """X0 = G / sqrt(1.01 ||G||_F^2); X <- a X + b X (X^T X), ten steps, fp64."""
    G = np.asarray(G, dtype=np.float64)
    X = G / np.sqrt(1.01 * np.sum(G * G))
    for a, b in _coeffs():
        X = a * X + b * (X @ (X.T @ X))
    return X


def test_coefficients_are_the_pages():
    assert [list(c) for c in oracle.step.CANS_COEFFS] == _coeffs()


@pytest.mark.parametrize("shape,kind", [((64, 48), "gaussian"), ((40, 90), "gaussian"), ((96, 96), "powerlaw"),
                                        ((128, 256), "lowrank32"), ((120, 60), "sparserows")])
def test_matches_direct_matrix_iteration(shape, kind):
    wl = {"gaussian": "toy", "powerlaw": "w2048", "lowrank32": "w1024", "sparserows": "moe"}[kind]
    G = W.gradient(wl, 3, 1, shape=shape).astype(np.float64)
    O, info = oracle.polar_cans(G)
    assert info["flags"] == 0
    assert oracle.relative_frobenius(O, _direct_iteration(G)) < 1e-10


def test_in_range_spectrum_gives_polar_factor():
    """Singular values with sigma^2/L in [1e-6, 1]: within 3e-5 of U V^T, and
    O^T O within 2 * 3e-5 of I on each of its n eigenvalues."""
    rng = np.random.default_rng(5)
    m, n = 80, 50
    U, _ = np.linalg.qr(rng.standard_normal((m, n)))
    V, _ = np.linalg.qr(rng.standard_normal((n, n)))
    sig = 10.0 ** rng.uniform(-2.0, 0.0, n)  # sigma^2 / L >= 1e-4 / (1.01 sum sigma^2) >~ 1e-5
    G = (U * sig) @ V.T
    O, _ = oracle.polar_cans(G)
    assert oracle.relative_frobenius(O, U @ V.T) < 3e-5
    assert np.linalg.norm(O.T @ O - np.eye(n)) < 2 * 3e-5 * np.sqrt(n)


def test_diagonal_and_rank1_closed_forms():
    coeffs = _coeffs()

    def phi(x):
        for a, b in coeffs:
            x = x * (a + b * x * x)
        return x

    d = np.array([3.0, -1.0, 0.5, 0.0])
    G = np.diag(d)
    O, info = oracle.polar_cans(G)
    L = 1.01 * np.sum(d * d)
    assert info["bound"] == pytest.approx(L, rel=1e-15)
    np.testing.assert_allclose(O, np.diag(np.sign(d) * phi(np.abs(d) / np.sqrt(L))), rtol=1e-13, atol=1e-15)
    u, v = np.array([1.0, 2.0, 2.0]), np.array([3.0, 4.0])
    O, _ = oracle.polar_cans(-2.5 * np.outer(u, v))
    expect = -phi(1.0 / np.sqrt(1.01)) * np.outer(u / 3.0, v / 5.0)
    np.testing.assert_allclose(O, expect, rtol=1e-13, atol=1e-15)


def test_invariances():
    rng = np.random.default_rng(6)
    G = rng.standard_normal((30, 20))
    O, _ = oracle.polar_cans(G)
    Q1, _ = np.linalg.qr(rng.standard_normal((30, 30)))
    Q2, _ = np.linalg.qr(rng.standard_normal((20, 20)))
    assert oracle.relative_frobenius(oracle.polar_cans(Q1 @ G @ Q2.T)[0], Q1 @ O @ Q2.T) < 1e-12
    assert oracle.relative_frobenius(oracle.polar_cans(G.T)[0], O.T) < 1e-12
    assert oracle.relative_frobenius(oracle.polar_cans(7.5 * G)[0], O) < 1e-13


def test_flags():
    O, info = oracle.polar_cans(np.zeros((5, 3)))
    assert info["flags"] == oracle.FLAG_ZERO_TRACE and not O.any()
    G = np.ones((4, 4))
    G[1, 1] = np.nan
    O, info = oracle.polar_cans(G)
    assert info["flags"] == oracle.FLAG_NONFINITE and np.isnan(O).all()
