"""Plain CPU fp64 oracle for the EMA-Gram quarter-power preconditioner step.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import or run this module. The product path (the HIP
library and its Python binding) never calls it and must fail loudly when the
HIP library is missing.

What it computes, and where the pages define it:

* marin.community, "Sharding EMA-Gram eigensolves", section "Background":
  for every linear weight the optimizer keeps an exponential moving average of
  G·Gᵀ (the left Gram) and of Gᵀ·G (the right Gram, factors in reverse order). At
  each update it rescales both Grams, decomposes each into eigenvectors and
  eigenvalues, adds a small regulariser to the eigenvalues, raises them to
  -1/4, rebuilds the matrices, and uses these inverse quarter powers to shape
  the direction of the update.
* The two-sided shape U = L^-1/4 · G · R^-1/4 is the Shampoo form described
  in tilderesearch, "Online KL Shampoo", section 1 (its formulas did not
  survive extraction; the quarter powers on both sides are the EMA-Gram
  page's).
* The inverse square root of a symmetric positive definite matrix, the root
  tilderesearch, "Online KL Shampoo", computes for its preconditioner
  (sections 2.2-2.4, appendix D), as the same eigenvalue map with power -1/2.
* The step around the preconditioner: a momentum EMA of the gradient and
  the MuonH norm-preserving (hyperball) update of the weight
  (ai.thesatyajit.com, "Marin 535B-A23B", section "A sphere for
  every matrix").
* The polar orthogonalisation its CANS coefficients were designed for
  (section 2.3), as the odd polynomial those ten steps apply to the
  singular values (numpy.linalg.svd, LAPACK gesdd).

Readings taken where the pages are silent (each is listed with its reason in
the design notes):

* rescale = divide by the trace, so the rescaled Gram has unit trace;
* EMA = beta*S + (1-beta)*Gram, starting from zero, no bias correction;
* the regulariser eps is added to the eigenvalues of the rescaled Gram;
* the rescale is not undone after the root;
* no clamping of eigenvalues: a Gram whose shifted spectrum is not positive is
  reported as not positive definite;
* the input of the root is taken as the symmetric part (A + Aᵀ)/2;
* the output root is symmetrised, (X + Xᵀ)/2 (the OKLS page, appendix D, does
  the same to its root).

Everything is float64. numpy's ``@`` (BLAS dgemm), ``numpy.linalg.eigh``
(LAPACK dsyevd) and ``numpy.linalg.svd`` (LAPACK gesdd) are the only library
steps; nothing is blocked, fused or
reordered beyond the definitions above.
"""

from __future__ import annotations

import numpy as np

# Per-matrix outcome flags (same meaning as the library's info flags).
FLAG_NONFINITE = 1
FLAG_ZERO_TRACE = 2
FLAG_NOT_PD = 4

NORM_NONE = "none"
NORM_TRACE = "trace"


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def left_gram(G) -> np.ndarray:
    """G·Gᵀ (m×m): the product the left Gram averages (EMA-Gram page, Background)."""
    G = _f64(G)
    return G @ G.T


def right_gram(G) -> np.ndarray:
    """Gᵀ·G (n×n): the product with the factors in reverse order (EMA-Gram page, Background)."""
    G = _f64(G)
    return G.T @ G


def gram_ema_update(L, R, G, beta: float):
    """One EMA step of both Grams: S <- beta*S + (1-beta)*Gram(G).

    EMA-Gram page, Background: each Gram is an exponential moving average of
    gradient products. The weighting convention is not printed; this is the
    plain one. Returns new (L, R) in float64; the inputs are not modified.
    """
    beta = float(beta)
    L_new = beta * _f64(L) + (1.0 - beta) * left_gram(G)
    R_new = beta * _f64(R) + (1.0 - beta) * right_gram(G)
    return L_new, R_new


def rescale(A, normalize: str = NORM_TRACE):
    """Rescale a Gram before its root (EMA-Gram page, Background and Approach).

    TRACE: s = tr(A), returns (A/s, s). NONE: s = 1, returns (A, 1).
    A zero trace returns (A, 0.0); the caller reports ZERO_TRACE.
    """
    A = _f64(A)
    if normalize == NORM_NONE:
        return A.copy(), 1.0
    if normalize != NORM_TRACE:
        raise ValueError(f"unknown normalize mode {normalize!r}")
    s = float(np.trace(A))
    if s == 0.0:
        return A.copy(), 0.0
    return A / s, s


def inv_quarter_root(A, eps: float, normalize: str = NORM_TRACE):
    """X = (Â + eps·I)^(-1/4) by a dense symmetric eigensolver.

    EMA-Gram page, Background: decompose into eigenvectors and eigenvalues,
    add a small regulariser to the eigenvalues, raise them to -1/4 and
    rebuild the matrix.  Â = sym(A)/s with s from :func:`rescale`.

    Returns (X, info) with info = {"scale": s, "flags": bits,
    "eigenvalues": eigenvalues of Â (ascending)}.  Special cases:
    non-finite input -> X all NaN, NONFINITE; zero trace -> X = eps^(-1/4)·I,
    ZERO_TRACE; some eigenvalue + eps <= 0 -> X all NaN, NOT_PD.
    """
    A = _f64(A)
    d = A.shape[0]
    if A.shape != (d, d):
        raise ValueError("A must be square")
    eps = float(eps)
    if not np.all(np.isfinite(A)):
        return np.full((d, d), np.nan), {"scale": float("nan"), "flags": FLAG_NONFINITE,
                                         "eigenvalues": None}
    A = 0.5 * (A + A.T)
    Ahat, s = rescale(A, normalize)
    if s == 0.0:
        return eps ** -0.25 * np.eye(d), {"scale": 0.0, "flags": FLAG_ZERO_TRACE,
                                          "eigenvalues": np.zeros(d)}
    w, V = np.linalg.eigh(Ahat)
    shifted = w + eps
    if np.min(shifted) <= 0.0:
        return np.full((d, d), np.nan), {"scale": s, "flags": FLAG_NOT_PD, "eigenvalues": w}
    f = shifted ** -0.25
    X = (V * f) @ V.T
    X = 0.5 * (X + X.T)
    return X, {"scale": s, "flags": 0, "eigenvalues": w}


def inv_sqrt_root(A, eps: float, normalize: str = NORM_NONE):
    """W = (Â + eps·I)^(-1/2) by a dense symmetric eigensolver.

    tilderesearch, "Online KL Shampoo", appendix D: the batched root returns
    the inverse square root of a symmetric positive definite matrix S (its
    section 2.2 computes it by a coupled Newton-Schulz iteration; what that
    iteration converges to is this matrix function).  Here S = Â + eps·I with
    Â = sym(A)/s from :func:`rescale`; normalize="none" and eps=0 give the
    page's S^(-1/2) of sym(A) itself.

    Returns (W, info) like :func:`inv_quarter_root`: NaN for non-finite
    input (NONFINITE) or some eigenvalue + eps <= 0 (NOT_PD);
    eps^(-1/2)·I for a zero trace (ZERO_TRACE).
    """
    A = _f64(A)
    d = A.shape[0]
    if A.shape != (d, d):
        raise ValueError("A must be square")
    eps = float(eps)
    if not np.all(np.isfinite(A)):
        return np.full((d, d), np.nan), {"scale": float("nan"), "flags": FLAG_NONFINITE,
                                         "eigenvalues": None}
    A = 0.5 * (A + A.T)
    Ahat, s = rescale(A, normalize)
    if s == 0.0:
        W = eps ** -0.5 * np.eye(d) if eps > 0.0 else np.full((d, d), np.nan)
        return W, {"scale": 0.0, "flags": FLAG_ZERO_TRACE | (0 if eps > 0.0 else FLAG_NOT_PD),
                   "eigenvalues": np.zeros(d)}
    w, V = np.linalg.eigh(Ahat)
    shifted = w + eps
    if np.min(shifted) <= 0.0:
        return np.full((d, d), np.nan), {"scale": s, "flags": FLAG_NOT_PD, "eigenvalues": w}
    f = shifted ** -0.5
    W = (V * f) @ V.T
    W = 0.5 * (W + W.T)
    return W, {"scale": s, "flags": 0, "eigenvalues": w}


# The ten CANS polynomial coefficient pairs (a_k, b_k) printed in
# tilderesearch, "Online KL Shampoo", appendix D.
CANS_COEFFS = (
    (5.182503604966906, -5.178098480082684), (2.586120737395915, -0.6479542005271643),
    (2.567364126726186, -0.6454968804392178), (2.520560084348265, -0.6393528082067044),
    (2.410759275435182, -0.6248683598710716), (2.1883348130094173, -0.5952022073798908),
    (1.8595760874873613, -0.5504490972723968), (1.589020160467417, -0.5126569802066718),
    (1.5051653981684994, -0.5007377068751799), (1.5, -0.5),
)


def polar_cans(G):
    """The orthogonalised update of the ten CANS polar steps.

    tilderesearch, "Online KL Shampoo", section 2.3: the CANS coefficients
    were built for Muon's polar factor, where each step X <- a_k X +
    b_k X Xᵀ X moves every singular value by s <- s (a_k + b_k s²) and
    leaves the singular vectors alone.  So from X0 = G / sqrt(L) the ten
    steps give exactly U · diag(phi(sigma / sqrt(L))) · Vᵀ with G = U Σ Vᵀ
    (thin SVD) and phi the composition of the ten odd polynomials; phi is
    within 3e-5 of 1 for sigma² / L in [1e-6, 0.99], so this is the polar
    factor U Vᵀ wherever the spectrum lies in that range.  L = 1.01 ||G||_F²
    (the Frobenius normalisation Muon uses, with the OKLS page's 1.01
    safety factor), so sigma² / L <= 1/1.01.

    Returns (O, info), info = {"scale": ||G||_F², "bound": L, "flags"}:
    non-finite G -> O all NaN, NONFINITE; zero G -> O = 0, ZERO_TRACE.
    """
    G = _f64(G)
    if not np.all(np.isfinite(G)):
        return np.full(G.shape, np.nan), {"scale": float("nan"), "bound": float("nan"), "flags": FLAG_NONFINITE}
    f2 = float(np.sum(G * G))
    if f2 == 0.0:
        return np.zeros(G.shape), {"scale": 0.0, "bound": 0.0, "flags": FLAG_ZERO_TRACE}
    L = 1.01 * f2
    U, sigma, Vt = np.linalg.svd(G, full_matrices=False)
    x = sigma / np.sqrt(L)
    for a, b in CANS_COEFFS:
        x = x * (a + b * x * x)
    return (U * x) @ Vt, {"scale": f2, "bound": L, "flags": 0}


def momentum_ema(M, G, mu: float) -> np.ndarray:
    """M <- mu M + (1 - mu) G: the momentum the preconditioned direction is
    taken of (EMA-Gram page, "Results", compares update directions at equal
    Grams and momentum; the MuonH notes of the Marin 535B-A23B article take the momentum of
    each matrix's gradient first).  The EMA form is a reading: its scale
    cancels in the norm-preserving update below."""
    return float(mu) * _f64(M) + (1.0 - float(mu)) * _f64(G)


def hyperball_update(W, U, lr: float):
    """The MuonH hyperball step (ai.thesatyajit.com, "Marin 535B-A23B",
    section "A sphere for every matrix"): move W against U by lr times W's own norm, then rescale back to
    W's original norm, with the page's 1e-10 floors on both divisors:

        c = lr ||W|| / max(||U||, 1e-10),  W' = W - c U,
        W_new = W' ||W|| / max(||W'||, 1e-10).

    Norms are Frobenius norms of the whole matrix.  Returns (W_new,
    {"w_norm", "u_norm", "new_norm"}) with new_norm = ||W'||.
    """
    W, U = _f64(W), _f64(U)
    wn = float(np.sqrt(np.sum(W * W)))
    un = float(np.sqrt(np.sum(U * U)))
    Wp = W - float(lr) * U * (wn / max(un, 1e-10))
    pn = float(np.sqrt(np.sum(Wp * Wp)))
    return Wp / max(pn, 1e-10) * wn, {"w_norm": wn, "u_norm": un, "new_norm": pn}


def precondition_apply(XL, G, XR, alpha: float = 1.0) -> np.ndarray:
    """U = alpha · X_L · G · X_R (the two-sided quarter-power direction)."""
    return float(alpha) * ((_f64(XL) @ _f64(G)) @ _f64(XR))


def preconditioner_step(L, R, G, beta: float, eps: float, normalize: str = NORM_TRACE):
    """The whole per-weight step: EMA both Grams, root both, apply to G.

    Returns (L, R, XL, XR, U, flags) where flags ORs both roots' flags.
    """
    L, R = gram_ema_update(L, R, G, beta)
    XL, il = inv_quarter_root(L, eps, normalize)
    XR, ir = inv_quarter_root(R, eps, normalize)
    U = precondition_apply(XL, G, XR)
    return L, R, XL, XR, U, il["flags"] | ir["flags"]


def run_sequence(grads, beta: float, eps: float, normalize: str = NORM_TRACE, L0=None, R0=None):
    """Run the step over a sequence of gradients of one weight from zero state.

    Yields (t, L, R, XL, XR, U, flags) for t = 1, 2, ...
    """
    L = R = None
    for t, G in enumerate(grads, start=1):
        G = _f64(G)
        m, n = G.shape
        if L is None:
            L = np.zeros((m, m)) if L0 is None else _f64(L0)
            R = np.zeros((n, n)) if R0 is None else _f64(R0)
        L, R, XL, XR, U, flags = preconditioner_step(L, R, G, beta, eps, normalize)
        yield t, L, R, XL, XR, U, flags


def relative_frobenius(x, ref) -> float:
    """‖x − ref‖_F / ‖ref‖_F: the comparison the EMA-Gram page uses for update
    directions (section "Results")."""
    x = _f64(x)
    ref = _f64(ref)
    den = np.linalg.norm(ref)
    if den == 0.0:
        return float(np.linalg.norm(x))
    return float(np.linalg.norm(x - ref) / den)
