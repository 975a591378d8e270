"""Properties of the HIP path that hold at any size, beside the parity tests.

* The bound c the Newton route scales by is an upper bound on the largest
  eigenvalue of A/s + eps I with its 1% margin (the OKLS page, appendix D,
  normalises its iteration by a strict upper bound computed in O(d^2)),
  checked against LAPACK's eigenvalues on inputs where the Wolkowicz-Styan
  bound is tight (flat spectra, one dominant eigenvalue: there the
  fourth-moment bound is exact too) and loose (log-uniform and low-rank
  spectra), with and without the rescale; c is never above 1.01 x
  Wolkowicz-Styan and, on the loose ones, where the fourth-moment bound takes
  over, well below it; the rescale s is the trace.
* Relabelling rows and columns of the gradients relabels the roots and the
  update: G -> P G Q^T gives X_L -> P X_L P^T, X_R -> Q X_R Q^T and
  U -> P U Q^T (within rounding: the sums run in another order).
* The eigendecomposition route reports what it cannot do: an input whose
  shifted spectrum is not positive is flagged NOT_PD with a NaN root, and a
  sweep cap too low to converge leaves NOT_CONVERGED with the root built
  from where the sweeps stopped.
* A converged Newton iterate stays put: the roots of A and of the root's own
  inverse fourth power agree (the coupled iteration's fixed point is stable).
"""

import numpy as np
import pytest

import oracle
import parity
from matrix_roots_amd import binding as B
from matrix_roots_amd import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


@pytest.fixture(scope="module")
def torch_dev(gpu_available):
    import torch

    B.library()
    return torch, torch.device("cuda:0")


def _spectrum_cases(rng):
    out = []
    for d in (129, 256, 300, 512):
        q = W.haar_columns(rng, d, d)
        flat = np.full(d, 1.0)
        dominant = np.concatenate([[1.0], np.full(d - 1, 1e-7)])
        loguni = 10.0 ** rng.uniform(-8, 0, size=d)
        lowrank = np.concatenate([rng.uniform(0.5, 1.0, size=8), np.zeros(d - 8)])
        for lam in (flat, dominant, loguni, lowrank):
            A = (q * lam) @ q.T
            out.append((0.5 * (A + A.T)).astype(np.float32))
    return out


@pytest.mark.parametrize("normalize", ["trace", "none"])
def test_bound_is_above_the_largest_eigenvalue(torch_dev, normalize):
    torch, dev = torch_dev
    rng = W.rng_for(94, 0 if normalize == "trace" else 1)
    mats = _spectrum_cases(rng)
    eps = 1e-6
    _, info = B.inv_quarter_root_batched([torch.from_numpy(a).to(dev) for a in mats], eps, normalize=normalize,
                                         method="newton")
    tighter = 0
    for a, rec in zip(mats, info):
        A = a.astype(np.float64)
        Ahat, s = oracle.rescale(0.5 * (A + A.T), normalize)
        lam_max = float(np.linalg.eigvalsh(Ahat)[-1]) + eps
        # c carries the stated 1% margin over lambda_max ...
        assert rec["bound"] >= 1.01 * lam_max * (1.0 - 1e-12), (a.shape, rec["bound"], lam_max)
        # ... and is never looser than 1.01 x Wolkowicz-Styan (the fourth-moment
        # bound only replaces it where it is tighter)
        d = A.shape[0]
        Bm = Ahat + eps * np.eye(d)
        m = np.trace(Bm) / d
        ws = m + np.sqrt(max(np.sum(Bm * Bm) / d - m * m, 0.0)) * np.sqrt(d - 1.0)
        # (relative 1e-6: on flat spectra the variance term is rounding noise)
        assert rec["bound"] <= 1.01 * ws * (1.0 + 1e-6), (a.shape, rec["bound"], ws)
        tighter += rec["bound"] < 0.8 * 1.01 * ws
        if normalize == "trace":
            assert rec["scale"] == pytest.approx(float(np.trace(A)), rel=1e-12)
        else:
            assert rec["scale"] == 1.0
    # the spread spectra (log-uniform, low-rank: 8 of the 16) take the
    # fourth-moment bound, 1.6-2.2 times below Wolkowicz-Styan there
    assert tighter >= 6, tighter


def test_permutation_equivariance(torch_dev):
    torch, dev = torch_dev
    rng = np.random.default_rng(95)
    shapes = [(96, 200), (160, 96), (300, 130)]  # Jacobi and Newton roots
    grads = [[W.gradient("w1024", k, t, shape=s) for k, s in enumerate(shapes)] for t in (1, 2)]
    perms = [(np.eye(m)[rng.permutation(m)], np.eye(n)[rng.permutation(n)]) for m, n in shapes]
    runs = []
    for permuted in (False, True):
        Ls = [torch.zeros(m, m, dtype=torch.float64, device=dev) for m, n in shapes]
        Rs = [torch.zeros(n, n, dtype=torch.float64, device=dev) for m, n in shapes]
        for t in range(2):
            gs = [P @ g @ Q.T if permuted else g for g, (P, Q) in zip(grads[t], perms)]
            Gd = [torch.from_numpy(np.ascontiguousarray(g, dtype=np.float32)).to(dev) for g in gs]
            B.gram_ema_update(Gd, Ls, Rs, 0.95)
            Xs, info = B.inv_quarter_root_batched(Ls + Rs, 1e-6)
            assert (info["flags"] == 0).all()
            Us = B.precondition_apply(Xs[:len(shapes)], Gd, Xs[len(shapes):])
        torch.cuda.synchronize()
        runs.append(([x.cpu().numpy() for x in Xs], [u.cpu().numpy() for u in Us]))
    (Xa, Ua), (Xb, Ub) = runs
    k = len(shapes)
    for i, (P, Q) in enumerate(perms):
        parity.assert_close(Xb[i], P @ Xa[i] @ P.T, 1e-5, f"left root {shapes[i]}")
        parity.assert_close(Xb[k + i], Q @ Xa[k + i] @ Q.T, 1e-5, f"right root {shapes[i]}")
        parity.assert_close(Ub[i], P @ Ua[i] @ Q.T, 1e-4, f"update {shapes[i]}")


@pytest.mark.parametrize("d", [17, 64, 96, 128])
def test_jacobi_not_pd(torch_dev, d):
    """lambda + eps <= 0 for one eigenvalue (no rescale): NOT_PD, NaN root;
    the other matrix of the batch is unaffected."""
    torch, dev = torch_dev
    rng = W.rng_for(96, d)
    q = W.haar_columns(rng, d, d)
    lam = np.geomspace(1e-3, 1.0, d)
    lam[d // 3] = -0.2
    bad = ((q * lam) @ q.T).astype(np.float32)
    good = W.spd_loguniform(d, rng, -4.0, 0.0)
    As = [torch.from_numpy(bad).to(dev), torch.from_numpy(good).to(dev)]
    Xs, info = B.inv_quarter_root_batched(As, 1e-6, normalize="none", method="jacobi")
    assert info["flags"][0] == B.MR_INFO_NOT_PD
    assert np.isnan(Xs[0].cpu().numpy()).all()
    assert info["flags"][1] == 0
    ref, _ = oracle.inv_quarter_root(good.astype(np.float64), 1e-6, "none")
    parity.assert_root(Xs[1], ref, f"good matrix beside a NOT_PD one, d={d}")


@pytest.mark.parametrize("d", [40, 100, 128])
def test_jacobi_not_converged_under_a_sweep_cap(torch_dev, d):
    """One sweep cannot diagonalise a dense matrix: NOT_CONVERGED, iters = 1,
    a finite symmetric root; with the default cap the same call converges."""
    torch, dev = torch_dev
    A = W.spd_loguniform(d, W.rng_for(97, d), -6.0, 0.0)
    Ad = [torch.from_numpy(A).to(dev)]
    prev = B.set_jacobi_max_sweeps(1)
    try:
        Xs, info = B.inv_quarter_root_batched(Ad, 1e-6, method="jacobi")
    finally:
        B.set_jacobi_max_sweeps(prev)
    assert info["flags"][0] == B.MR_INFO_NOT_CONVERGED and info["iters"][0] == 1
    X = Xs[0].cpu().numpy()
    assert np.isfinite(X).all() and np.array_equal(X, X.T)
    Xs2, info2 = B.inv_quarter_root_batched(Ad, 1e-6, method="jacobi")
    assert info2["flags"][0] == 0 and 1 < info2["iters"][0] <= 30
    ref, _ = oracle.inv_quarter_root(A.astype(np.float64), 1e-6)
    parity.assert_root(Xs2[0], ref, f"default sweep cap d={d}")


def test_newton_fixed_point_is_stable(torch_dev):
    """With X the computed (A + eps I)^(-1/4) (no rescale), B = X^-4 has
    B^(-1/4) = X exactly; the Newton route on B (eps tiny against its
    spectrum) returns X again within float32 rounding."""
    torch, dev = torch_dev
    d = 256
    A = W.spd_loguniform(d, W.rng_for(98, 0), -3.0, 0.0).astype(np.float64)
    X, _ = oracle.inv_quarter_root(A, 1e-6, "none")
    X2 = X @ X
    Bm = np.linalg.inv(X2 @ X2)
    Bm = (0.5 * (Bm + Bm.T)).astype(np.float32)
    ref, _ = oracle.inv_quarter_root(Bm.astype(np.float64), 1e-12, "none")
    Xs, info = B.inv_quarter_root_batched([torch.from_numpy(Bm).to(dev)], 1e-12, normalize="none",
                                          method="newton")
    assert info["flags"][0] == 0
    parity.assert_root(Xs[0], ref, "root of X^-4")
    parity.assert_close(Xs[0], X, 1e-4, "back to X")


def test_no_rescale_floor_below_the_cap_is_flagged(torch_dev):
    """Without a rescale the host launches the schedule of the floor 1e-16 and
    never waits for the device: a matrix whose floor eps / c lies below that
    (here lambda_max = 1e3, eps = 1e-14: floor about 3e-18) runs that
    schedule, flagged NOT_CONVERGED, with a finite root (its eigenvalues
    all lie above 1e-16 of c, so the root is the oracle's), while the other
    matrix of the same call converges to the oracle unflagged."""
    torch, dev = torch_dev
    rng = W.rng_for(99, 0)
    far = (1e3 * W.spd_loguniform(160, rng, -2.0, 0.0).astype(np.float64)).astype(np.float32)
    near = W.spd_loguniform(160, rng, -3.0, 0.0)
    As = [torch.from_numpy(far).to(dev), torch.from_numpy(near).to(dev)]
    Xs, info = B.inv_quarter_root_batched(As, 1e-14, normalize="none", method="newton")
    assert info["flags"][0] == B.MR_INFO_NOT_CONVERGED, info[0]
    assert np.isfinite(Xs[0].cpu().numpy()).all()
    cap, cap_j = B.newton_schedule(1e-16)
    assert info["iters"][0] == len(cap) and info["fp64_iters"][0] == cap_j
    ref_far, _ = oracle.inv_quarter_root(far.astype(np.float64), 1e-14, "none")
    parity.assert_root(Xs[0], ref_far, "capped matrix")
    cap = len(cap)
    assert info["flags"][1] == 0 and info["iters"][1] < cap
    ref, _ = oracle.inv_quarter_root(near.astype(np.float64), 1e-14, "none")
    parity.assert_root(Xs[1], ref, "converged neighbour of a capped matrix")
