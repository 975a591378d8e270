"""GPU parity of the HIP path against the fp64 oracle (sizes the oracle
finishes in seconds, spanning several 128-wide tiles and ragged tails).

Tolerances: relative Frobenius error <= 1e-4 on every root and <= 1e-3 on
every update direction (the comparison the EMA-Gram page uses between update
directions, section "Results").  Gram states in float64 are held to 1e-12
(float32 products are exact in float64; only the summation order differs).
"""

import numpy as np
import pytest

import oracle
import parity
from matrix_roots_amd import binding as B
from matrix_roots_amd import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

ROOT_TOL = 1e-4
UPDATE_TOL = 1e-3


@pytest.fixture(scope="module")
def torch_dev(gpu_available):
    import torch

    B.library()
    return torch, torch.device("cuda:0")


def to_dev(torch, dev, a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev)


def spd(d, rng, lo=-6.0, hi=0.0):
    return W.spd_loguniform(d, rng, lo, hi)


# ------------------------------------------------------------------ Gram EMA
@pytest.mark.parametrize("state", ["f64", "f32"])
def test_gram_ema_matches_oracle(torch_dev, state):
    torch, dev = torch_dev
    # (64, 128), (128, 256), (176, 336) and (96, 400) take the direct-to-LDS
    # core on both sides (contractions multiples of 16; 176, 336 and 400 leave
    # ragged last tiles), the others the register-staged one on one or both
    shapes = [(64, 128), (200, 328), (130, 7), (1, 5), (257, 129), (128, 256), (33, 97), (176, 336), (96, 400)]
    sdt = torch.float64 if state == "f64" else torch.float32
    beta = 0.95
    rng = np.random.default_rng(5)
    Ls = [torch.zeros(m, m, dtype=sdt, device=dev) for m, n in shapes]
    Rs = [torch.zeros(n, n, dtype=sdt, device=dev) for m, n in shapes]
    Lo = [np.zeros((m, m)) for m, n in shapes]
    Ro = [np.zeros((n, n)) for m, n in shapes]
    for step in range(3):
        Gs = [rng.standard_normal((m, n)).astype(np.float32) for m, n in shapes]
        B.gram_ema_update([to_dev(torch, dev, g) for g in Gs], Ls, Rs, beta)
        torch.cuda.synchronize()
        for i, G in enumerate(Gs):
            Lo[i], Ro[i] = oracle.gram_ema_update(Lo[i], Ro[i], G, beta)
            tol = 1e-12 if state == "f64" else 2e-7
            for got, ref in ((Ls[i], Lo[i]), (Rs[i], Ro[i])):
                g = got.cpu().numpy().astype(np.float64)
                assert np.array_equal(g, g.T), f"state not exactly symmetric, shape {shapes[i]}"
                err = oracle.relative_frobenius(g, ref)
                assert err <= tol, (shapes[i], step, err)


def test_gram_ema_beta_zero_ignores_old_state(torch_dev):
    torch, dev = torch_dev
    rng = np.random.default_rng(6)
    G = rng.standard_normal((96, 40)).astype(np.float32)
    L = torch.full((96, 96), float("nan"), dtype=torch.float64, device=dev)
    R = torch.full((40, 40), float("nan"), dtype=torch.float64, device=dev)
    B.gram_ema_update([to_dev(torch, dev, G)], [L], [R], 0.0)
    Lo, Ro = oracle.gram_ema_update(np.zeros((96, 96)), np.zeros((40, 40)), G, 0.0)
    assert oracle.relative_frobenius(L.cpu().numpy(), Lo) < 1e-13
    assert oracle.relative_frobenius(R.cpu().numpy(), Ro) < 1e-13


# --------------------------------------------------------------------- roots
def _check_roots(torch, dev, mats, eps, normalize, method, a_dtype, tol):
    As = [to_dev(torch, dev, a, a_dtype) for a in mats]
    Xs, info = B.inv_quarter_root_batched(As, eps, normalize=normalize, method=method)
    for i, a in enumerate(mats):
        ref, rinfo = oracle.inv_quarter_root(As[i].cpu().numpy().astype(np.float64), eps, normalize)
        X = Xs[i].cpu().numpy()
        assert np.array_equal(X, X.T), f"root {i} (d={a.shape[0]}) not exactly symmetric"
        err = oracle.relative_frobenius(X, ref)
        assert info["flags"][i] == 0, (i, a.shape, info[i])
        assert err <= tol, (i, a.shape, err, info[i])
    return Xs, info


@pytest.mark.parametrize("a_dtype", ["f32", "f64"])
@pytest.mark.parametrize("normalize", ["trace", "none"])
def test_jacobi_root_matches_oracle(torch_dev, a_dtype, normalize):
    torch, dev = torch_dev
    rng = W.rng_for(90, 1)
    sizes = [1, 2, 3, 17, 64, 100, 127, 128]
    mats = [spd(d, rng) for d in sizes]
    dt = torch.float64 if a_dtype == "f64" else torch.float32
    _, info = _check_roots(torch, dev, mats, 1e-6, normalize, "jacobi", dt, ROOT_TOL)
    assert (info["iters"] <= 30).all()


@pytest.mark.parametrize("method", ["newton", "newton_f32", "newton_f64"])
@pytest.mark.parametrize("a_dtype", ["f32", "f64"])
def test_newton_root_matches_oracle(torch_dev, method, a_dtype):
    torch, dev = torch_dev
    rng = W.rng_for(90, 2)
    # 270: even but not a multiple of 8, with whole float64 tiles (the mirror
    # through LDS slabs with element stores of the split copy)
    sizes = [129, 200, 256, 301, 384, 270]
    mats = [spd(d, rng) for d in sizes]
    dt = torch.float64 if a_dtype == "f64" else torch.float32
    tol = 1e-6 if method == "newton_f64" else ROOT_TOL
    for normalize in ("trace", "none"):
        _check_roots(torch, dev, mats, 1e-6, normalize, method, dt, tol)


def test_newton_wide_tiles_ragged(torch_dev):
    """Multiples of 32 from d = 1024 take the split-fp16 stages on 256 x 256
    tiles: four whole tile rows plus a 32-row strip (1056), plus 160 rows
    (1184) and plus 224 (1248), so the last tile row and column are partial
    and take the element stores; smaller multiples of 32 (160, 288, 544 on
    128 x 128 direct-to-LDS tiles) and of 8 (264, 200: register-staged 128 x
    128 tiles) share the call."""
    torch, dev = torch_dev
    rng = W.rng_for(90, 5)
    mats = [spd(d, rng) for d in (1056, 160, 288, 1184, 264, 544, 200, 1248)]
    for normalize in ("trace", "none"):
        _check_roots(torch, dev, mats, 1e-6, normalize, "newton", torch.float32, ROOT_TOL)


def test_newton_digit_plane_placements(torch_dev):
    """From d = 1024 the float64 steps' products run on int8 digit planes,
    placed in the float64 slots a float64 step leaves idle where they fit:
    1024 (every plane there), 1056 (padded to 1152: some planes past the
    slots), 1030 (d % 4 != 0: every plane past the slots, ragged tiles) and
    1027 (odd: unaligned rows of the float64 M read element by element),
    next to a 1000 that keeps the float64 kernel, in one call; log-uniform
    spectra down to 1e-8 keep several float64 steps."""
    torch, dev = torch_dev
    rng = W.rng_for(90, 11)
    mats = [spd(d, rng, lo=-8.0) for d in (1024, 1056, 1030, 1027, 1000)]
    for normalize in ("trace", "none"):
        _check_roots(torch, dev, mats, 1e-6, normalize, "newton", torch.float32, ROOT_TOL)


def test_newton_read_ahead_chunk_counts(torch_dev):
    """Chunk counts at the edges of the main loops that read fragments one
    k-step ahead: one chunk (d = 16 in the float64 core, d = 32 in the
    direct-to-LDS split-fp16 core), two (d = 32 in float64) and an odd count
    (d = 48: three float64 chunks)."""
    torch, dev = torch_dev
    rng = W.rng_for(90, 7)
    mats = [spd(d, rng) for d in (16, 32, 48)]
    for method in ("newton", "newton_f64"):
        _check_roots(torch, dev, mats, 1e-6, "trace", method, torch.float32, ROOT_TOL)


def test_newton_small_d_matches_jacobi(torch_dev):
    """Forced Newton on Jacobi-sized inputs agrees with the oracle too."""
    torch, dev = torch_dev
    rng = W.rng_for(90, 3)
    mats = [spd(d, rng) for d in (5, 64, 128)]
    _check_roots(torch, dev, mats, 1e-6, "trace", "newton", torch.float32, ROOT_TOL)


def test_illconditioned_subset(torch_dev):
    """A slice of the ill-conditioned 512 x 512 batch at every eps."""
    torch, dev = torch_dev
    mats = [W.spd_loguniform(512, W.rng_for(W.WORKLOAD_IDS["illcond"], 0, i, 0)) for i in range(6)]
    for eps in W.WORKLOADS["illcond"].eps_list:
        _check_roots(torch, dev, mats, eps, "none", "auto", torch.float32, ROOT_TOL)


def test_root_flags(torch_dev):
    torch, dev = torch_dev
    eps = 1e-4
    for d, method in ((16, "jacobi"), (160, "newton")):
        z = np.zeros((d, d), dtype=np.float32)
        nan = np.eye(d, dtype=np.float32)
        nan[1, 2] = np.nan
        As = [to_dev(torch, dev, z), to_dev(torch, dev, nan)]
        Xs, info = B.inv_quarter_root_batched(As, eps, normalize="trace", method=method)
        assert info["flags"][0] == B.MR_INFO_ZERO_TRACE
        np.testing.assert_allclose(Xs[0].cpu().numpy(), eps ** -0.25 * np.eye(d), rtol=1e-6)
        assert info["flags"][1] & B.MR_INFO_NONFINITE
        assert np.isnan(Xs[1].cpu().numpy()).all()


def test_newton_flags_indefinite_input(torch_dev):
    """A + eps I with an eigenvalue well below zero has no inverse quarter
    root: the Newton iterate never nears I, whichever last update the schedule
    picks, and the residual check flags it (d = 1056: through the int8 digit
    planes, whose digits clamp on such input)."""
    torch, dev = torch_dev
    rng = W.rng_for(90, 6)
    for d in (160, 288, 1056):
        q, _ = np.linalg.qr(rng.standard_normal((d, d)))
        lam = np.geomspace(1e-3, 1.0, d)
        lam[d // 2] = -0.3
        A = ((q * lam) @ q.T).astype(np.float32)
        for normalize in ("none", "trace"):
            _, info = B.inv_quarter_root_batched([to_dev(torch, dev, A)], 1e-6, normalize=normalize, method="newton")
            assert info["flags"][0] & B.MR_INFO_NOT_CONVERGED, (d, normalize, info[0])


# --------------------------------------------------------------------- apply
def test_apply_matches_oracle(torch_dev):
    torch, dev = torch_dev
    rng = np.random.default_rng(8)
    shapes = [(64, 128), (200, 328), (130, 7), (1, 5), (257, 129)]
    XLs, Gs, XRs, refs = [], [], [], []
    for m, n in shapes:
        XL = rng.standard_normal((m, m)).astype(np.float32)
        XL = (XL + XL.T) / 2
        XR = rng.standard_normal((n, n)).astype(np.float32)
        XR = (XR + XR.T) / 2
        G = rng.standard_normal((m, n)).astype(np.float32)
        XLs.append(to_dev(torch, dev, XL))
        XRs.append(to_dev(torch, dev, XR))
        Gs.append(to_dev(torch, dev, G))
        refs.append(oracle.precondition_apply(XL, G, XR, 0.5))
    Us = B.precondition_apply(XLs, Gs, XRs, alpha=0.5)
    torch.cuda.synchronize()
    for U, ref, sh in zip(Us, refs, shapes):
        err = oracle.relative_frobenius(U.cpu().numpy(), ref)
        assert err <= 1e-5, (sh, err)


def test_apply_asymmetric_operands(torch_dev):
    """precondition_apply computes alpha XL G XR for any square XL and XR,
    symmetric or not (the right product reads XR through a transposed split
    copy): ragged shapes, several tiles, one 1 x 1 case."""
    torch, dev = torch_dev
    rng = np.random.default_rng(10)
    shapes = [(64, 128), (200, 328), (130, 7), (1, 1), (257, 129), (96, 300)]
    XLs, Gs, XRs, refs = [], [], [], []
    for m, n in shapes:
        XL = rng.standard_normal((m, m)).astype(np.float32)
        XR = rng.standard_normal((n, n)).astype(np.float32)
        G = rng.standard_normal((m, n)).astype(np.float32)
        XLs.append(to_dev(torch, dev, XL))
        XRs.append(to_dev(torch, dev, XR))
        Gs.append(to_dev(torch, dev, G))
        refs.append(oracle.precondition_apply(XL, G, XR, -0.75))
    Us = B.precondition_apply(XLs, Gs, XRs, alpha=-0.75)
    torch.cuda.synchronize()
    for U, ref, sh in zip(Us, refs, shapes):
        parity.assert_close(U, ref, 1e-5, f"asymmetric apply {sh}")


def test_apply_any_input_scale(torch_dev):
    """Gradients from 1e-30 to 1e30 and roots from 1e-6 to 1e6 (far outside
    fp16's range either way) keep float32-level accuracy: every operand is
    scaled by a power of two before its fp16 split."""
    torch, dev = torch_dev
    rng = np.random.default_rng(9)
    m, n = 160, 96
    XL0 = rng.standard_normal((m, m)).astype(np.float32)
    XL0 = (XL0 + XL0.T) / 2  # the roots are symmetric
    XR0 = rng.standard_normal((n, n)).astype(np.float32)
    XR0 = (XR0 + XR0.T) / 2
    G0 = rng.standard_normal((m, n)).astype(np.float32)
    for gs, xs in ((1e-30, 1.0), (1e30, 1e-6), (1e-8, 1e6), (3e-3, 7e2)):
        XL, XR, G = (XL0 * np.float32(xs)), (XR0 / np.float32(xs)), G0 * np.float32(gs)
        ref = oracle.precondition_apply(XL.astype(np.float64), G.astype(np.float64), XR.astype(np.float64), 1.0)
        (U,) = B.precondition_apply([to_dev(torch, dev, XL)], [to_dev(torch, dev, G)], [to_dev(torch, dev, XR)])
        err = oracle.relative_frobenius(U.cpu().numpy().astype(np.float64), ref)
        assert np.isfinite(U.cpu().numpy()).all() and err <= 1e-5, (gs, xs, err)


# ----------------------------------------------------------- end to end: toy
def run_pipeline(torch, dev, grads_per_step, beta, eps, method="auto", state_dtype=None):
    """Drive the three entry points over steps; yield per-step device results."""
    sdt = state_dtype or torch.float64
    shapes = [g.shape for g in grads_per_step[0]]
    Ls = [torch.zeros(m, m, dtype=sdt, device=dev) for m, n in shapes]
    Rs = [torch.zeros(n, n, dtype=sdt, device=dev) for m, n in shapes]
    ws = B.RootWorkspace()
    for grads in grads_per_step:
        Gd = [to_dev(torch, dev, g) for g in grads]
        B.gram_ema_update(Gd, Ls, Rs, beta)
        Xs, info = B.inv_quarter_root_batched(Ls + Rs, eps, method=method, workspace=ws)
        k = len(grads)
        Us = B.precondition_apply(Xs[:k], Gd, Xs[k:])
        torch.cuda.synchronize()
        yield Xs[:k], Xs[k:], Us, info


@pytest.mark.parametrize("method", ["auto", "jacobi"])
def test_toy_end_to_end(torch_dev, method):
    """The toy workload's 10 steps, by the default route (Newton for its 64^2
    and 128^2 Grams) and by the eigendecomposition route."""
    torch, dev = torch_dev
    wl = W.WORKLOADS["toy"]
    steps = [[W.gradient("toy", w, t) for w in range(len(wl.shapes))] for t in range(1, wl.steps + 1)]
    refs = [list(oracle.run_sequence([steps[t][w] for t in range(wl.steps)], wl.beta, wl.eps))
            for w in range(len(wl.shapes))]
    worst = [0.0, 0.0]
    for t, (XL, XR, U, info) in enumerate(run_pipeline(torch, dev, steps, wl.beta, wl.eps, method=method)):
        assert (info["flags"] == 0).all(), info
        for w in range(len(wl.shapes)):
            _, _, _, rXL, rXR, rU, _ = refs[w][t]
            e_root = max(oracle.relative_frobenius(XL[w].cpu().numpy(), rXL),
                         oracle.relative_frobenius(XR[w].cpu().numpy(), rXR))
            e_u = oracle.relative_frobenius(U[w].cpu().numpy(), rU)
            worst = [max(worst[0], e_root), max(worst[1], e_u)]
            assert e_root <= ROOT_TOL and e_u <= UPDATE_TOL, (t, w, e_root, e_u)
    print(f"toy ({method}) worst root err {worst[0]:.3e} update err {worst[1]:.3e}")


@pytest.mark.parametrize("method", ["auto", "newton", "newton_f32"])
def test_small_transformer_like_end_to_end(torch_dev, method):
    """Low-rank gradients on ragged shapes above the Jacobi size, 3 steps."""
    torch, dev = torch_dev
    shapes = [(160, 160), (160, 644), (644, 160), (96, 260)]
    steps = [[W.gradient("w1024", w, t, shape=shapes[w]) for w in range(len(shapes))] for t in (1, 2, 3)]
    refs = [list(oracle.run_sequence([steps[t][w] for t in range(3)], 0.95, 1e-6)) for w in range(len(shapes))]
    for t, (XL, XR, U, info) in enumerate(run_pipeline(torch, dev, steps, 0.95, 1e-6, method=method)):
        assert (info["flags"] == 0).all(), info
        for w in range(len(shapes)):
            _, _, _, rXL, rXR, rU, _ = refs[w][t]
            e_root = max(oracle.relative_frobenius(XL[w].cpu().numpy(), rXL),
                         oracle.relative_frobenius(XR[w].cpu().numpy(), rXR))
            e_u = oracle.relative_frobenius(U[w].cpu().numpy(), rU)
            assert e_root <= ROOT_TOL and e_u <= UPDATE_TOL, (t, w, shapes[w], e_root, e_u)


# ------------------------------------------------------------- properties
def test_determinism_and_power_of_two_scaling(torch_dev):
    torch, dev = torch_dev
    shapes = [(64, 128), (160, 260)]
    steps = [[W.gradient("toy", w, t, shape=shapes[w]) for w in range(2)] for t in (1, 2)]
    a = [tuple(x.cpu().clone() for x in (XL + XR + U)) for XL, XR, U, _ in run_pipeline(torch, dev, steps, 0.9, 1e-6)]
    b = [tuple(x.cpu().clone() for x in (XL + XR + U)) for XL, XR, U, _ in run_pipeline(torch, dev, steps, 0.9, 1e-6)]
    for ra, rb in zip(a, b):
        for x, y in zip(ra, rb):
            assert torch.equal(x, y)
    scaled = [[np.float32(8.0) * g for g in s] for s in steps]
    c = [tuple(x.cpu().clone() for x in (XL + XR + U)) for XL, XR, U, _ in run_pipeline(torch, dev, scaled, 0.9, 1e-6)]
    for ra, rc in zip(a, c):
        for k in range(4):  # roots identical
            assert torch.equal(ra[k], rc[k])
        for k in range(4, 6):  # U scales exactly
            assert torch.equal(8.0 * ra[k], rc[k])
