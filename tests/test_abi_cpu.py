"""C ABI checks that need no GPU: the library loads, exports every symbol of
include/matrix_roots.h, and rejects invalid arguments before enqueuing
anything (validation never dereferences the device pointers it is given)."""

import ctypes
import json
import os
import re
import subprocess

import numpy as np
import pytest

from matrix_roots_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "matrix_roots.h")

# fake, never-dereferenced "device" addresses, far apart and 256-byte aligned
P1, P2, P3, P4, P5 = (0x10000000 * k for k in range(1, 6))


@pytest.fixture(scope="module")
def lib():
    return B.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)
    kw = {"if", "while", "sizeof", "defined", "return"}
    return sorted({n for n in names if n not in kw})


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(B.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_abi_version_and_strings(lib):
    assert lib.mr_abi_version() == 3
    for s in range(9):
        assert lib.mr_status_string(s)
    assert b"unknown" in lib.mr_status_string(99)


def test_newton_iteration_count_matches_okls_page(lib):
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "okls_coupled_ns_iterations.json")))
    k = lib.mr_newton_iterations(g["p"], g["m0"], g["tol"])
    assert k in g["accept"], k
    assert lib.mr_newton_iterations(3, 0.5, 1e-3) == -1
    assert lib.mr_newton_iterations(4, 0.0, 1e-3) == -1
    assert lib.mr_newton_iterations(4, 1.0, 1e-3) == 0
    # p = 4 converges from 1e-6 faster than p = 2 per iteration count
    assert lib.mr_newton_iterations(4, 1e-6, 1e-6) < lib.mr_newton_iterations(2, 1e-6, 1e-6)


def gram(m, n, G=P1, ldg=None, L=P2, ldl=None, R=P3, ldr=None):
    return B.GramProblem(m, n, G, ldg if ldg is not None else n, L, ldl if ldl is not None else m, R,
                         ldr if ldr is not None else n)


def call_gram(lib, probs, count=None, dt=B.MR_F64, beta=0.9, sides=3):
    arr = (B.GramProblem * max(len(probs), 1))(*probs)
    c = len(probs) if count is None else count
    return lib.gram_ema_update(ctypes.addressof(arr) if probs else None, c, dt, beta, sides, None, 0, None)


def test_gram_validation(lib):
    assert call_gram(lib, [], count=0) == B.MR_OK  # empty batch is a no-op
    assert call_gram(lib, [gram(4, 4)], count=-1) == 4
    assert lib.gram_ema_update(None, 1, B.MR_F64, 0.9, 3, None, 0, None) == 1
    assert call_gram(lib, [gram(4, 4)], dt=7) == 4
    assert call_gram(lib, [gram(4, 4)], beta=1.0) == 4
    assert call_gram(lib, [gram(4, 4)], beta=-0.1) == 4
    assert call_gram(lib, [gram(4, 4)], beta=float("nan")) == 4
    assert call_gram(lib, [gram(4, 4)], sides=0) == 4
    assert call_gram(lib, [gram(4, 4)], sides=4) == 4
    assert call_gram(lib, [gram(0, 4)]) == 2
    assert call_gram(lib, [gram(4, 70000)]) == 2
    assert call_gram(lib, [gram(4, 4, G=0)]) == 1
    assert call_gram(lib, [gram(4, 4, L=0)]) == 1
    assert call_gram(lib, [gram(4, 4, L=0)], sides=B.MR_RIGHT) != 1  # L unused
    assert call_gram(lib, [gram(4, 8, ldg=7)]) == 3
    assert call_gram(lib, [gram(4, 8, ldl=3)]) == 3
    assert call_gram(lib, [gram(4, 8, ldr=7)]) == 3
    assert call_gram(lib, [gram(4, 8, L=P1 + 16)]) == 8  # L inside G
    assert call_gram(lib, [gram(4, 8, R=P2 + 8)]) == 8  # R overlaps L
    assert call_gram(lib, [gram(4, 8, L=P2 + 4)]) == 4  # misaligned float64 state
    # the second problem is bad: nothing may be enqueued for the first either
    assert call_gram(lib, [gram(4, 4), gram(4, 4, G=0)]) == 1
    assert b"problem 1" in lib.mr_last_error_message()


def root(d, A=P1, lda=None, X=P2, ldx=None):
    return B.RootProblem(d, A, lda if lda is not None else d, X, ldx if ldx is not None else d)


def call_root(lib, probs, dt=B.MR_F32, eps=1e-6, norm=1, method=0, ws=None, ws_bytes=0):
    arr = (B.RootProblem * len(probs))(*probs)
    return lib.inv_quarter_root_batched(ctypes.addressof(arr), len(probs), dt, eps, norm, method, None, ws, ws_bytes,
                                        None)


def test_root_validation(lib):
    assert call_root(lib, [root(8)], eps=0.0) == 4
    assert call_root(lib, [root(8)], eps=float("inf")) == 4
    assert call_root(lib, [root(8)], norm=2) == 4
    assert call_root(lib, [root(8)], method=9) == 4
    assert call_root(lib, [root(8)], dt=3) == 4
    assert call_root(lib, [root(0)]) == 2
    assert call_root(lib, [root(8, A=0)]) == 1
    assert call_root(lib, [root(8, lda=7)]) == 3
    assert call_root(lib, [root(8, ldx=4)]) == 3
    assert call_root(lib, [root(8, X=P1 + 64)]) == 8
    assert call_root(lib, [root(200)], method=B.MR_JACOBI) == 7
    # valid request, no workspace: rejected before any launch
    assert call_root(lib, [root(200)]) == 5
    probs = (B.RootProblem * 2)(root(64), root(300, A=P3, X=P4))
    need = lib.inv_quarter_root_batched_workspace(ctypes.addressof(probs), 2, B.MR_F32, 0)
    assert need >= 40 * 300 * 300  # the d = 64 Jacobi root keeps its eigenvectors in LDS
    probs128 = (B.RootProblem * 1)(root(128))
    need128 = lib.inv_quarter_root_batched_workspace(ctypes.addressof(probs128), 1, B.MR_F32, B.MR_JACOBI)
    assert need128 >= 8 * 128 * 128  # ... a d = 128 one in the workspace
    assert call_root(lib, [root(64), root(300, A=P3, X=P4)], ws=P5, ws_bytes=need - 1) == 5
    assert call_root(lib, [root(64), root(300, A=P3, X=P4)], ws=P5 + 8, ws_bytes=need) == 5


def test_noalloc_root_validation(lib):
    """The allocation-free root rejects invalid arguments like the workspace
    call, and a batch whose workspace exceeds its scratch array with
    MR_ERR_WORKSPACE, before it touches any device."""
    def call(ps, eps=1e-6):
        probs = (B.RootProblem * len(ps))(*ps)
        return lib.inv_quarter_root_batched_noalloc(ctypes.addressof(probs), len(ps), B.MR_F32, eps,
                                                    B.MR_NORM_TRACE, B.MR_AUTO, None, None)
    assert call([root(8)], eps=0.0) == 4
    assert call([root(0)]) == 2
    assert call([root(8, X=P1 + 64)]) == 8
    assert call([root(1024)]) == 5
    assert b"scratch" in lib.mr_last_error_message()
    probs = (B.RootProblem * 1)(root(920))
    assert lib.inv_quarter_root_batched_workspace(ctypes.addressof(probs), 1, B.MR_F32, 0) > B.NOALLOC_SCRATCH_BYTES
    assert call([root(920)]) == 5


def apply_p(m, n, XL=P1, G=P2, XR=P3, U=P4, ldu=None):
    return B.ApplyProblem(m, n, XL, m, G, n, XR, n, U, ldu if ldu is not None else n)


def test_apply_validation(lib):
    def call(probs, alpha=1.0, ws=None, ws_bytes=0):
        arr = (B.ApplyProblem * len(probs))(*probs)
        return lib.precondition_apply(ctypes.addressof(arr), len(probs), alpha, ws, ws_bytes, None)

    assert call([apply_p(4, 8)], alpha=float("nan")) == 4
    assert call([apply_p(0, 8)]) == 2
    assert call([apply_p(4, 8, XR=0)]) == 1
    assert call([apply_p(4, 8, ldu=7)]) == 3
    assert call([apply_p(4, 8, U=P2 + 4)]) == 8
    arr = (B.ApplyProblem * 1)(apply_p(4, 8))
    need = lib.precondition_apply_workspace(ctypes.addressof(arr), 1)
    # split copies (4 bytes per element) of XR (8 x 32), G (4 x 32), XL (4 x 32)
    # and W^T (8 x 32), rows padded to 32 columns; W^T in float32 (8 x 4) and
    # the 4 operands' largest magnitudes: arrays 256-byte aligned
    assert need == 4 * (8 * 32 + 4 * 32 + 4 * 32 + 8 * 32) + 256 + 256
    assert call([apply_p(4, 8)], ws=None, ws_bytes=0) == 5


def test_newton_schedule_converges_every_eigenvalue(lib):
    """For the library's step scales, every eigenvalue m0 <= m <= 1/1.01 of
    M0 ends with x_K = m^(-1/4) to 1e-6: each step maps m -> g(m/s),
    x -> x s^(-1/4) (5 - m/s)/4, g(y) = y((5-y)/4)^4; with the plain last step
    x_K^4 m = m_K is within 1e-6 of 1, and a Taylor finish of degree n takes
    x -> x sum_{k<=n} c_k (1-m)^k with c_k the binomial coefficients of
    (1-e)^(-1/4), c_k = c_{k-1} (k - 3/4)/k.  Written here from the
    iteration's definition, independent of the library."""
    import numpy as np

    degrees = set()
    for m0 in (0.9, 0.5, 1e-2, 1e-3, 1e-4, 1e-5, 1e-6, 3e-7, 1e-8, 1e-10, 1e-14):
        scales, j, fin = B.newton_schedule(m0, final_degree=True)
        K = len(scales)
        assert 1 <= K <= 40 and 0 <= j <= K and fin in (1, 2, 4)
        degrees.add(fin)
        m = np.concatenate([np.geomspace(m0, 1 / 1.01, 4000), [m0, 1 / 1.01]])
        m_init = m.copy()
        x = np.ones_like(m)
        for t, s in enumerate(scales):
            if t == K - 1 and fin > 1:
                assert t >= max(j, 1)  # finishes run in the split steps
                c = [1.0]
                for k in range(1, fin + 1):
                    c.append(c[-1] * (k - 0.75) / k)
                e = 1.0 - m
                x = x * sum(ck * e ** k for k, ck in enumerate(c))
                break
            y = m / s
            x = x * s ** -0.25 * (5.0 - y) / 4.0
            m = y * ((5.0 - y) / 4.0) ** 4
            if t + 1 == j:
                assert m.min() >= 5e-4 * (1 - 1e-12)  # float32 steps start at a floor >= 5e-4
        if fin == 1:
            assert np.max(np.abs(1.0 - m)) <= 1.01e-6, (m0, np.max(np.abs(1 - m)))
        assert np.max(np.abs(x * m_init ** 0.25 - 1.0)) <= 1e-6, (m0, fin)
    assert degrees >= {2, 4}, degrees  # both finishes occur over these floors


def test_newton_schedule_monotone_in_floor(lib):
    """A larger eigenvalue floor never needs more steps, nor more float64
    steps: the host launches the schedule of the smallest floor it covers
    (and a matrix below it runs that schedule), so every matrix's steps and
    float64 steps must fit under it."""
    prev = None
    for m0 in np.geomspace(1e-30, 0.99, 2000):
        s, j = B.newton_schedule(float(m0))  # with the finishing rule
        K = len(s)
        if prev is not None:
            assert K <= prev[0] and j <= prev[1], (m0, K, j, prev)
        prev = (K, j)
    # the scaled schedule beats the classical count (same tolerance)
    assert len(B.newton_schedule(1e-6)[0]) < lib.mr_newton_iterations(4, 1e-6, 1e-6)


def call_sqrt(lib, probs, dt=B.MR_F32, eps=0.0, norm=0, prec=0, ws=None, ws_bytes=0):
    arr = (B.RootProblem * len(probs))(*probs)
    return lib.inv_sqrt_root_batched(ctypes.addressof(arr), len(probs), dt, eps, norm, prec, None, ws, ws_bytes,
                                     None)


def test_sqrt_root_validation(lib):
    assert call_sqrt(lib, [root(8)], eps=-1e-3) == 4
    assert call_sqrt(lib, [root(8)], eps=float("nan")) == 4
    assert call_sqrt(lib, [root(8)], norm=2) == 4
    assert call_sqrt(lib, [root(8)], prec=2) == 4
    assert call_sqrt(lib, [root(8)], dt=3) == 4
    assert call_sqrt(lib, [root(0)]) == 2
    assert call_sqrt(lib, [root(8, X=0)]) == 1
    assert call_sqrt(lib, [root(8, lda=7)]) == 3
    assert call_sqrt(lib, [root(8, X=P1 + 64)]) == 8
    arr = (B.RootProblem * 0)()
    assert lib.inv_sqrt_root_batched(ctypes.addressof(arr), 0, 0, 0.0, 0, 0, None, None, 0, None) == 0
    # eps = 0 is valid here (the page's S^(-1/2)); no workspace: rejected before any launch
    assert call_sqrt(lib, [root(200)]) == 5
    probs = (B.RootProblem * 2)(root(64), root(300, A=P3, X=P4))
    need = lib.inv_sqrt_root_batched_workspace(ctypes.addressof(probs), 2, B.MR_F32, 0)
    assert need >= 24 * (300 * 300 + 64 * 64)
    assert call_sqrt(lib, [root(64), root(300, A=P3, X=P4)], ws=P5, ws_bytes=need - 1) == 5
    assert call_sqrt(lib, [root(64), root(300, A=P3, X=P4)], ws=P5 + 8, ws_bytes=need) == 5


def test_cans_ceilings_match_okls_page():
    """The library's step bounds (from which its fp16 scales follow) against
    the ceilings the OKLS page prints for its coefficient table."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "okls_cans_table.json")))
    y, z, p = B.cans_ceilings()
    assert len(y) == len(z) == len(p) == g["steps"] + 1
    for k in range(g["steps"] + 1):
        assert z[k] == pytest.approx(g["z_ceilings"][k], rel=2e-4), k
        assert p[k] == pytest.approx(g["p_ceilings"][k], rel=1e-2), k
        assert y[k] <= g["y_ceilings"][k] * 1.005, k


def test_packed_validation(lib):
    """MR_PACKED: leading dimensions ignored, ranges of d(d+1)/2 elements."""
    F64P = B.MR_F64 | B.MR_PACKED
    assert call_gram(lib, [gram(4, 8, ldl=0, ldr=0)], dt=F64P) != 3  # ld ignored when packed
    assert call_gram(lib, [gram(4, 8)], dt=B.MR_F64 | 32) == 4
    assert call_gram(lib, [gram(4, 8)], dt=2 | B.MR_PACKED) == 4
    # packed L of m=4 spans 10 doubles = 80 bytes from P2: R at P2 + 72 overlaps, at P2 + 80 does not
    assert call_gram(lib, [gram(4, 8, R=P2 + 72)], dt=F64P) == 8
    assert call_gram(lib, [gram(4, 8, R=P2 + 80)], dt=F64P) != 8
    assert call_root(lib, [root(8, lda=0)], dt=B.MR_F32 | B.MR_PACKED) == 5  # valid; only the workspace is missing
    assert call_root(lib, [root(8, lda=0)], dt=B.MR_F32) == 3
    # packed A of d=8 spans 36 floats = 144 bytes from P1
    assert call_root(lib, [root(8, X=P1 + 140)], dt=B.MR_F32 | B.MR_PACKED) == 8
    assert call_root(lib, [root(8, X=P1 + 144)], dt=B.MR_F32 | B.MR_PACKED) == 5
    assert call_sqrt(lib, [root(8, lda=0)], dt=B.MR_F64 | B.MR_PACKED) == 5


def test_pack_helpers_roundtrip():
    import torch

    A = torch.randn(7, 7, dtype=torch.float64)
    A = A + A.T
    P = B.pack_upper(A)
    assert P.numel() == 28 and B.packed_dim(28) == 7
    # row-packed upper triangle: row i holds columns i..d-1
    assert P[0].item() == A[0, 0].item() and P[7].item() == A[1, 1].item() and P[27].item() == A[6, 6].item()
    assert torch.equal(B.unpack_upper(P), A)
    with pytest.raises(ValueError):
        B.packed_dim(27)


def test_polar_validation(lib):
    def call(probs, prec=0, ws=None, ws_bytes=0):
        arr = (B.PolarProblem * len(probs))(*probs)
        return lib.polar_cans_batched(ctypes.addressof(arr), len(probs), prec, None, ws, ws_bytes, None)

    def pp(m, n, G=P1, ldg=None, O=P2, ldo=None):
        return B.PolarProblem(m, n, G, ldg if ldg is not None else n, O, ldo if ldo is not None else n)

    assert call([pp(8, 4)], prec=5) == 4
    assert call([pp(0, 4)]) == 2
    assert call([pp(8, 70000)]) == 2
    assert call([pp(8, 4, O=0)]) == 1
    assert call([pp(8, 4, ldg=3)]) == 3
    assert call([pp(8, 4, ldo=3)]) == 3
    assert call([pp(8, 4, O=P1 + 100)]) == 8
    assert call([pp(8, 4, G=P1 + 2)]) == 4
    assert call([pp(8, 4)]) == 5  # valid; no workspace
    arr = (B.PolarProblem * 2)(pp(300, 100), pp(64, 200, G=P3, O=P4))
    need = lib.polar_cans_batched_workspace(ctypes.addressof(arr), 2, 0)
    assert need >= 4 * (3 * 300 * 100 + 100 * 100) + 4 * (3 * 200 * 64 + 64 * 64)
    assert call([pp(300, 100), pp(64, 200, G=P3, O=P4)], ws=P5, ws_bytes=need - 1) == 5


def test_momentum_and_hyperball_validation(lib):
    def mom(probs, mu=0.9):
        arr = (B.MomentumProblem * len(probs))(*probs)
        return lib.momentum_ema_batched(ctypes.addressof(arr), len(probs), mu, None)

    def hyp(probs, lr=0.1, ws=None, ws_bytes=0):
        arr = (B.HyperballProblem * len(probs))(*probs)
        return lib.hyperball_update_batched(ctypes.addressof(arr), len(probs), lr, None, ws, ws_bytes, None)

    assert mom([B.MomentumProblem(4, 8, P1, 8, P2, 8)], mu=1.0) == 4
    assert mom([B.MomentumProblem(4, 8, P1, 8, P2, 8)], mu=-0.1) == 4
    assert mom([B.MomentumProblem(0, 8, P1, 8, P2, 8)]) == 2
    assert mom([B.MomentumProblem(4, 8, 0, 8, P2, 8)]) == 1
    assert mom([B.MomentumProblem(4, 8, P1, 7, P2, 8)]) == 3
    assert mom([B.MomentumProblem(4, 8, P1, 8, P1 + 64, 8)]) == 8
    assert hyp([B.HyperballProblem(4, 8, P1, 8, P2, 8)], lr=float("inf")) == 4
    assert hyp([B.HyperballProblem(4, 8, P1, 8, P2, 8)], lr=-1.0) == 4
    assert hyp([B.HyperballProblem(4, 8, P1, 8, P1 + 4, 8)]) == 8
    assert hyp([B.HyperballProblem(4, 8, P1, 8, P2, 8)]) == 5  # valid; no workspace
    arr = (B.HyperballProblem * 2)(B.HyperballProblem(4096, 1024, P1, 1024, P2, 1024),
                                   B.HyperballProblem(3, 5, P3, 5, P4, 5))
    need = lib.hyperball_update_batched_workspace(ctypes.addressof(arr), 2)
    assert need >= 3 * 8 * 512 * 2  # 512 workgroups of 8 rows for the 4096 x 1024 matrix


def test_measure_peaks_rejects_null(lib):
    """mr_measure_peaks validates its output pointer before any HIP call."""
    assert lib.mr_measure_peaks(None, None) == 1  # MR_ERR_NULL
    assert "NULL" in lib.mr_last_error_message().decode()


def test_aliasing_across_problems_is_rejected(lib):
    """Validation covers the whole batch: an output of one problem may not
    overlap an output or input of another (inputs may be shared).  Every case
    is rejected with MR_ERR_ALIAS before anything is enqueued."""
    Q = 0x1000  # 4 KiB apart: an 8 x 8 float64 or a 16 x 16 float32 matrix fits in between
    # Gram EMA: two problems updating one state; a state inside another problem's gradient
    assert call_gram(lib, [gram(8, 8, G=P1, L=P2, R=P3), gram(8, 8, G=P1 + Q, L=P2, R=P3 + Q)]) == 8
    assert b"overlaps" in lib.mr_last_error_message()
    assert call_gram(lib, [gram(8, 8, G=P1, L=P2, R=P3), gram(8, 8, G=P2, L=P4, R=P5)]) == 8
    # roots: X_1 over A_0, X_0 over X_1; a shared input is fine (then: no workspace)
    assert call_root(lib, [root(8, A=P1, X=P2), root(8, A=P3, X=P1 + 64)]) == 8
    assert call_root(lib, [root(8, A=P1, X=P2), root(8, A=P3, X=P2 + 128)]) == 8
    assert call_root(lib, [root(8, A=P1, X=P2), root(8, A=P1, X=P3)]) == 5
    assert call_sqrt(lib, [root(8, A=P1, X=P2), root(8, A=P3, X=P1)]) == 8
    # apply: U_1 over XR_0; U_0 over U_1; shared roots are fine
    assert lib.precondition_apply(ctypes.addressof((B.ApplyProblem * 2)(
        apply_p(8, 8, XL=P1, G=P2, XR=P3, U=P4), apply_p(8, 8, XL=P1 + Q, G=P2 + Q, XR=P3 + Q, U=P3))),
        2, 1.0, None, 0, None) == 8
    assert lib.precondition_apply(ctypes.addressof((B.ApplyProblem * 2)(
        apply_p(8, 8, U=P4), apply_p(8, 8, U=P4 + 32))), 2, 1.0, None, 0, None) == 8
    assert lib.precondition_apply(ctypes.addressof((B.ApplyProblem * 2)(
        apply_p(8, 8, U=P4), apply_p(8, 8, U=P5))), 2, 1.0, None, 0, None) == 5
    # polar, momentum, hyperball
    arr = (B.PolarProblem * 2)(B.PolarProblem(8, 4, P1, 4, P2, 4), B.PolarProblem(8, 4, P3, 4, P1, 4))
    assert lib.polar_cans_batched(ctypes.addressof(arr), 2, 0, None, None, 0, None) == 8
    arr = (B.MomentumProblem * 2)(B.MomentumProblem(4, 8, P1, 8, P2, 8), B.MomentumProblem(4, 8, P3, 8, P2, 8))
    assert lib.momentum_ema_batched(ctypes.addressof(arr), 2, 0.9, None) == 8
    arr = (B.HyperballProblem * 2)(B.HyperballProblem(4, 8, P1, 8, P2, 8), B.HyperballProblem(4, 8, P2, 8, P3, 8))
    assert lib.hyperball_update_batched(ctypes.addressof(arr), 2, 0.1, None, None, 0, None) == 8


def test_empty_batches_are_no_ops(lib):
    """count = 0 returns MR_OK without touching the device (NULL arrays
    allowed); a negative count is a parameter error."""
    assert lib.inv_quarter_root_batched(None, 0, B.MR_F32, 1e-6, B.MR_NORM_TRACE, B.MR_AUTO, None, None, 0, None) == 0
    assert lib.inv_quarter_root_batched_workspace(None, 0, B.MR_F32, B.MR_AUTO) == 0
    assert lib.inv_quarter_root_batched_noalloc(None, 0, B.MR_F32, 1e-6, B.MR_NORM_TRACE, B.MR_AUTO, None,
                                                None) == 0
    assert lib.precondition_apply(None, 0, 1.0, None, 0, None) == 0
    assert lib.precondition_apply_workspace(None, 0) == 0
    assert lib.inv_sqrt_root_batched(None, 0, B.MR_F32, 1e-3, 0, 0, None, None, 0, None) == 0
    assert lib.polar_cans_batched(None, 0, 0, None, None, 0, None) == 0
    assert lib.momentum_ema_batched(None, 0, 0.9, None) == 0
    assert lib.hyperball_update_batched(None, 0, 0.1, None, None, 0, None) == 0
    assert lib.inv_quarter_root_batched(None, -1, B.MR_F32, 1e-6, B.MR_NORM_TRACE, B.MR_AUTO, None, None, 0,
                                        None) == 4
