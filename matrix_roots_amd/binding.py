"""ctypes binding of libmatrix_roots.so (include/matrix_roots.h).

Argument marshalling only: torch tensors provide device memory and the
current stream; every step of the computation runs in the library's HIP
kernels.  A missing library raises; there is no other code path.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmatrix_roots.so")

MR_OK = 0
MR_F32, MR_F64 = 0, 1
MR_LEFT, MR_RIGHT = 1, 2
MR_NORM_NONE, MR_NORM_TRACE = 0, 1
MR_AUTO, MR_JACOBI, MR_NEWTON, MR_NEWTON_F64, MR_NEWTON_F32 = 0, 1, 2, 3, 4
MR_INFO_NONFINITE, MR_INFO_ZERO_TRACE, MR_INFO_NOT_PD, MR_INFO_NOT_CONVERGED = 1, 2, 4, 8
MR_CANS_F16, MR_CANS_SPLIT = 0, 1
MR_PACKED = 16

_METHODS = {"auto": MR_AUTO, "jacobi": MR_JACOBI, "newton": MR_NEWTON, "newton_f64": MR_NEWTON_F64,
            "newton_f32": MR_NEWTON_F32}
_NORMS = {"none": MR_NORM_NONE, "trace": MR_NORM_TRACE}
_PRECISIONS = {"f16": MR_CANS_F16, "split": MR_CANS_SPLIT}

EXPORTED = (
    "gram_ema_update",
    "gram_ema_update_workspace",
    "inv_quarter_root_batched",
    "inv_quarter_root_batched_workspace",
    "inv_quarter_root_batched_noalloc",
    "inv_sqrt_root_batched",
    "inv_sqrt_root_batched_workspace",
    "mr_cans_ceilings",
    "polar_cans_batched",
    "polar_cans_batched_workspace",
    "momentum_ema_batched",
    "hyperball_update_batched",
    "hyperball_update_batched_workspace",
    "precondition_apply",
    "precondition_apply_workspace",
    "mr_newton_iterations",
    "mr_newton_schedule",
    "mr_measure_peaks",
    "mr_trace_enable",
    "mr_trace_collect",
    "mr_set_jacobi_max_sweeps",
    "mr_status_string",
    "mr_last_error_message",
    "mr_abi_version",
)


class GramProblem(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("G", ctypes.c_void_p), ("ldg", ctypes.c_int64),
                ("L", ctypes.c_void_p), ("ldl", ctypes.c_int64), ("R", ctypes.c_void_p), ("ldr", ctypes.c_int64)]


class RootProblem(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int64), ("A", ctypes.c_void_p), ("lda", ctypes.c_int64), ("X", ctypes.c_void_p),
                ("ldx", ctypes.c_int64)]


class PolarProblem(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("G", ctypes.c_void_p), ("ldg", ctypes.c_int64),
                ("O", ctypes.c_void_p), ("ldo", ctypes.c_int64)]


class MomentumProblem(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("G", ctypes.c_void_p), ("ldg", ctypes.c_int64),
                ("M", ctypes.c_void_p), ("ldm", ctypes.c_int64)]


class HyperballProblem(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("W", ctypes.c_void_p), ("ldw", ctypes.c_int64),
                ("U", ctypes.c_void_p), ("ldu", ctypes.c_int64)]


class ApplyProblem(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("n", ctypes.c_int64), ("XL", ctypes.c_void_p), ("ldxl", ctypes.c_int64),
                ("G", ctypes.c_void_p), ("ldg", ctypes.c_int64), ("XR", ctypes.c_void_p), ("ldxr", ctypes.c_int64),
                ("U", ctypes.c_void_p), ("ldu", ctypes.c_int64)]


ROOT_INFO_DTYPE = np.dtype([("scale", "<f8"), ("bound", "<f8"), ("iters", "<i4"), ("fp64_iters", "<i4"),
                            ("residual", "<f4"), ("flags", "<u4"), ("final_degree", "<i4"), ("reserved", "<i4")])
ROOT_INFO_BYTES = ROOT_INFO_DTYPE.itemsize
assert ROOT_INFO_BYTES == 40


class TraceRecord(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


class MatrixRootsError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


_lib = None


def library() -> ctypes.CDLL:
    """Load libmatrix_roots.so (built in-tree by matrix_roots_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m matrix_roots_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz, f32, f64, u32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                      ctypes.c_float, ctypes.c_double, ctypes.c_uint32)
    lib.gram_ema_update.argtypes = [vp, i32, i32, f64, u32, vp, sz, vp]
    lib.gram_ema_update.restype = i32
    lib.gram_ema_update_workspace.argtypes = [vp, i32, i32, u32]
    lib.gram_ema_update_workspace.restype = sz
    lib.inv_quarter_root_batched.argtypes = [vp, i32, i32, f64, i32, i32, vp, vp, sz, vp]
    lib.inv_quarter_root_batched.restype = i32
    lib.inv_quarter_root_batched_workspace.argtypes = [vp, i32, i32, i32]
    lib.inv_quarter_root_batched_workspace.restype = sz
    lib.inv_quarter_root_batched_noalloc.argtypes = [vp, i32, i32, f64, i32, i32, vp, vp]
    lib.inv_quarter_root_batched_noalloc.restype = i32
    lib.inv_sqrt_root_batched.argtypes = [vp, i32, i32, f64, i32, i32, vp, vp, sz, vp]
    lib.inv_sqrt_root_batched.restype = i32
    lib.inv_sqrt_root_batched_workspace.argtypes = [vp, i32, i32, i32]
    lib.inv_sqrt_root_batched_workspace.restype = sz
    lib.mr_cans_ceilings.argtypes = [vp, vp, vp, i32]
    lib.mr_cans_ceilings.restype = i32
    lib.polar_cans_batched.argtypes = [vp, i32, i32, vp, vp, sz, vp]
    lib.polar_cans_batched.restype = i32
    lib.polar_cans_batched_workspace.argtypes = [vp, i32, i32]
    lib.polar_cans_batched_workspace.restype = sz
    lib.mr_measure_peaks.argtypes = [vp, vp]
    lib.mr_measure_peaks.restype = i32
    lib.momentum_ema_batched.argtypes = [vp, i32, f64, vp]
    lib.momentum_ema_batched.restype = i32
    lib.hyperball_update_batched.argtypes = [vp, i32, f64, vp, vp, sz, vp]
    lib.hyperball_update_batched.restype = i32
    lib.hyperball_update_batched_workspace.argtypes = [vp, i32]
    lib.hyperball_update_batched_workspace.restype = sz
    lib.precondition_apply.argtypes = [vp, i32, f32, vp, sz, vp]
    lib.precondition_apply.restype = i32
    lib.precondition_apply_workspace.argtypes = [vp, i32]
    lib.precondition_apply_workspace.restype = sz
    lib.mr_newton_iterations.argtypes = [i32, f64, f64]
    lib.mr_newton_iterations.restype = i32
    lib.mr_newton_schedule.argtypes = [f64, vp, i32, vp, vp]
    lib.mr_newton_schedule.restype = i32
    lib.mr_trace_enable.argtypes = [i32]
    lib.mr_trace_enable.restype = i32
    lib.mr_trace_collect.argtypes = [vp, i32]
    lib.mr_trace_collect.restype = i32
    lib.mr_set_jacobi_max_sweeps.argtypes = [i32]
    lib.mr_set_jacobi_max_sweeps.restype = i32
    lib.mr_status_string.argtypes = [i32]
    lib.mr_status_string.restype = ctypes.c_char_p
    lib.mr_last_error_message.argtypes = []
    lib.mr_last_error_message.restype = ctypes.c_char_p
    lib.mr_abi_version.argtypes = []
    lib.mr_abi_version.restype = i32
    if lib.mr_abi_version() != 3:
        raise RuntimeError("libmatrix_roots.so ABI version mismatch")
    _lib = lib
    return lib


def _check(status: int):
    if status != MR_OK:
        lib = library()
        raise MatrixRootsError(status, lib.mr_last_error_message().decode())


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _ld(t) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("matrices must be 2-D with unit column stride")
    return int(t.stride(0))


def packed_dim(n: int) -> int:
    """d with d (d + 1) / 2 == n (the size of a packed symmetric matrix)."""
    d = int((np.sqrt(8.0 * n + 1.0) - 1.0) / 2.0 + 0.5)
    if d * (d + 1) // 2 != n:
        raise ValueError(f"{n} elements is not a packed symmetric matrix")
    return d


def _sym(t):
    """(d, leading dimension, packed) of a symmetric-matrix argument: a 2-D
    (d, d) tensor (full storage) or a 1-D tensor of d (d + 1) / 2 elements
    (upper triangle packed by rows, MR_PACKED)."""
    if t.dim() == 1:
        if t.stride(0) != 1:
            raise ValueError("packed matrices must be contiguous")
        return packed_dim(t.numel()), 0, True
    if t.shape[0] != t.shape[1]:
        raise ValueError("symmetric matrices must be square")
    return int(t.shape[0]), _ld(t), False


def pack_upper(A):
    """Packed copy (upper triangle by rows) of a full symmetric tensor --
    host-side indexing with torch, for tests and callers converting state."""
    import torch

    d = A.shape[0]
    i, j = torch.triu_indices(d, d, device=A.device)
    return A[i, j].contiguous()


def unpack_upper(P):
    """Full symmetric tensor from a packed one (torch indexing)."""
    import torch

    d = packed_dim(P.numel())
    i, j = torch.triu_indices(d, d, device=P.device)
    A = torch.empty(d, d, dtype=P.dtype, device=P.device)
    A[i, j] = P
    A[j, i] = P
    return A


def _stream(stream) -> int:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _in_use_on(stream, *tensors):
    """Tell torch's caching allocator that these tensors are used by work on
    `stream` (when it is not the current stream), so that their memory is not
    handed out again before that work ends."""
    if stream is None:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


def _workspace(nbytes: int, device):
    import torch

    if nbytes == 0:
        return None
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ API
def gram_ema_update(grads: Sequence, lefts: Optional[Sequence], rights: Optional[Sequence], beta: float,
                    stream=None):
    """In place: L <- beta L + (1-beta) G G^T, R <- beta R + (1-beta) G^T G.

    grads: float32 (m, n) device tensors; lefts / rights: (m, m) / (n, n)
    float32 or float64 tensors of one dtype, or None to skip that side.
    """
    lib = library()
    count = len(grads)
    sides = (MR_LEFT if lefts is not None else 0) | (MR_RIGHT if rights is not None else 0)
    states = [s for s in (lefts or []) + (rights or [])]
    dts = {str(s.dtype) for s in states}
    if len(dts) != 1:
        raise ValueError("all Gram states must share one dtype")
    dt = MR_F64 if dts.pop() == "torch.float64" else MR_F32
    layouts = {s.dim() == 1 for s in states}
    if len(layouts) != 1:
        raise ValueError("Gram states must be all full (2-D) or all packed (1-D)")
    packed = layouts.pop()
    if packed:
        dt |= MR_PACKED
    probs = (GramProblem * max(count, 1))()
    for i, G in enumerate(grads):
        L = lefts[i] if lefts is not None else None
        R = rights[i] if rights is not None else None
        for S, dim in ((L, G.shape[0]), (R, G.shape[1])):
            if S is not None and _sym(S)[0] != dim:
                raise ValueError("Gram state size does not match the gradient")
        probs[i] = GramProblem(G.shape[0], G.shape[1], _ptr(G), _ld(G), _ptr(L), _sym(L)[1] if L is not None else 0,
                               _ptr(R), _sym(R)[1] if R is not None else 0)
    _check(lib.gram_ema_update(ctypes.addressof(probs), count, dt, float(beta), sides, None, 0, _stream(stream)))


class RootWorkspace:
    """Reusable workspace + info buffer for inv_quarter_root_batched."""

    def __init__(self):
        self.buf = None
        self.info = None

    def get(self, nbytes: int, count: int, device):
        import torch

        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != torch.device(device):
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        if self.info is None or self.info.numel() < ROOT_INFO_BYTES * count or self.info.device != torch.device(device):
            self.info = torch.empty(ROOT_INFO_BYTES * max(count, 1), dtype=torch.uint8, device=device)
        return self.buf, self.info


def inv_quarter_root_batched(As: Sequence, eps: float, normalize: str = "trace", method: str = "auto",
                             Xs: Optional[Sequence] = None, workspace: Optional[RootWorkspace] = None,
                             stream=None, return_info: bool = True, info_out=None):
    """X_i = (A_i/s_i + eps I)^(-1/4) for every device tensor A_i: (d, d)
    full, or 1-D packed (upper triangle by rows, d (d + 1) / 2 elements).

    Returns (Xs, info) where info is a numpy structured array (fields of
    mr_root_info) read after synchronising the stream, or (Xs, None).
    info_out: optional device uint8 tensor of ROOT_INFO_BYTES*len(As) bytes that receives
    the info records instead of the workspace's buffer (no synchronisation
    when return_info is False); decode it later with decode_info().
    """
    lib = library()
    return _root_call(lib.inv_quarter_root_batched, lib.inv_quarter_root_batched_workspace, _METHODS[method], As,
                      eps, normalize, Xs, workspace, stream, return_info, info_out)


def _root_call(entry, size_entry, code, As, eps, normalize, Xs, workspace, stream, return_info, info_out):
    import torch

    lib = library()
    count = len(As)
    if count == 0:
        return [], None
    dts = {str(a.dtype) for a in As}
    if len(dts) != 1:
        raise ValueError("all A must share one dtype")
    dt = MR_F64 if dts.pop() == "torch.float64" else MR_F32
    syms = [_sym(a) for a in As]
    layouts = {p for _, _, p in syms}
    if len(layouts) != 1:
        raise ValueError("A must be all full (2-D) or all packed (1-D)")
    if layouts.pop():
        dt |= MR_PACKED
    dev = As[0].device
    own_x = Xs is None
    if own_x:
        Xs = [torch.empty(d, d, dtype=torch.float32, device=dev) for d, _, _ in syms]
    probs = (RootProblem * count)()
    for i, (A, X) in enumerate(zip(As, Xs)):
        probs[i] = RootProblem(syms[i][0], _ptr(A), syms[i][1], _ptr(X), _ld(X))
    need = size_entry(ctypes.addressof(probs), count, dt, code)
    ws = workspace or RootWorkspace()
    buf, info = ws.get(need, count, dev)
    if info_out is not None:
        if info_out.numel() < ROOT_INFO_BYTES * count:
            raise ValueError("info_out too small")
        info = info_out
    _in_use_on(stream, buf, info, *(Xs if own_x else ()))
    _check(entry(ctypes.addressof(probs), count, dt, float(eps), _NORMS[normalize], code, _ptr(info), _ptr(buf),
                 buf.numel(), _stream(stream)))
    if not return_info:
        return Xs, None
    torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()
    return Xs, decode_info(info, count)


NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024


def inv_quarter_root_batched_noalloc(As: Sequence, eps: float, Xs: Sequence, info_out, normalize: str = "trace",
                                     method: str = "auto", stream=None):
    """inv_quarter_root_batched with the library's own scratch array as the
    workspace: the caller passes the outputs Xs (float32 (d, d) device
    tensors) and info_out (device uint8 tensor of ROOT_INFO_BYTES*len(As)
    bytes, or None), and neither the library nor this wrapper allocates
    device memory.  Nothing is synchronised; decode info_out with
    decode_info() after the stream."""
    lib = library()
    count = len(As)
    if count == 0:
        return Xs
    dts = {str(a.dtype) for a in As}
    if len(dts) != 1:
        raise ValueError("all A must share one dtype")
    dt = MR_F64 if dts.pop() == "torch.float64" else MR_F32
    syms = [_sym(a) for a in As]
    layouts = {p for _, _, p in syms}
    if len(layouts) != 1:
        raise ValueError("A must be all full (2-D) or all packed (1-D)")
    if layouts.pop():
        dt |= MR_PACKED
    if len(Xs) != count:
        raise ValueError("one output per input")
    if info_out is not None and info_out.numel() < ROOT_INFO_BYTES * count:
        raise ValueError("info_out too small")
    probs = (RootProblem * count)()
    for i, (A, X) in enumerate(zip(As, Xs)):
        probs[i] = RootProblem(syms[i][0], _ptr(A), syms[i][1], _ptr(X), _ld(X))
    _check(lib.inv_quarter_root_batched_noalloc(ctypes.addressof(probs), count, dt, float(eps), _NORMS[normalize],
                                                _METHODS[method], _ptr(info_out), _stream(stream)))
    return Xs


def inv_sqrt_root_batched(As: Sequence, eps: float = 0.0, normalize: str = "none", precision: str = "f16",
                          Xs: Optional[Sequence] = None, workspace: Optional[RootWorkspace] = None,
                          stream=None, return_info: bool = True, info_out=None):
    """W_i = (sym(A_i)/s_i + eps I)^(-1/2) by the scaled CANS coupled
    Newton-Schulz iteration; precision "f16" (fp16 products) or "split"
    (float32-accurate split-fp16 products).  Returns (Ws, info) like
    inv_quarter_root_batched."""
    lib = library()
    return _root_call(lib.inv_sqrt_root_batched, lib.inv_sqrt_root_batched_workspace, _PRECISIONS[precision], As,
                      eps, normalize, Xs, workspace, stream, return_info, info_out)


def polar_cans_batched(Gs: Sequence, precision: str = "f16", Os: Optional[Sequence] = None,
                       workspace: Optional[RootWorkspace] = None, stream=None, return_info: bool = True,
                       info_out=None):
    """O_i = the ten CANS polar steps on G_i / sqrt(1.01 ||G_i||_F^2) (float32
    (m, n) device tensors): U phi(Sigma) V^T, the polar factor for singular
    values in the polynomials' range.  precision "f16" or "split".  Returns
    (Os, info) like inv_quarter_root_batched."""
    import torch

    lib = library()
    count = len(Gs)
    if count == 0:
        return [], None
    dev = Gs[0].device
    own_o = Os is None
    if own_o:
        Os = [torch.empty_like(G) for G in Gs]
    probs = (PolarProblem * count)()
    for i, (G, O) in enumerate(zip(Gs, Os)):
        probs[i] = PolarProblem(G.shape[0], G.shape[1], _ptr(G), _ld(G), _ptr(O), _ld(O))
    code = _PRECISIONS[precision]
    need = lib.polar_cans_batched_workspace(ctypes.addressof(probs), count, code)
    ws = workspace or RootWorkspace()
    buf, info = ws.get(need, count, dev)
    if info_out is not None:
        if info_out.numel() < ROOT_INFO_BYTES * count:
            raise ValueError("info_out too small")
        info = info_out
    _in_use_on(stream, buf, info, *(Os if own_o else ()))
    _check(lib.polar_cans_batched(ctypes.addressof(probs), count, code, _ptr(info), _ptr(buf), buf.numel(),
                                  _stream(stream)))
    if not return_info:
        return Os, None
    torch.cuda.current_stream().synchronize() if stream is None else stream.synchronize()
    return Os, decode_info(info, count)


def momentum_ema_batched(Gs: Sequence, Ms: Sequence, mu: float, stream=None):
    """In place: M_i <- mu M_i + (1 - mu) G_i (float32 (m, n) device tensors)."""
    lib = library()
    count = len(Gs)
    if count == 0:
        return Ms
    probs = (MomentumProblem * count)()
    for i, (G, M) in enumerate(zip(Gs, Ms)):
        if tuple(G.shape) != tuple(M.shape):
            raise ValueError("G and M shapes differ")
        probs[i] = MomentumProblem(G.shape[0], G.shape[1], _ptr(G), _ld(G), _ptr(M), _ld(M))
    _check(lib.momentum_ema_batched(ctypes.addressof(probs), count, float(mu), _stream(stream)))
    return Ms


def hyperball_update_batched(Ws: Sequence, Us: Sequence, lr: float, return_norms: bool = False, stream=None):
    """In place, the MuonH norm-preserving step: W_i <- (W_i - c U_i) ||W_i|| /
    ||W_i - c U_i||, c = lr ||W_i|| / ||U_i||.  With return_norms, also a
    (count, 3) float64 device tensor of ||W||, ||U||, ||W - c U||."""
    import torch

    lib = library()
    count = len(Ws)
    if count == 0:
        return None
    dev = Ws[0].device
    probs = (HyperballProblem * count)()
    for i, (W, U) in enumerate(zip(Ws, Us)):
        if tuple(W.shape) != tuple(U.shape):
            raise ValueError("W and U shapes differ")
        probs[i] = HyperballProblem(W.shape[0], W.shape[1], _ptr(W), _ld(W), _ptr(U), _ld(U))
    need = lib.hyperball_update_batched_workspace(ctypes.addressof(probs), count)
    ws = _workspace(need, dev)
    norms = torch.empty(count, 3, dtype=torch.float64, device=dev) if return_norms else None
    _in_use_on(stream, ws, norms)
    _check(lib.hyperball_update_batched(ctypes.addressof(probs), count, float(lr), _ptr(norms), _ptr(ws), need,
                                        _stream(stream)))
    return norms


def cans_ceilings():
    """(y, z, p) suprema of the CANS scalar recurrence at steps 0..10."""
    arrs = [(ctypes.c_double * 11)() for _ in range(3)]
    n = library().mr_cans_ceilings(*[ctypes.addressof(a) for a in arrs], 11)
    return tuple([a[i] for i in range(n)] for a in arrs)


def decode_info(info, count: int):
    """Device or host uint8 buffer of mr_root_info records -> numpy records."""
    host = info[: ROOT_INFO_BYTES * count].cpu().numpy()
    return host.view(ROOT_INFO_DTYPE).copy()


def precondition_apply(XLs: Sequence, Gs: Sequence, XRs: Sequence, alpha: float = 1.0,
                       Us: Optional[Sequence] = None, stream=None):
    """U_i = alpha XL_i G_i XR_i (float32 device tensors).  Returns the Us."""
    import torch

    lib = library()
    count = len(Gs)
    if count == 0:
        return []
    dev = Gs[0].device
    own_u = Us is None
    if own_u:
        Us = [torch.empty_like(G) for G in Gs]
    probs = (ApplyProblem * count)()
    for i in range(count):
        XL, G, XR, U = XLs[i], Gs[i], XRs[i], Us[i]
        probs[i] = ApplyProblem(G.shape[0], G.shape[1], _ptr(XL), _ld(XL), _ptr(G), _ld(G), _ptr(XR), _ld(XR),
                                _ptr(U), _ld(U))
    need = lib.precondition_apply_workspace(ctypes.addressof(probs), count)
    ws = _workspace(need, dev)
    _in_use_on(stream, ws, *(Us if own_u else ()))
    _check(lib.precondition_apply(ctypes.addressof(probs), count, float(alpha), _ptr(ws), need, _stream(stream)))
    return Us


def newton_schedule(m0: float, final_degree: bool = False):
    """(scales, fp64_steps) of the library's Newton schedule for floor m0, and
    the degree of the last X update when final_degree is set."""
    buf = (ctypes.c_double * 128)()
    j = ctypes.c_int32(0)
    deg = ctypes.c_int32(0)
    K = library().mr_newton_schedule(float(m0), ctypes.addressof(buf), 128, ctypes.addressof(j), ctypes.addressof(deg))
    if K < 0:
        raise ValueError("bad m0")
    out = ([buf[i] for i in range(K)], int(j.value))
    return out + (int(deg.value),) if final_degree else out


class PeakInfo(ctypes.Structure):
    _fields_ = [("cu_count", ctypes.c_int32), ("clock_khz", ctypes.c_int32),
                ("prop_tflops", ctypes.c_double * 4), ("measured_tflops", ctypes.c_double * 4),
                ("measured_random_tflops", ctypes.c_double * 4)]


PEAK_KINDS = ("f32", "f64", "f16", "i8")


def measure_peaks(stream=None) -> dict:
    """Matrix-core peaks of the current device: from CU count x clock, and
    measured by register-only MFMA loops (synchronises the stream)."""
    out = PeakInfo()
    _check(library().mr_measure_peaks(ctypes.addressof(out), _stream(stream)))
    return {"cu_count": int(out.cu_count), "clock_mhz": out.clock_khz / 1e3,
            "device_prop_tflops": {k: round(out.prop_tflops[i], 1) for i, k in enumerate(PEAK_KINDS)},
            "measured_tflops": {k: round(out.measured_tflops[i], 1) for i, k in enumerate(PEAK_KINDS)},
            "measured_random_tflops": {k: round(out.measured_random_tflops[i], 1) for i, k in enumerate(PEAK_KINDS)}}


def newton_iterations(p: int, m0: float, tol: float) -> int:
    return int(library().mr_newton_iterations(p, m0, tol))


def set_jacobi_max_sweeps(sweeps: int) -> int:
    """Cap the Jacobi route's sweeps (process-wide); returns the previous cap."""
    prev = int(library().mr_set_jacobi_max_sweeps(int(sweeps)))
    if prev < 0:
        raise ValueError(f"sweep cap {sweeps} outside [1, 100]")
    return prev


def trace_enable(on: bool = True) -> bool:
    """Bracket every library launch with HIP events on its stream."""
    return bool(library().mr_trace_enable(1 if on else 0))


def trace_collect() -> dict:
    """{kernel class: (launches, total_ms)} since the last collect (waits for them)."""
    recs = (TraceRecord * 32)()
    k = library().mr_trace_collect(ctypes.addressof(recs), 32)
    return {recs[i].name.decode(): (int(recs[i].launches), float(recs[i].total_ms)) for i in range(k)}
