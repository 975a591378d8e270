"""Seeded synthetic inputs for the five layer-shaped workloads.

This module only draws random inputs; it holds none of the preconditioner's
arithmetic, and both the HIP path's tests and the fp64 oracle take their
inputs from here.  Every input is float32, row-major, and is a pure function
of (workload id, layer, weight, step): each draw gets its own
``numpy.random.Generator(PCG64(SeedSequence(0, spawn_key=key)))``, so any
single gradient can be regenerated without drawing the others.

Workloads (shapes are rows × cols = m × n of the weight gradient G):

1. toy      2 weights 64×128, G i.i.d. N(0,1), 10 steps.
2. w1024    8 layers × {q,k,v,o 1024×1024; up 1024×4096; down 4096×1024};
            G = A·Bᵀ + 0.1·N with A (m×32), B (n×32), N all i.i.d. N(0,1); 5 steps.
3. w2048    24 layers × {q,k,v,o 2048×2048; up 2048×8192; down 8192×2048};
            G = U·diag(σ)·Vᵀ, σ_i = i^-0.7, U and V Haar (QR of a Gaussian with
            the signs of diag(R) fixed); 3 steps.
4. illcond  256 symmetric positive definite 512×512 matrices Q·diag(λ)·Qᵀ,
            Q Haar, λ = 10^u with u ~ U(-8, 0), built in float64 and rounded to
            float32 once; one root call per eps in {1e-8, 1e-6, 1e-4}.
5. moe      64 weights 3072×1536 then 64 weights 1536×3072; G i.i.d. N(0,1)
            with floor(0.3·m) rows set to zero, the rows re-drawn per
            (weight, step); 4 steps.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

WORKLOAD_IDS = {"toy": 1, "w1024": 2, "w2048": 3, "illcond": 4, "moe": 5}


@dataclass(frozen=True)
class Workload:
    name: str
    shapes: tuple  # ((label, m, n), ...)
    kind: str  # gradient distribution
    steps: int
    beta: float = 0.95
    eps: float = 1e-6
    normalize: str = "trace"
    eps_list: tuple = field(default=())


def _transformer_shapes(layers: int, width: int):
    out = []
    for layer in range(layers):
        for name in ("q", "k", "v", "o"):
            out.append((f"L{layer}.{name}", width, width))
        out.append((f"L{layer}.up", width, 4 * width))
        out.append((f"L{layer}.down", 4 * width, width))
    return tuple(out)


WORKLOADS = {
    "toy": Workload("toy", (("W0", 64, 128), ("W1", 64, 128)), "gaussian", 10),
    "w1024": Workload("w1024", _transformer_shapes(8, 1024), "lowrank32", 5),
    "w2048": Workload("w2048", _transformer_shapes(24, 2048), "powerlaw", 3),
    "moe": Workload("moe", tuple([(f"E{e}.in", 3072, 1536) for e in range(64)]
                                 + [(f"E{e}.out", 1536, 3072) for e in range(64)]),
                    "sparserows", 4),
    "illcond": Workload("illcond", (), "spd_loguniform", 1, normalize="none",
                        eps_list=(1e-8, 1e-6, 1e-4)),
}


def rng_for(workload_id: int, *key: int) -> np.random.Generator:
    """One independent generator per (workload, key...) tuple."""
    ss = np.random.SeedSequence(0, spawn_key=(int(workload_id),) + tuple(int(k) for k in key))
    return np.random.Generator(np.random.PCG64(ss))


def haar_columns(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """rows×cols matrix with orthonormal columns, Haar-distributed (float64).

    QR of a Gaussian matrix with the signs of diag(R) moved into Q (Mezzadri,
    "How to generate random matrices from the classical compact groups").
    """
    Z = rng.standard_normal((rows, cols))
    Q, Rm = np.linalg.qr(Z)
    sgn = np.sign(np.diag(Rm))
    sgn[sgn == 0] = 1.0
    return Q * sgn


def draw_gradient(kind: str, m: int, n: int, rng: np.random.Generator) -> np.ndarray:
    """One m×n float32 gradient of the given distribution."""
    if kind == "gaussian":
        return rng.standard_normal((m, n), dtype=np.float32)
    if kind == "lowrank32":
        r = 32
        A = rng.standard_normal((m, r), dtype=np.float32)
        B = rng.standard_normal((n, r), dtype=np.float32)
        N = rng.standard_normal((m, n), dtype=np.float32)
        return (A @ B.T + np.float32(0.1) * N).astype(np.float32)
    if kind == "powerlaw":
        r = min(m, n)
        U = haar_columns(rng, m, r)
        V = haar_columns(rng, n, r)
        sigma = np.arange(1, r + 1, dtype=np.float64) ** -0.7
        return ((U * sigma) @ V.T).astype(np.float32)
    if kind == "sparserows":
        G = rng.standard_normal((m, n), dtype=np.float32)
        zero = rng.choice(m, size=int(np.floor(0.3 * m)), replace=False)
        G[zero, :] = 0.0
        return G
    raise ValueError(f"unknown gradient kind {kind!r}")


def gradient(workload: str, weight: int, step: int, shape=None) -> np.ndarray:
    """Gradient of weight `weight` at step `step` (1-based) of a workload.

    `shape` = (m, n) overrides the workload's shape (same distribution, same
    seeding), which the tests use for smaller instances.
    """
    w = WORKLOADS[workload]
    if shape is None:
        _, m, n = w.shapes[weight]
    else:
        m, n = shape
    rng = rng_for(WORKLOAD_IDS[workload], 0, weight, step)
    return draw_gradient(w.kind, m, n, rng)


def spd_loguniform(d: int, rng: np.random.Generator, lo_exp: float = -8.0,
                   hi_exp: float = 0.0) -> np.ndarray:
    """Q·diag(10^u)·Qᵀ, u ~ U(lo_exp, hi_exp), Q Haar; built in float64,
    rounded to float32 once (exactly symmetric after rounding)."""
    Q = haar_columns(rng, d, d)
    lam = 10.0 ** rng.uniform(lo_exp, hi_exp, size=d)
    A = (Q * lam) @ Q.T
    A = 0.5 * (A + A.T)
    return A.astype(np.float32)


def illcond_batch(count: int = 256, d: int = 512) -> np.ndarray:
    """The ill-conditioned batch: (count, d, d) float32."""
    out = np.empty((count, d, d), dtype=np.float32)
    for i in range(count):
        out[i] = spd_loguniform(d, rng_for(WORKLOAD_IDS["illcond"], 0, i, 0))
    return out


def _device_seed(workload_id: int, *key: int) -> int:
    ss = np.random.SeedSequence(0, spawn_key=(int(workload_id), 1) + tuple(int(k) for k in key))
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64(2 ** 63 - 1))


def gradient_device(workload: str, weight: int, step: int, device, shape=None):
    """A gradient with the same distribution, shape and structure as
    `gradient`, drawn on a torch device with torch's own generator.

    The values differ from the host draws (another random stream, seeded
    from the same (workload, weight, step) key); throughput runs use these
    where host generation would take minutes (the width-2048 set's Haar
    factors), parity tests never do.
    """
    import torch

    w = WORKLOADS[workload]
    if shape is None:
        _, m, n = w.shapes[weight]
    else:
        m, n = shape
    g = torch.Generator(device=device)
    g.manual_seed(_device_seed(WORKLOAD_IDS[workload], weight, step))

    def normal(*size, dtype=torch.float32):
        return torch.randn(*size, generator=g, device=device, dtype=dtype)

    if w.kind == "gaussian":
        return normal(m, n)
    if w.kind == "lowrank32":
        A, B, N = normal(m, 32), normal(n, 32), normal(m, n)
        return A @ B.T.contiguous() + 0.1 * N
    if w.kind == "powerlaw":
        r = min(m, n)

        def haar(rows):
            Q, Rm = torch.linalg.qr(normal(rows, r, dtype=torch.float64))
            sgn = torch.sign(torch.diagonal(Rm))
            sgn[sgn == 0] = 1.0
            return Q * sgn

        U, V = haar(m), haar(n)
        sigma = torch.arange(1, r + 1, device=device, dtype=torch.float64) ** -0.7
        return ((U * sigma) @ V.T.contiguous()).to(torch.float32)
    if w.kind == "sparserows":
        G = normal(m, n)
        zero = torch.randperm(m, generator=g, device=device)[: int(np.floor(0.3 * m))]
        G[zero, :] = 0.0
        return G
    raise ValueError(f"unknown gradient kind {w.kind!r}")
