"""Throughput of the EMA-Gram quarter-power preconditioner step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload w1024]

One step = one pass of the whole hot path over one batch of synthetic
gradients already resident in HBM: gram_ema_update for every weight (both
Grams, float64 state), inv_quarter_root_batched over all 2 x weights Grams
(trace rescale, eps = 1e-6), precondition_apply for every weight.  The
default workload is the width-1024 transformer weight set (8 layers x
{q,k,v,o 1024x1024, up 1024x4096, down 4096x1024}, rank-32 + noise
gradients); the Gram state evolves across steps and the gradients cycle
through the workload's 5 seeded steps.  --workload toy runs the 2 x
64x128 set the same way; --workload illcond times one root call per eps on
the 256 ill-conditioned 512 x 512 matrices (roots/s).

Printed: one JSON line with the throughput, every kernel class's time, work
and fraction of the roofline of the unit it runs on (fp64 or fp16 matrix
cores, or HBM), the dominant kernel's roofline, per-size-class root figures,
a state-reset repetition protocol (median and every per-step time), and the
fp64 CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f32": 157.3, "f64": 78.6, "f16": 2500.0, "i8": 5000.0}  # MI355X dense MFMA (vendor figures; i8 in TOP/s)
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E (vendor figure)
# kernel class -> matrix-core unit it runs on
CLASS_ENGINE = {"newton_f64": "f64", "syrk_ema": "f64", "newton_f32": "f32", "newton_x3": "f16", "apply_x3": "f16",
                "newton_i8": "i8", "root_moment": "f16"}
MOMENT_MIN_D = 256  # Newton roots from this size take the moment bounds


def moment_flops(d: int) -> float:
    """The moment bounds' two plain fp16 products of a Newton root (H H and
    P16 P16, symmetric: d^2 (d + 1) algorithmic flops each); 0 below the
    size that takes them."""
    return 2.0 * d * d * (d + 1) if d >= MOMENT_MIN_D else 0.0
# matrix-core products per algorithmic product: three fp16 products per
# float32-accurate one (split classes), 21 int8 digit-plane products per
# float64-accurate one (the default path's float64 steps)
MFMA_PER_PRODUCT = {"newton_x3": 3, "apply_x3": 3, "newton_i8": 21}
SPLIT_CLASSES = tuple(MFMA_PER_PRODUCT)
DTYPE = "f64(int8 digit-plane products)+f32(split-f16 products)"
METRIC = "preconditioned matrix updates/sec + TFLOP/s as % fp32 MFMA peak, d=1024–4096"
ILLCOND_METRIC = "inverse quarter roots/s (256 ill-conditioned 512x512, one call per eps, no rescale)"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def host_cores():
    """(cores this process may run on, BLAS/LAPACK threads numpy uses)."""
    cores = len(os.sched_getaffinity(0))
    try:
        import threadpoolctl

        blas = max(int(i.get("num_threads", 1)) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:  # pragma: no cover
        blas = cores
    return cores, blas


def blas_vendor() -> str:
    """The BLAS/LAPACK library numpy's oracle runs on (name and version)."""
    try:
        import threadpoolctl

        libs = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            return f"{libs[0].get('internal_api', '?')} {libs[0].get('version', '?')}"
    except Exception:  # pragma: no cover
        pass
    return "unknown"


I8_MIN_D = 1024  # the library's kI8MinD: Grams from this size take the int8 digit-plane products


def f64_class(d: int) -> str:
    """Kernel class of the float64 steps' products of a d x d Gram on the
    default path: int8 digit planes from I8_MIN_D, the float64 kernel below."""
    return "newton_i8" if d >= I8_MIN_D else "newton_f64"


def sym_gemm_flops(d: int) -> float:
    """One symmetric-output product of d x d matrices: d(d+1)/2 outputs x d MACs x 2."""
    return float(d) * d * (d + 1)


def newton_flops(d: int, K: int, j: int, x_low: bool = True, final_degree: int = 1):
    """Algorithmic (upper-triangle) flops of one Newton root, split by the
    kernel class that runs them: iterations t < K-1 take 4 symmetric products
    (M^2, T2^2, T4 M, X M), the last one only X q(M): one product for the
    step's own degree-1 polynomial, two for the degree-2 Taylor finish (q(M)
    from M^2, then X q) and three for the degree-4 one (M^2, E^2 R, X q);
    t < j run M's products float64-accurate (on int8 digit planes with x_low,
    in float64 otherwise), and the X product too unless x_low
    (then it runs on the split-fp16 kernel, like every product of the float32
    steps).  With x_low the first X product (X0 = I) is no product: the init
    writes X1."""
    f64 = low = 0.0
    g = sym_gemm_flops(d)
    for t in range(K):
        m_products = 3 * g if t < K - 1 else {1: 0.0, 2: g, 4: 2 * g}[max(final_degree, 1)]
        x_product = 0.0 if (x_low and t == 0) else g
        if t < j:
            f64 += m_products
            if x_low:
                low += x_product
            else:
                f64 += x_product
        else:
            low += m_products + x_product
    return f64, low


def root_stream_bytes(d: int, state_bytes: int, packed: bool, K: int, j: int):
    """Algorithmic HBM bytes of the streaming kernels of one Newton root
    (default path: float32 X in split storage), by kernel class:
      root_stats    reads A once (the stored elements);
      root_init     reads A once, writes M0 (float64) and the split copies of
                    M0 and X1 (4 bytes each) per element;
      newton_convert  at the float64 -> split switch: reads M (8), writes its
                    split copy (4) per element;
      newton_slice  each float64 step with products (t < min(j, K - 1)) of a
                    Gram of I8_MIN_D or more: reads M (8 per element), writes
                    its six digit planes (6 per element of the matrix padded
                    to dp, a multiple of 128) and dp row exponents (4 each);
      root_finalize reads X (split, 4) and M_{K-1} (8 in float64, 4 split),
                    writes X (float32, 4) per element."""
    n = d * d
    dp = (d + 127) // 128 * 128
    stored = d * (d + 1) // 2 if packed else n
    m_last = 8 if (K - 1) < j else 4
    return {"root_stats": state_bytes * stored,
            "root_init": state_bytes * stored + 16 * n,
            "newton_convert": 12 * n if j < K else 0,
            "newton_slice": (8 * n + 6 * dp * dp + 4 * dp) * max(min(j, K - 1), 0) if d >= I8_MIN_D else 0,
            "root_finalize": (4 + m_last + 4) * n}


# ------------------------------------------------------------------ oracle
def cpu_baseline(workload: str, max_seconds: float = 30.0):
    """The fp64 oracle (as it stands), stateful: for each weight shape class
    of the workload, one weight of that class runs its own sequence of steps
    (Gram EMA, two eigendecomposition roots, apply) from zero state, as many
    steps as fit its share of `max_seconds` (at least one).  seconds per
    optimizer step = sum over the workload's weights of their class's mean
    seconds per step; value = weights / that."""
    import oracle
    from matrix_roots_amd import workloads as W

    cores, blas = host_cores()
    wl = W.WORKLOADS[workload]
    classes = {}
    for i, (name, m, n) in enumerate(wl.shapes):
        classes.setdefault((m, n), []).append(i)
    budget = max_seconds / len(classes)
    per_class = {}
    total = 0.0
    for (m, n), idx in classes.items():
        w = idx[0]
        L, R = np.zeros((m, m)), np.zeros((n, n))
        secs, steps, t = 0.0, 0, 0
        while True:
            t += 1
            G = W.gradient(workload, w, (t - 1) % wl.steps + 1)
            t0 = time.perf_counter()
            L, R, *_ = oracle.preconditioner_step(L, R, G, wl.beta, wl.eps, wl.normalize)
            secs += time.perf_counter() - t0
            steps += 1
            if secs + secs / steps > budget or steps >= 100 * wl.steps:
                break
        per_class[f"{m}x{n}"] = {"weights": len(idx), "steps_timed": steps, "seconds_per_step": secs / steps}
        total += secs
    step_seconds = sum(v["weights"] * v["seconds_per_step"] for v in per_class.values())
    shown = "; ".join(f"{k}: {v['steps_timed']} steps of {wl.shapes[classes[tuple(map(int, k.split('x')))][0]][0]}, "
                      f"{v['seconds_per_step']:.3f}s each" for k, v in per_class.items())
    sample = (f"one weight per shape class runs its own steps from zero state ({shown}); "
              f"per-step seconds weighted by the workload's {len(wl.shapes)} weights; fp64 numpy/LAPACK")
    return {"value": len(wl.shapes) / step_seconds, "unit": "matrix updates/s", "cores": blas,
            "host_cores": cores, "kind": "oracle", "blas": blas_vendor(), "sample": sample, "seconds": round(total, 2),
            "seconds_per_optimizer_step": round(step_seconds, 3)}


def cpu_baseline_illcond(mats, eps_list, max_seconds: float = 20.0):
    """The fp64 oracle's root (eigh) on the ill-conditioned matrices, in order
    and cycling through the eps values, until `max_seconds`."""
    import oracle

    cores, blas = host_cores()
    secs, roots = 0.0, 0
    while secs < max_seconds and roots < len(mats) * len(eps_list):
        A = mats[roots % len(mats)].astype(np.float64)
        eps = eps_list[(roots // len(mats)) % len(eps_list)]
        t0 = time.perf_counter()
        oracle.inv_quarter_root(A, eps, "none")
        secs += time.perf_counter() - t0
        roots += 1
    return {"value": roots / secs, "unit": "roots/s", "cores": blas, "host_cores": cores, "kind": "oracle", "blas": blas_vendor(),
            "sample": f"the first {roots} 512x512 roots of the batch (eigh, fp64 numpy/LAPACK, eps 1e-8 first)",
            "seconds": round(secs, 2)}


# ----------------------------------------------------------- roofline helpers
def recorded_traffic(kernel: str, workload: str, family: str = "quarter"):
    """HBM bytes per working launch of `kernel` (FETCH_SIZE + WRITE_SIZE,
    calibrated) from the committed counter summary, if the kernel sources are
    unchanged since the counters were taken; None for a summary covering
    several kernels."""
    from matrix_roots_amd import profile_summary

    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    rec = {}
    keys = ("traffic_bytes_per_working_launch", "traffic_bytes_per_launch", "source_sha256")
    for line in open(path):
        if ":" in line and line.split(":", 1)[0].strip() in keys:
            k, v = line.split(":", 1)
            if k.strip() in rec and k.strip() != "source_sha256":
                return None
            rec[k.strip()] = v.strip().strip("`")
    if rec.get("source_sha256") != profile_summary.sources_sha256(family):
        return None
    try:
        return float(rec.get("traffic_bytes_per_working_launch", rec["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def kernel_table(trace, flops, bytes_, launches_working=None):
    """Per kernel class: launches, time, and its rate against the roofline of
    the unit it runs on: matrix-core classes in algorithmic TFLOP/s (split
    classes also in the matrix-core work they issue: three fp16 products per
    float32-accurate product, 21 int8 products per float64-accurate one)
    against their own unit's peak; streaming classes in algorithmic GB/s
    against HBM."""
    out = {}
    for name, (launches, ms) in sorted(trace.items()):
        ent = {"launches": launches, "ms_total": round(ms, 3), "ms_avg": round(ms / launches, 4)}
        if launches_working and name in launches_working:
            ent["launches_working"] = launches_working[name]
        f = flops.get(name)
        if f:
            eng = CLASS_ENGINE[name]
            tf = f / (ms / 1e3) / 1e12
            ent.update({"engine": eng, "tflops": round(tf, 2)})
            if name in SPLIT_CLASSES:
                x = MFMA_PER_PRODUCT[name]
                ent.update({"mfma_tflops": round(x * tf, 2), "peak": PEAK_TFLOPS[eng],
                            "frac": round(x * tf / PEAK_TFLOPS[eng], 4),
                            "frac_algorithmic": round(tf / PEAK_TFLOPS[eng], 4)})
                if eng == "i8":
                    ent["note"] = ("tflops: float64-accurate algorithmic TFLOP/s; mfma_tflops: int8 TOP/s "
                                   "(21 digit-plane products each)")
            else:
                ent.update({"peak": PEAK_TFLOPS[eng], "frac": round(tf / PEAK_TFLOPS[eng], 4)})
        b = bytes_.get(name)
        if b:
            gbs = b / (ms / 1e3) / 1e9
            ent.update({"gb_per_s": round(gbs, 1), "hbm_peak_gb_per_s": HBM_PEAK_GBS,
                        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)})
        out[name] = ent
    return out


def engine_table(kernels):
    """Time and work per matrix-core unit over its kernel classes."""
    out = {}
    for eng in ("f64", "i8", "f16", "f32"):
        names = [n for n, k in kernels.items() if k.get("engine") == eng]
        if not names:
            continue
        ms = sum(kernels[n]["ms_total"] for n in names)
        work = sum((kernels[n]["mfma_tflops"] if n in SPLIT_CLASSES else kernels[n]["tflops"])
                   * kernels[n]["ms_total"] for n in names) / ms
        out[eng] = {"classes": names, "ms_total": round(ms, 3), "mfma_tflops": round(work, 2),
                    "peak": PEAK_TFLOPS[eng], "frac": round(work / PEAK_TFLOPS[eng], 4)}
    return out


def annotate_engines(engines, peaks):
    """Each unit's rate beside what the vendor GEMM sustains on it in the same
    run and what its register-only MFMA loop reaches on random operands (the
    clock real data leave the chip); the roofline fractions stay against
    the published peaks."""
    vend = peaks.get("vendor_gemm_tflops") or {}
    rnd = peaks.get("measured_random_tflops") or {}
    for eng, e in engines.items():
        if eng in vend:
            e["vendor_gemm_tflops"] = vend[eng]
            e["frac_of_vendor_gemm"] = round(e["mfma_tflops"] / vend[eng], 4)
        if rnd.get(eng):
            e["random_operand_loop_tflops"] = rnd[eng]
            e["frac_of_random_operand_loop"] = round(e["mfma_tflops"] / rnd[eng], 4)


# classes whose counters come from the optimizer-step run (their own source family)
STEP_CLASSES = ("momentum", "hyperball_reduce", "hyperball_update")


def roofline_for(kernels, name, workload):
    k = kernels[name]
    traffic = (recorded_traffic(name, f"{workload}_step", "step") if name in STEP_CLASSES
               else recorded_traffic(name, workload))
    if "tflops" in k:
        split = name in SPLIT_CLASSES
        r = {"bound": "mfma", "kernel": name, "engine": k["engine"],
             "achieved": k["mfma_tflops"] if split else k["tflops"], "peak": k["peak"],
             "unit": "TOP/s" if k["engine"] == "i8" else "TFLOP/s",
             "frac": k["frac"], "traffic": traffic,
             "traffic_per": "working launch (calibrated FETCH_SIZE + WRITE_SIZE, profiles/)",
             "achieved_per_launch": "algorithmic flops of the class over the timed steps (x3 fp16 products "
                                    "for split-fp16 classes, x21 int8 products for newton_i8) / sum of its "
                                    "event-measured launch durations"}
    else:
        r = {"bound": "hbm", "kernel": name, "achieved": k["gb_per_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": k["hbm_frac"], "traffic": traffic,
             "traffic_per": "working launch (calibrated FETCH_SIZE + WRITE_SIZE, profiles/)",
             "achieved_per_launch": "algorithmic bytes of the class over the timed steps / sum of its "
                                    "event-measured launch durations"}
    if "launches_working" in k:
        r["launches"] = k["launches"]
        r["launches_working"] = k["launches_working"]
    return r


# ---------------------------------------------------------- per size class
def per_size_class(B, torch, grams, wl, min_d=129):
    """One inv_quarter_root_batched call per Gram size d >= min_d on the given
    (final) state, after one untimed call, with the library's per-launch
    events: time, fp32-accurate algorithmic TFLOP/s (against the fp32 MFMA
    peak, as the metric states it), and the float64 and split-fp16 classes
    against the peaks of the units they run on."""
    out = {}
    dims = [B.packed_dim(A.numel()) if A.dim() == 1 else int(A.shape[0]) for A in grams]
    for d in sorted(set(dims)):
        if d < min_d:
            continue
        As = [A for A, dd in zip(grams, dims) if dd == d]
        Xs = [torch.empty(d, d, dtype=torch.float32, device=A.device) for A in As]
        ws = B.RootWorkspace()
        B.inv_quarter_root_batched(As, wl.eps, normalize=wl.normalize, Xs=Xs, workspace=ws, return_info=False)
        raw = torch.empty(B.ROOT_INFO_BYTES * len(As), dtype=torch.uint8, device=As[0].device)
        torch.cuda.synchronize()
        B.trace_collect()
        B.trace_enable(True)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        B.inv_quarter_root_batched(As, wl.eps, normalize=wl.normalize, Xs=Xs, workspace=ws, return_info=False,
                                   info_out=raw)
        e1.record()
        torch.cuda.synchronize()
        B.trace_enable(False)
        tr = B.trace_collect()
        info = B.decode_info(raw, len(As))
        ms = e0.elapsed_time(e1)
        f64 = low = 0.0
        for r in info:
            a, b = newton_flops(d, int(r["iters"]), int(r["fp64_iters"]), final_degree=int(r["final_degree"]))
            f64 += a
            low += b
        # (one size per call: its float64 products ran on one kernel class, f64_class(d))
        tf = (f64 + low) / (ms / 1e3) / 1e12
        ent = {"count": len(As), "ms": round(ms, 3), "tflops": round(tf, 2),
               "fp32_equivalent_pct_of_fp32_peak": round(100 * tf / PEAK_TFLOPS["f32"], 2),
               "iters": [int(info["iters"].min()), int(info["iters"].max())],
               "fp64_iters": [int(info["fp64_iters"].min()), int(info["fp64_iters"].max())]}
        if "newton_f64" in tr and f64 > 0:
            t64 = f64 / (tr["newton_f64"][1] / 1e3) / 1e12
            ent["newton_f64"] = {"ms": round(tr["newton_f64"][1], 3), "tflops": round(t64, 2),
                                 "frac_of_f64_peak": round(t64 / PEAK_TFLOPS["f64"], 4)}
        if "newton_i8" in tr and f64 > 0:
            t8 = f64 / (tr["newton_i8"][1] / 1e3) / 1e12
            ent["newton_i8"] = {"ms": round(tr["newton_i8"][1], 3), "f64_equivalent_tflops": round(t8, 2),
                                "int8_tops": round(21 * t8, 1),
                                "frac_of_i8_peak": round(21 * t8 / PEAK_TFLOPS["i8"], 4)}
        if "newton_x3" in tr and low > 0:
            tx = low / (tr["newton_x3"][1] / 1e3) / 1e12
            ent["newton_x3"] = {"ms": round(tr["newton_x3"][1], 3), "tflops": round(tx, 2),
                                "mfma_tflops": round(3 * tx, 2),
                                "frac_of_f16_peak": round(3 * tx / PEAK_TFLOPS["f16"], 4)}
        out[str(d)] = ent
        log(f"size class {d}: {ent}")
        del Xs, ws
    return out


# ------------------------------------------------------------ the main step
def bench_steps(args, torch, B, W, peaks):
    dev = torch.device("cuda:0")
    wl = W.WORKLOADS[args.workload]
    shapes = [(m, n) for _, m, n in wl.shapes]
    nw = len(shapes)
    gen = args.gradients if args.gradients != "auto" else ("device" if args.workload == "w2048" else "host")
    log(f"workload {args.workload}: {nw} weights, generating {wl.steps} steps of gradients on the {gen}")
    t0 = time.perf_counter()
    grads = []
    for t in range(1, wl.steps + 1):
        if gen == "host":
            grads.append([torch.from_numpy(W.gradient(args.workload, w, t)).to(dev) for w in range(nw)])
        else:
            grads.append([W.gradient_device(args.workload, w, t, dev) for w in range(nw)])
        torch.cuda.synchronize()
        log(f"  step {t} gradients resident ({time.perf_counter() - t0:.1f}s)")
    sdt = torch.float64 if args.state_dtype == "f64" else torch.float32
    if args.packed_state:
        Ls = [torch.zeros(m * (m + 1) // 2, dtype=sdt, device=dev) for m, n in shapes]
        Rs = [torch.zeros(n * (n + 1) // 2, dtype=sdt, device=dev) for m, n in shapes]
    else:
        Ls = [torch.zeros(m, m, dtype=sdt, device=dev) for m, n in shapes]
        Rs = [torch.zeros(n, n, dtype=sdt, device=dev) for m, n in shapes]
    state_bytes = sum(x.numel() * x.element_size() for x in Ls + Rs)
    log(f"Gram state: {state_bytes / 1e9:.2f} GB ({'packed' if args.packed_state else 'full'})")
    Xs = [torch.empty(m, m, dtype=torch.float32, device=dev) for m, n in shapes] + \
         [torch.empty(n, n, dtype=torch.float32, device=dev) for m, n in shapes]
    Us = [torch.empty(m, n, dtype=torch.float32, device=dev) for m, n in shapes]
    ws = B.RootWorkspace()
    total = args.warmup + args.steps
    infos = [torch.empty(B.ROOT_INFO_BYTES * 2 * nw, dtype=torch.uint8, device=dev) for _ in range(total)]

    if args.optimizer_step:
        Ms = [torch.zeros(m, n, dtype=torch.float32, device=dev) for m, n in shapes]
        Wts = [torch.randn(m, n, dtype=torch.float32, device=dev) / (m ** 0.5) for m, n in shapes]

    def step(i, info_buf):
        G = grads[i % wl.steps]
        if args.optimizer_step:
            B.momentum_ema_batched(G, Ms, 0.9)
        B.gram_ema_update(G, Ls, Rs, wl.beta)
        B.inv_quarter_root_batched(Ls + Rs, wl.eps, normalize=wl.normalize, method=args.method, Xs=Xs,
                                   workspace=ws, return_info=False, info_out=info_buf)
        B.precondition_apply(Xs[:nw], Ms if args.optimizer_step else G, Xs[nw:], Us=Us)
        if args.optimizer_step:
            B.hyperball_update_batched(Wts, Us, 0.02)

    for i in range(args.warmup):
        step(i, infos[i])
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")

    graphs = None
    if args.graph:
        # one HIP graph per gradient of the cycle (each bakes in its buffers);
        # the entry points only enqueue kernels, so they capture as they run
        graphs = []
        for k in range(wl.steps):
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                step(k, infos[args.warmup + k] if args.warmup + k < total else infos[-1])
            graphs.append(gr)
        torch.cuda.synchronize()
        log(f"captured {len(graphs)} step graphs")

    # the timed region: exactly --steps steps, no per-launch events
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, total):
        if graphs is not None:
            graphs[i % wl.steps].replay()
        else:
            step(i, infos[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    log(f"timed {args.steps} steps in {t1 - t0:.3f}s{' (graph replays)' if graphs is not None else ''}")
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = nw / (ms_per_step / 1e3)

    # the same number of steps again, each launch bracketed by events on its
    # stream: per-class durations for the rooflines (the state keeps evolving)
    B.trace_collect()
    B.trace_enable(True)
    for i in range(args.warmup, total):
        step(i, infos[i])
    torch.cuda.synchronize()
    B.trace_enable(False)
    trace = B.trace_collect()

    # algorithmic work and bytes over the timed steps
    es = 8 if args.state_dtype == "f64" else 4
    f64 = {"newton_i8": 0.0, "newton_f64": 0.0}
    low = 0.0
    sbytes = {"root_stats": 0, "root_init": 0, "newton_convert": 0, "newton_slice": 0, "root_finalize": 0}
    iters = []
    n_newton = 0
    for i in range(args.warmup, total):
        info = B.decode_info(infos[i], 2 * nw)
        assert (info["flags"] == 0).all(), info[info["flags"] != 0]
        for k, rec in enumerate(info):
            d = shapes[k % nw][0] if k < nw else shapes[k % nw][1]
            if int(rec["final_degree"]) == 0:  # eigendecomposition route: no matrix-core work to count
                continue
            n_newton += 1
            K, j = int(rec["iters"]), int(rec["fp64_iters"])
            a, b = newton_flops(d, K, j, final_degree=int(rec["final_degree"]))
            f64[f64_class(d)] += a
            low += b
            for kk, v in root_stream_bytes(d, es, args.packed_state, K, j).items():
                sbytes[kk] += v
            iters.append((K, j))
    syrk = sum(m * (m + 1) * n + n * (n + 1) * m for m, n in shapes) * args.steps
    apply_f = sum(2.0 * m * n * (m + n) for m, n in shapes) * args.steps
    step_flops = (sum(f64.values()) + low + syrk + apply_f) / args.steps

    elems = sum(m * n for m, n in shapes) * args.steps
    sbytes.update({"momentum": 12 * elems, "hyperball_reduce": 8 * elems, "hyperball_update": 12 * elems,
                   # maxima and split copies of XR, G, XL and W^T: 8 bytes read and 4 written per element
                   "apply_split": 12 * sum(m * m + 2 * m * n + n * n for m, n in shapes) * args.steps})
    moment = sum(moment_flops(m) + moment_flops(n) for m, n in shapes) * args.steps
    flops = {**f64, "newton_x3": low, "syrk_ema": syrk, "apply_x3": apply_f, "root_moment": moment}
    kernels = kernel_table(trace, flops, sbytes)
    # the syrk's HBM bytes (state read + write, gradient read) as context: it is matrix-core bound
    if "syrk_ema" in kernels:
        st_el = sum((m * (m + 1) // 2 if args.packed_state else m * m) + (n * (n + 1) // 2 if args.packed_state
                    else n * n) for m, n in shapes)
        kernels["syrk_ema"]["hbm_bytes_per_step"] = 2 * es * st_el + 2 * 4 * sum(m * n for m, n in shapes)
    engines = engine_table(kernels)
    annotate_engines(engines, peaks)
    dname = max((kv for kv in kernels.items() if "tflops" in kv[1]), key=lambda kv: kv[1]["ms_total"])[0]
    roofline = roofline_for(kernels, dname, args.workload)
    rooflines = {n: roofline_for(kernels, n, args.workload) for n in kernels
                 if "tflops" in kernels[n] or "gb_per_s" in kernels[n]}

    # state-reset repetitions: the workload's own steps from zero state, each
    # step bracketed by events (the parity tests' inputs; outside the timed region)
    protocol = None
    if args.reps > 0:
        per_rep = []
        e = [torch.cuda.Event(enable_timing=True) for _ in range(wl.steps + 1)]
        for r in range(args.reps):
            for S in Ls + Rs:
                S.zero_()
            if args.optimizer_step:
                for M in Ms:
                    M.zero_()
            torch.cuda.synchronize()
            e[0].record()
            for t in range(wl.steps):
                step(t, infos[0])
                e[t + 1].record()
            torch.cuda.synchronize()
            per_rep.append([round(e[t].elapsed_time(e[t + 1]), 3) for t in range(wl.steps)])
            log(f"repetition {r + 1}/{args.reps} from zero state: {per_rep[-1]} ms")
        flat = [x for rep in per_rep for x in rep]
        runs = [sum(rep) for rep in per_rep]
        protocol = {"repetitions": args.reps, "steps_per_repetition": wl.steps,
                    "state": "Gram states (and momentum) zeroed before each repetition",
                    "median_ms_per_step": round(statistics.median(flat), 3),
                    "median_ms_per_repetition": round(statistics.median(runs), 3),
                    "median_updates_per_s": round(nw / (statistics.median(flat) / 1e3), 4),
                    "per_step_ms": per_rep}

    size_classes = None
    if args.size_classes:
        # the per-class calls take their own workspaces: free the step's first
        # (the width-2048 set needs most of the 288 GB otherwise)
        del Xs, Us, grads
        ws.buf = ws.info = None
        torch.cuda.empty_cache()
        size_classes = per_size_class(B, torch, Ls + Rs, wl)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on its sample")
        cpu = cpu_baseline(args.workload)
        log(f"oracle: {cpu['value']:.4f} matrix updates/s on {cpu['cores']} BLAS threads ({cpu['seconds']:.1f}s)")

    kmin = min((k for k, _ in iters), default=0)
    kmax = max((k for k, _ in iters), default=0)
    tf_step = step_flops / (ms_per_step / 1e3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 4),
        "unit": "matrix updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "data": "synthetic",
        "config": {"workload": args.workload, "weights": nw, "grams_per_step": 2 * nw,
                   "shapes": sorted({f"{m}x{n}" for m, n in shapes}), "beta": wl.beta, "eps": wl.eps,
                   "normalize": wl.normalize, "state_dtype": args.state_dtype, "gradients": gen,
                   "state_layout": "packed" if args.packed_state else "full", "state_gb": round(state_bytes / 1e9, 3),
                   "optimizer_step": bool(args.optimizer_step), "method": args.method,
                   "timing": "HIP graph replays" if args.graph else "eager launches"},
        "tflops": round(tf_step, 2),
        "pct_fp32_mfma_peak": round(100 * tf_step / PEAK_TFLOPS["f32"], 2),
        "pct_fp32_mfma_peak_note": "the metric's headline: float32-accurate algorithmic TFLOP/s of the whole step "
                                   "over the fp32 MFMA peak; the work runs on the int8, fp16 and fp64 matrix "
                                   "cores, not the fp32 ones, so this is not a fraction of any unit's roofline "
                                   "(those are in engines, kernels and rooflines)",
        "newton_iters": {"min": kmin, "max": kmax},
        "engines": engines,
        "roofline": roofline,
        "rooflines": rooflines,
        "kernels": kernels,
        "protocol": protocol,
        "cpu_baseline": cpu,
        "peaks": peaks,
    }
    if size_classes is not None:
        out["size_classes"] = size_classes
    print(json.dumps(out), flush=True)
    return 0


def bench_illcond(args, torch, B, W, peaks):
    """One step = one inv_quarter_root_batched call per eps in {1e-8, 1e-6,
    1e-4} over the 256 ill-conditioned 512 x 512 matrices (no rescale, as
    the workload states), inputs resident in HBM."""
    dev = torch.device("cuda:0")
    wl = W.WORKLOADS["illcond"]
    t0 = time.perf_counter()
    mats = W.illcond_batch()
    log(f"illcond batch drawn ({time.perf_counter() - t0:.1f}s)")
    As = [torch.from_numpy(a).to(dev) for a in mats]
    Xs = [torch.empty(512, 512, dtype=torch.float32, device=dev) for _ in As]
    ws = B.RootWorkspace()
    count = len(As)
    infos = {eps: torch.empty(B.ROOT_INFO_BYTES * count, dtype=torch.uint8, device=dev) for eps in wl.eps_list}

    def step():
        for eps in wl.eps_list:
            B.inv_quarter_root_batched(As, eps, normalize="none", Xs=Xs, workspace=ws, return_info=False,
                                       info_out=infos[eps])

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")
    B.trace_collect()
    B.trace_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    B.trace_enable(False)
    trace = B.trace_collect()
    ms = (t1 - t0) * 1e3 / args.steps
    # per-eps call time (events around single calls, after the timed region)
    per_eps = {}
    f64 = low = 0.0
    sbytes = {"root_stats": 0, "root_init": 0, "newton_convert": 0, "newton_slice": 0, "root_finalize": 0}
    for eps in wl.eps_list:
        info = B.decode_info(infos[eps], count)
        assert (info["flags"] == 0).all(), info[info["flags"] != 0]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        B.inv_quarter_root_batched(As, eps, normalize="none", Xs=Xs, workspace=ws, return_info=False,
                                   info_out=infos[eps])
        e1.record()
        torch.cuda.synchronize()
        ef64 = elow = 0.0
        for r in info:
            K, j = int(r["iters"]), int(r["fp64_iters"])
            a, b = newton_flops(512, K, j, final_degree=int(r["final_degree"]))
            ef64 += a
            elow += b
            for kk, v in root_stream_bytes(512, 4, False, K, j).items():
                sbytes[kk] += v * args.steps
        f64 += ef64 * args.steps
        low += elow * args.steps
        cms = e0.elapsed_time(e1)
        per_eps[f"{eps:g}"] = {"ms_per_call": round(cms, 3), "roots_per_s": round(count / (cms / 1e3), 1),
                               "iters": [int(info["iters"].min()), int(info["iters"].max())],
                               "fp64_iters": [int(info["fp64_iters"].min()), int(info["fp64_iters"].max())],
                               "tflops": round((ef64 + elow) / (cms / 1e3) / 1e12, 2)}
        log(f"eps {eps:g}: {per_eps[f'{eps:g}']}")
    moment = moment_flops(512) * count * len(per_eps) * args.steps
    kernels = kernel_table(trace, {f64_class(512): f64, "newton_x3": low, "root_moment": moment}, sbytes)
    engines = engine_table(kernels)
    annotate_engines(engines, peaks)
    dname = max((kv for kv in kernels.items() if "tflops" in kv[1]), key=lambda kv: kv[1]["ms_total"])[0]
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on its sample")
        cpu = cpu_baseline_illcond(mats, wl.eps_list)
        log(f"oracle: {cpu['value']:.3f} roots/s on {cpu['cores']} BLAS threads")
    out = {
        "metric": ILLCOND_METRIC,
        "value": round(len(wl.eps_list) * count / (ms / 1e3), 3),
        "unit": "roots/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "data": "synthetic",
        "config": {"workload": "illcond", "matrices": count, "d": 512, "eps": list(wl.eps_list),
                   "normalize": "none", "calls_per_step": len(wl.eps_list)},
        "per_eps": per_eps,
        "engines": engines,
        "roofline": roofline_for(kernels, dname, "illcond"),
        "rooflines": {n: roofline_for(kernels, n, "illcond") for n in kernels
                      if "tflops" in kernels[n] or "gb_per_s" in kernels[n]},
        "kernels": kernels,
        "cpu_baseline": cpu,
        "peaks": peaks,
    }
    print(json.dumps(out), flush=True)
    return 0


CANS_METRIC = "inverse square roots/s (scaled CANS coupled Newton-Schulz, S^-1/2 of SPD 8192x8192, batch 4)"


def bench_cans(args, torch, B, peaks):
    """The OKLS page's root benchmark shape (section 2.4, figure 4): one
    inv_sqrt_root_batched call on 4 SPD matrices of 8192 x 8192 (float32,
    S = G G^T / 8192 + eps I with G Gaussian: condition number about 1e3),
    timed per call with the library's HIP events around each launch."""
    d, batch, eps = 8192, 4, 4e-3
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(8192)
    As = []
    for _ in range(batch):
        G = torch.randn(d, d, generator=gen, device=dev, dtype=torch.float32)
        As.append(G @ G.T.contiguous() / d)
    del G
    Ws = [torch.empty(d, d, dtype=torch.float32, device=dev) for _ in As]
    ws = B.RootWorkspace()
    infos = torch.empty(B.ROOT_INFO_BYTES * batch, dtype=torch.uint8, device=dev)

    def step():
        B.inv_sqrt_root_batched(As, eps, normalize="none", precision=args.precision, Xs=Ws, workspace=ws,
                                return_info=False, info_out=infos)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup call {i + 1}/{args.warmup} done")
    B.trace_collect()
    B.trace_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    B.trace_enable(False)
    trace = B.trace_collect()
    info = B.decode_info(infos, batch)
    assert (info["flags"] == 0).all(), info
    ms = (t1 - t0) * 1e3 / args.steps
    g = sym_gemm_flops(d)
    # 27 products, all symmetric in exact arithmetic: 9 P products (cans_p), 18 Y/Z products (cans_yz)
    flops = {"cans_p": 9 * g * batch * args.steps, "cans_yz": 18 * g * batch * args.steps}
    prec = "f16"
    kernels = {}
    for name, (launches, kms) in sorted(trace.items()):
        ent = {"launches": launches, "ms_total": round(kms, 3), "ms_avg": round(kms / launches, 4)}
        if name in flops:
            tf = flops[name] / (kms / 1e3) / 1e12
            mult = 3 if args.precision == "split" else 1
            ent.update({"tflops": round(tf, 2), "mfma_tflops": round(mult * tf, 2), "peak": PEAK_TFLOPS[prec],
                        "frac": round(mult * tf / PEAK_TFLOPS[prec], 4)})
        kernels[name] = ent
    dname, dk = max(((k, v) for k, v in kernels.items() if k in flops), key=lambda kv: kv[1]["ms_total"])
    roofline = {"bound": "mfma", "kernel": dname, "achieved": dk["mfma_tflops"], "peak": dk["peak"],
                "unit": "TFLOP/s", "frac": dk["frac"],
                "traffic": recorded_traffic(dname, f"cans8192_{args.precision}", "cans"),
                "achieved_per_launch": "algorithmic fp16 MFMA flops of the class (symmetric-product count; "
                                       "x3 for split products) / sum of its event-measured launch durations"}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        import numpy as np

        log("timing the fp64 oracle on one 8192 x 8192 root")
        A0 = As[0].double().cpu().numpy()
        host, cores = host_cores()
        c0 = time.perf_counter()
        oracle.inv_sqrt_root(A0, eps, "none")
        sec = time.perf_counter() - c0
        cpu = {"value": round(1.0 / sec, 5), "unit": "roots/s", "cores": cores, "host_cores": host, "kind": "oracle", "blas": blas_vendor(),
               "sample": "one 8192 x 8192 root of the batch (eigh, fp64 numpy/LAPACK)", "seconds": round(sec, 2)}
        log(f"oracle: {sec:.1f}s per root on {cores} threads")
    out = {
        "metric": CANS_METRIC,
        "value": round(batch / (ms / 1e3), 4),
        "unit": "roots/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 products, f32 accumulation" if args.precision == "f16" else "split-f16 products (f32-accurate)",
        "data": "synthetic",
        "config": {"workload": "cans8192", "d": d, "batch": batch, "eps": eps, "normalize": "none",
                   "precision": args.precision, "steps_per_root": 10, "products_per_root": 27},
        "tflops": round((flops["cans_p"] + flops["cans_yz"]) / args.steps / (ms / 1e3) / 1e12, 2),
        "roofline": roofline,
        "kernels": kernels,
        "residual_max": float(info["residual"].max()),
        "cpu_baseline": cpu,
        "peaks": peaks,
    }
    print(json.dumps(out), flush=True)
    return 0


POLAR_METRIC = "orthogonalised matrices/s (CANS polar, 10 steps; MoE share 64 x 3072x1536 + 64 x 1536x3072)"


def bench_polar(args, torch, B, peaks):
    """One polar_cans_batched call over the 128 expert gradients of the MoE
    share (step-1 sparse-row gradients, host-drawn), timed per call with the
    library's HIP events around each launch."""
    from matrix_roots_amd import workloads as W

    wl = W.WORKLOADS["moe"]
    dev = torch.device("cuda:0")
    Gs = [torch.from_numpy(W.gradient("moe", w, 1)).to(dev) for w in range(len(wl.shapes))]
    Os = [torch.empty_like(G) for G in Gs]
    ws = B.RootWorkspace()
    infos = torch.empty(B.ROOT_INFO_BYTES * len(Gs), dtype=torch.uint8, device=dev)

    def step():
        B.polar_cans_batched(Gs, precision=args.precision, Os=Os, workspace=ws, return_info=False, info_out=infos)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup call {i + 1}/{args.warmup} done")
    B.trace_collect()
    B.trace_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    B.trace_enable(False)
    trace = B.trace_collect()
    info = B.decode_info(infos, len(Gs))
    assert (info["flags"] == 0).all(), info
    ms = (t1 - t0) * 1e3 / args.steps
    gram = update = 0.0
    for G in Gs:
        M, N = max(G.shape), min(G.shape)
        gram += 10 * float(N) * (N + 1) * M  # A = X^T X, symmetric count
        update += 10 * 2.0 * M * N * N  # X A
    flops = {"polar_gram": gram * args.steps, "polar_update": update * args.steps}
    mult = 3 if args.precision == "split" else 1
    kernels = {}
    for name, (launches, kms) in sorted(trace.items()):
        ent = {"launches": launches, "ms_total": round(kms, 3), "ms_avg": round(kms / launches, 4)}
        if name in flops:
            tf = flops[name] / (kms / 1e3) / 1e12
            ent.update({"tflops": round(tf, 2), "mfma_tflops": round(mult * tf, 2), "peak": PEAK_TFLOPS["f16"],
                        "frac": round(mult * tf / PEAK_TFLOPS["f16"], 4)})
        kernels[name] = ent
    dname, dk = max(((k, v) for k, v in kernels.items() if k in flops), key=lambda kv: kv[1]["ms_total"])
    roofline = {"bound": "mfma", "kernel": dname, "achieved": dk["mfma_tflops"], "peak": dk["peak"],
                "unit": "TFLOP/s", "frac": dk["frac"],
                "traffic": recorded_traffic(dname, f"polar_moe_{args.precision}", "polar"),
                "achieved_per_launch": "algorithmic fp16 MFMA flops of the class (symmetric Gram counted once; "
                                       "x3 for split products) / sum of its event-measured launch durations"}
    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        host, cores = host_cores()
        sample = [Gs[0].cpu().numpy(), Gs[-1].cpu().numpy()]
        c0 = time.perf_counter()
        for _ in range(4):
            for g in sample:
                oracle.polar_cans(g)
        sec = (time.perf_counter() - c0) / 8
        cpu = {"value": round(1.0 / sec, 4), "unit": "matrices/s", "cores": cores, "host_cores": host, "kind": "oracle", "blas": blas_vendor(),
               "sample": "E0.in (3072x1536) and E63.out (1536x3072), 4 times each (thin SVD, fp64 numpy/LAPACK)",
               "seconds": round(8 * sec, 2)}
        log(f"oracle: {sec:.2f}s per matrix on {cores} threads")
    out = {
        "metric": POLAR_METRIC,
        "value": round(len(Gs) / (ms / 1e3), 4),
        "unit": "matrices/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 products, f32 accumulation" if args.precision == "f16" else "split-f16 products (f32-accurate)",
        "data": "synthetic",
        "config": {"workload": "polar_moe", "matrices": len(Gs), "shapes": ["3072x1536", "1536x3072"],
                   "precision": args.precision, "steps_per_matrix": 10},
        "tflops": round((gram + update) / (ms / 1e3) / 1e12, 2),
        "roofline": roofline,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "peaks": peaks,
    }
    print(json.dumps(out), flush=True)
    return 0


def calibration_copies(torch, dev, mib):
    src = torch.ones(mib * 2 ** 18, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"calibration copies of {mib} MiB done")


def vendor_gemm(torch, dev):
    """torch.matmul (hipBLASLt / rocBLAS) on the shape of the width-1024 set's
    4096 x 4096 Grams, full products, contiguous operands: what the vendor
    library sustains on this device with real data, as context for the
    hand-written kernels' rates (which count symmetric products as d^2 (d+1))."""
    out = {"shape": "batch 16 (fp16) / 4 (fp64) of 4096 x 4096 x 4096, C = A B, flops 2 m n k; int8: "
                    "torch._int_mm of one 8192 x 8192 x 8192 product (int32 result), operations 2 m n k"}
    for name, dt, b, reps in (("f16", torch.float16, 16, 10), ("f64", torch.float64, 4, 4)):
        g = torch.Generator(device=dev)
        g.manual_seed(0)
        A = torch.randn(b, 4096, 4096, device=dev, dtype=dt, generator=g)
        Bm = torch.randn(b, 4096, 4096, device=dev, dtype=dt, generator=g)
        C = torch.empty_like(A)
        for _ in range(2):
            torch.matmul(A, Bm, out=C)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.matmul(A, Bm, out=C)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        out[name] = round(2.0 * b * 4096 ** 3 / (ms / 1e3) / 1e12, 1)
        del A, Bm, C
    # int8 with int32 accumulation (the digit-plane products' arithmetic)
    n = 8192
    A = torch.randint(-64, 64, (n, n), device=dev, dtype=torch.int8)
    Bm = torch.randint(-64, 64, (n, n), device=dev, dtype=torch.int8)
    for _ in range(2):
        torch._int_mm(A, Bm)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        torch._int_mm(A, Bm)
    e1.record()
    torch.cuda.synchronize()
    out["i8"] = round(2.0 * n ** 3 / (e0.elapsed_time(e1) / 5 / 1e3) / 1e12, 1)
    del A, Bm
    torch.cuda.empty_cache()
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="w1024",
                    choices=["toy", "w1024", "w2048", "moe", "illcond", "cans8192", "polar_moe"])
    ap.add_argument("--precision", default="f16", choices=["f16", "split"],
                    help="products of the cans8192 (inv_sqrt_root_batched) and polar_moe (polar_cans_batched) "
                         "workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--state-dtype", default="f64", choices=["f64", "f32"])
    ap.add_argument("--optimizer-step", action="store_true",
                    help="time the whole optimizer step: momentum EMA, Gram EMA, roots, apply to the momentum, "
                         "hyperball update of the weights")
    ap.add_argument("--packed-state", action="store_true",
                    help="keep the Gram states packed (upper triangle by rows, d(d+1)/2 elements)")
    ap.add_argument("--gradients", default="auto", choices=["auto", "host", "device"],
                    help="where the synthetic gradients are drawn: host = the seeded numpy draws the "
                         "parity tests use; device = same distribution drawn with torch on the GPU "
                         "(auto: device for w2048, whose Haar factors take seconds each on the host)")
    ap.add_argument("--reps", type=int, default=None,
                    help="state-reset repetitions of the workload's own steps after the timed region "
                         "(default 3; 1 for w2048)")
    ap.add_argument("--no-size-classes", dest="size_classes", action="store_false",
                    help="skip the per-size-class root calls on the final state")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as HIP graph replays (one captured graph per gradient of the cycle)")
    ap.add_argument("--method", default="auto", choices=["auto", "jacobi", "newton"],
                    help="root method of the step's root call (auto: Jacobi for d <= 32, else Newton)")
    ap.add_argument("--no-vendor-gemm", dest="vendor_gemm", action="store_false",
                    help="skip timing torch.matmul (the vendor GEMM) on the 4096^3 shape as context")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="run a plain device copy of this many MiB 3 times first (counter calibration)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path has no "
              f"cross-GPU exchange to time)", file=sys.stderr)
        return 2
    if args.reps is None:
        args.reps = 1 if args.workload == "w2048" else 3

    import torch

    from matrix_roots_amd import binding as B
    from matrix_roots_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    B.library()
    dev = torch.device("cuda:0")
    # the device's matrix-core peaks: from CU count x clock, and measured by
    # register-only MFMA loops (reported beside the published figures the
    # roofline fractions use)
    peaks = B.measure_peaks()
    peaks["published_tflops"] = dict(PEAK_TFLOPS)
    if args.vendor_gemm:
        peaks["vendor_gemm_tflops"] = vendor_gemm(torch, dev)
    log(f"peaks: {peaks}")
    if args.calibration_copy_mib > 0:
        calibration_copies(torch, dev, args.calibration_copy_mib)
    if args.workload == "cans8192":
        return bench_cans(args, torch, B, peaks)
    if args.workload == "polar_moe":
        return bench_polar(args, torch, B, peaks)
    if args.workload == "illcond":
        return bench_illcond(args, torch, B, W, peaks)
    return bench_steps(args, torch, B, W, peaks)


if __name__ == "__main__":
    sys.exit(main())
