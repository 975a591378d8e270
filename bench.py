"""Throughput of the EMA-Gram quarter-power preconditioner step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload w1024]

One step = one pass of the whole hot path over one batch of synthetic
gradients already resident in HBM: gram_ema_update for every weight (both
Grams, float64 state), inv_quarter_root_batched over all 2 x weights Grams
(trace rescale, eps = 1e-6), precondition_apply for every weight.  The
default workload is the width-1024 transformer weight set (8 layers x
{q,k,v,o 1024x1024, up 1024x4096, down 4096x1024}, rank-32 + noise
gradients); the Gram state evolves across steps and the gradients cycle
through the workload's 5 seeded steps.

Printed: one JSON line with matrix updates/s, the dominant kernel's roofline
(algorithmic flops / event-measured launch time on the library's stream) and
the fp64 CPU oracle timed on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f32": 157.3, "f64": 78.6, "f16": 2500.0}  # MI355X dense MFMA (vendor figures)
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E (vendor figure)
# kernel class -> arithmetic whose peak bounds it
CLASS_PREC = {"newton_f64": "f64", "syrk_ema": "f64", "newton_f32": "f32", "apply_f32": "f32", "newton_x3": "f16",
              "apply_x3": "f16"}
SPLIT_CLASSES = ("newton_x3", "apply_x3")  # three fp16 MFMA products per float32-accurate product
METRIC = "preconditioned matrix updates/sec + TFLOP/s as % fp32 MFMA peak, d=1024–4096"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def sym_gemm_flops(d: int) -> float:
    """One symmetric-output product of d x d matrices: d(d+1)/2 outputs x d MACs x 2."""
    return float(d) * d * (d + 1)


def newton_flops(d: int, K: int, j: int, x_low: bool = True, final_degree: int = 1):
    """Algorithmic (upper-triangle) flops of one Newton root, split by the
    kernel class that runs them: iterations t < K-1 take 4 symmetric products
    (M^2, T2^2, T4 M, X M), the last one only X q(M): one product for the
    step's own degree-1 polynomial, two for the degree-2 Taylor finish (q(M)
    from M^2, then X q) and three for the degree-4 one (M^2, E^2 R, X q);
    t < j run M's products in float64, and the X product too unless x_low
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


def cpu_baseline(workload: str, min_seconds: float = 10.0, max_seconds: float = 30.0):
    """The fp64 oracle (as it stands): one step from zero state (Gram EMA, two
    eigendecomposition roots, apply) per (step, weight) pair, step 1's weights
    in order first (layer 0 first), until at least `min_seconds` of oracle
    time; a weight whose shape already took longer than what is left of
    `max_seconds` is skipped.  value = pairs timed / seconds."""
    import oracle
    from matrix_roots_amd import workloads as W

    try:
        import threadpoolctl

        cores = max(int(i.get("num_threads", 1)) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    wl = W.WORKLOADS[workload]
    total = 0.0
    cost = {}  # seconds per shape class (m x n and n x m cost the same)
    timed = []
    pairs = [(t, i) for t in range(1, wl.steps + 1) for i in range(len(wl.shapes))]
    for q in range(100000):  # cycles over (step, weight) only for workloads of tiny weights
        if total >= min_seconds:
            break
        t, i = pairs[q % len(pairs)]
        name, m, n = wl.shapes[i]
        key = (min(m, n), max(m, n))
        if key in cost and total + cost[key] > max_seconds:
            continue
        G = W.gradient(workload, i, t)
        t0 = time.perf_counter()
        oracle.preconditioner_step(np.zeros((m, m)), np.zeros((n, n)), G, wl.beta, wl.eps)
        dt = time.perf_counter() - t0
        cost[key] = max(cost.get(key, 0.0), dt)
        total += dt
        timed.append(f"{name} {m}x{n} {dt:.2f}s")
    shown = "; ".join(timed[:12]) + ("; ..." if len(timed) > 12 else "")
    sample = (f"one step from zero state for each of the first {len(timed)} (step, weight) pairs, step 1's "
              f"weights first ({shown}); fp64 numpy/LAPACK")
    return {"value": len(timed) / total, "unit": "matrix updates/s", "cores": cores, "kind": "oracle",
            "sample": sample, "seconds": round(total, 2)}


def per_size_class(B, torch, grams, wl):
    """One inv_quarter_root_batched call per Gram size d > 128 on the given
    (final) state, timed with events on the current stream after one untimed
    call: ms, algorithmic TFLOP/s and its fraction of the fp32 MFMA peak."""
    out = {}
    dims = [B.packed_dim(A.numel()) if A.dim() == 1 else int(A.shape[0]) for A in grams]
    for d in sorted(set(dims)):
        if d <= 128:
            continue
        As = [A for A, dd in zip(grams, dims) if dd == d]
        Xs = [torch.empty(d, d, dtype=torch.float32, device=A.device) for A in As]
        ws = B.RootWorkspace()
        B.inv_quarter_root_batched(As, wl.eps, normalize=wl.normalize, Xs=Xs, workspace=ws, return_info=False)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        raw = torch.empty(B.ROOT_INFO_BYTES * len(As), dtype=torch.uint8, device=As[0].device)
        e0.record()
        B.inv_quarter_root_batched(As, wl.eps, normalize=wl.normalize, Xs=Xs, workspace=ws, return_info=False,
                                   info_out=raw)
        e1.record()
        torch.cuda.synchronize()
        info = B.decode_info(raw, len(As))
        ms = e0.elapsed_time(e1)
        flops = sum(sum(newton_flops(d, int(r["iters"]), int(r["fp64_iters"]), final_degree=int(r["final_degree"])))
                    for r in info)
        tf = flops / (ms / 1e3) / 1e12
        out[str(d)] = {"count": len(As), "ms": round(ms, 3), "tflops": round(tf, 2),
                       "pct_fp32_mfma_peak": round(100 * tf / PEAK_TFLOPS["f32"], 2),
                       "iters": [int(info["iters"].min()), int(info["iters"].max())],
                       "fp64_iters": [int(info["fp64_iters"].min()), int(info["fp64_iters"].max())]}
        log(f"size class {d}: {out[str(d)]}")
        del Xs, ws
    return out


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
        try:
            import threadpoolctl

            cores = max(int(i.get("num_threads", 1)) for i in threadpoolctl.threadpool_info()) or 1
        except Exception:  # pragma: no cover
            cores = len(os.sched_getaffinity(0))
        c0 = time.perf_counter()
        oracle.inv_sqrt_root(A0, eps, "none")
        sec = time.perf_counter() - c0
        cpu = {"value": round(1.0 / sec, 5), "unit": "roots/s", "cores": cores, "kind": "oracle",
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

        try:
            import threadpoolctl

            cores = max(int(i.get("num_threads", 1)) for i in threadpoolctl.threadpool_info()) or 1
        except Exception:  # pragma: no cover
            cores = len(os.sched_getaffinity(0))
        sample = [Gs[0].cpu().numpy(), Gs[-1].cpu().numpy()]
        c0 = time.perf_counter()
        for _ in range(4):
            for g in sample:
                oracle.polar_cans(g)
        sec = (time.perf_counter() - c0) / 8
        cpu = {"value": round(1.0 / sec, 4), "unit": "matrices/s", "cores": cores, "kind": "oracle",
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


def recorded_traffic(kernel: str, workload: str, family: str = "quarter"):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    if the kernel sources are unchanged since the counters were taken."""
    from matrix_roots_amd import profile_summary

    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and line.split(":", 1)[0].strip() in ("traffic_bytes_per_launch", "source_sha256"):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip().strip("`")
    if rec.get("source_sha256") != profile_summary.sources_sha256(family):
        return None
    try:
        return float(rec["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def calibration_copies(torch, dev, mib):
    src = torch.ones(mib * 2 ** 18, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"calibration copies of {mib} MiB done")


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--workload", default="w1024", choices=["toy", "w1024", "w2048", "moe", "cans8192", "polar_moe"])
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
    ap.add_argument("--per-size-class", action="store_true",
                    help="after the timed steps, time one root call per Gram size class on the final state")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="run a plain device copy of this many MiB 3 times first (counter calibration)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path has no "
              f"cross-GPU exchange to time)", file=sys.stderr)
        return 2

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
    log(f"peaks: {peaks}")
    if args.workload == "cans8192":
        if args.calibration_copy_mib > 0:
            calibration_copies(torch, dev, args.calibration_copy_mib)
        return bench_cans(args, torch, B, peaks)
    if args.workload == "polar_moe":
        if args.calibration_copy_mib > 0:
            calibration_copies(torch, dev, args.calibration_copy_mib)
        return bench_polar(args, torch, B, peaks)
    if args.calibration_copy_mib > 0:
        calibration_copies(torch, dev, args.calibration_copy_mib)
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

    def step(i):
        G = grads[i % wl.steps]
        if args.optimizer_step:
            B.momentum_ema_batched(G, Ms, 0.9)
        B.gram_ema_update(G, Ls, Rs, wl.beta)
        B.inv_quarter_root_batched(Ls + Rs, wl.eps, normalize=wl.normalize, Xs=Xs, workspace=ws,
                                   return_info=False, info_out=infos[i])
        B.precondition_apply(Xs[:nw], Ms if args.optimizer_step else G, Xs[nw:], Us=Us)
        if args.optimizer_step:
            B.hyperball_update_batched(Wts, Us, 0.02)

    for i in range(args.warmup):
        step(i)
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")
    B.trace_collect()
    B.trace_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, total):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    B.trace_enable(False)
    trace = B.trace_collect()
    log(f"timed {args.steps} steps in {t1 - t0:.3f}s")

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    value = nw / (ms_per_step / 1e3)

    # algorithmic work over the timed steps
    f64 = f32 = 0.0
    iters = []
    for i in range(args.warmup, total):
        info = B.decode_info(infos[i], 2 * nw)
        assert (info["flags"] == 0).all(), info[info["flags"] != 0]
        for k, rec in enumerate(info):
            d = shapes[k % nw][0] if k < nw else shapes[k % nw][1]
            if d <= 128:
                continue
            a, b = newton_flops(d, int(rec["iters"]), int(rec["fp64_iters"]), final_degree=int(rec["final_degree"]))
            f64 += a
            f32 += b
            iters.append((int(rec["iters"]), int(rec["fp64_iters"])))
    syrk = sum(m * (m + 1) * n + n * (n + 1) * m for m, n in shapes) * args.steps
    apply_f = sum(2.0 * m * n * (m + n) for m, n in shapes) * args.steps
    step_flops = (f64 + f32 + syrk + apply_f) / args.steps

    elems = sum(m * n for m, n in shapes) * args.steps
    stream_bytes = {"momentum": 12 * elems, "hyperball_reduce": 8 * elems, "hyperball_update": 12 * elems,
                    # maxima and split copies of XR, G, XL and W^T: 8 bytes read and 4 written per element
                    "apply_split": 12 * sum(m * m + 2 * m * n + n * n for m, n in shapes) * args.steps}
    kernels = {}
    for name, (launches, ms) in sorted(trace.items()):
        flops = {"newton_f64": f64, "newton_f32": f32, "newton_x3": f32, "syrk_ema": syrk,
                 "apply_f32": apply_f, "apply_x3": apply_f}.get(name)
        ent = {"launches": launches, "ms_total": round(ms, 3), "ms_avg": round(ms / launches, 4)}
        if name in stream_bytes:
            gbs = stream_bytes[name] / (ms / 1e3) / 1e9
            ent.update({"gb_per_s": round(gbs, 1), "peak_gb_per_s": HBM_PEAK_GBS, "frac": round(gbs / HBM_PEAK_GBS, 4)})
        if flops:
            prec = CLASS_PREC[name]
            tf = flops / (ms / 1e3) / 1e12
            ent.update({"tflops": round(tf, 2), "peak": PEAK_TFLOPS[prec], "frac": round(tf / PEAK_TFLOPS[prec], 4)})
            if name in SPLIT_CLASSES:
                ent["mfma_tflops"] = round(3 * tf, 2)
        kernels[name] = ent
    def roofline_for(name):
        k = kernels[name]
        r = {"bound": "mfma", "kernel": name, "achieved": k.get("tflops"), "peak": k.get("peak"),
             "unit": "TFLOP/s", "frac": k.get("frac"), "traffic": recorded_traffic(name, args.workload),
             "achieved_per_launch": "algorithmic flops of the class over the timed steps / sum of its "
                                    "event-measured launch durations"}
        if name in SPLIT_CLASSES:
            # float32-accurate products, each three fp16 MFMA products (hi*hi, hi*lo, lo*hi)
            r.update({"mfma_achieved": k.get("mfma_tflops"),
                      "mfma_frac": round(k["mfma_tflops"] / PEAK_TFLOPS["f16"], 4),
                      "frac_of_f32_peak": round(k["tflops"] / PEAK_TFLOPS["f32"], 4),
                      "note": "achieved/frac count the float32-accurate products against the fp16 MFMA peak "
                              "the kernel runs on; mfma_* count the three fp16 products each takes"})
        return r

    dname = max(kernels.items(), key=lambda kv: kv[1]["ms_total"])[0]
    roofline = roofline_for(dname)
    # newton_f64 and newton_x3 take about the same share of the step, so
    # which one leads changes from run to run: every MFMA class's roofline
    rooflines = {n: roofline_for(n) for n in kernels if "tflops" in kernels[n]}

    size_classes = None
    if args.per_size_class:
        del ws, Xs, Us, grads  # the per-class calls take their own workspaces
        torch.cuda.empty_cache()
        size_classes = per_size_class(B, torch, Ls + Rs, wl)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on its sample")
        cpu = cpu_baseline(args.workload)
        log(f"oracle: {cpu['value']:.4f} matrix updates/s on {cpu['cores']} threads ({cpu['seconds']:.1f}s)")

    kmin = min((k for k, _ in iters), default=0)
    kmax = max((k for k, _ in iters), default=0)
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
        "dtype": "f64+f32(split-f16 products)",
        "data": "synthetic",
        "config": {"workload": args.workload, "weights": nw, "grams_per_step": 2 * nw,
                   "shapes": sorted({f"{m}x{n}" for m, n in shapes}), "beta": wl.beta, "eps": wl.eps,
                   "normalize": wl.normalize, "state_dtype": args.state_dtype, "gradients": gen,
                   "state_layout": "packed" if args.packed_state else "full", "state_gb": round(state_bytes / 1e9, 3),
                   "optimizer_step": bool(args.optimizer_step)},
        "tflops": round(step_flops / (ms_per_step / 1e3) / 1e12, 2),
        "pct_fp32_mfma_peak": round(100 * step_flops / (ms_per_step / 1e3) / 1e12 / PEAK_TFLOPS["f32"], 2),
        "newton_iters": {"min": kmin, "max": kmax},
        "roofline": roofline,
        "rooflines": rooflines,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "peaks": peaks,
    }
    if size_classes is not None:
        out["size_classes"] = size_classes
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
