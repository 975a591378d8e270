"""Summarise rocprofv3 output for one kernel of this library.

    python -m matrix_roots_amd.profile_summary \
        --fetch prof/fetch --write prof/write \
        --kernel newton_f64_kernel --copy-mib 1024
    python -m matrix_roots_amd.profile_summary --trace prof/kt

Reads the `*counter_collection.csv` files of two `rocprofv3 --pmc` runs
(FETCH_SIZE, then WRITE_SIZE; both in KiB per dispatch) of the same program.
The program must also run a plain device copy of `--copy-mib` MiB (bench.py
--calibration-copy-mib does), whose dispatches calibrate each counter: the
copy moves exactly copy-mib MiB each way, so
    scale = copy bytes / counter reading of the copy
and the kernel's HBM bytes per dispatch = its mean reading x scale.
Also prints the sha256 of the kernel sources, which bench.py compares before
it reports the traffic.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
# Sources whose kernels a counter record covers, per kernel family.
KERNEL_SOURCES = {
    "quarter": ("csrc/gemm_core.hpp", "csrc/gemm_i8.hpp", "csrc/mr_common.hpp", "csrc/launch.hpp",
                "csrc/schedule.hpp", "csrc/epilogue.hpp", "csrc/root.hip", "csrc/gram.hip", "csrc/apply.hip"),
    "cans": ("csrc/gemm_core.hpp", "csrc/gemm_h16.hpp", "csrc/mr_common.hpp", "csrc/launch.hpp", "csrc/cans.hpp",
             "csrc/epilogue.hpp", "csrc/cans.hip"),
    "step": ("csrc/mr_common.hpp", "csrc/launch.hpp", "csrc/step.hpp", "csrc/step.hip"),
    "polar": ("csrc/gemm_core.hpp", "csrc/gemm_h16.hpp", "csrc/mr_common.hpp", "csrc/launch.hpp", "csrc/cans.hpp",
              "csrc/epilogue.hpp", "csrc/polar.hpp", "csrc/polar.hip"),
}


def code_only(text: str) -> str:
    """C++ source without its comments, whitespace runs collapsed to one
    space (string and character literals kept as written): what the compiler
    sees, so that editing a comment does not change a source hash."""
    out, i, n = [], 0, len(text)
    while i < n:
        ch = text[i]
        if ch in "\"'":
            j = i + 1
            while j < n and text[j] != ch:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(ch)
            i += 1
    return " ".join("".join(out).split())


def sources_sha256(family: str = "quarter") -> str:
    """sha256 over the family's sources, comments and layout left out."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[family]:
        with open(os.path.join(HERE, rel), encoding="utf-8") as f:
            h.update(rel.encode() + b"\0" + code_only(f.read()).encode())
    return h.hexdigest()


def read_counter(run_dir: str, counter: str):
    """{kernel name: [value per dispatch]} for one counter."""
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    out = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def pick(values: dict, needle: str):
    hits = {k: v for k, v in values.items() if needle in k}
    if not hits:
        raise KeyError(f"no kernel matching {needle!r}")
    vals = [x for v in hits.values() for x in v]
    return sorted(hits), vals


def summarise(fetch_dir, write_dir, kernel, copy_mib):
    copy_bytes = copy_mib * 2 ** 20
    res = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = read_counter(d, name)
        _, copy_vals = pick(vals, "copyBuffer" if any("copyBuffer" in k for k in vals) else "copy")
        # the calibration copies are the largest copy dispatches
        top = sorted(copy_vals)[-3:]
        copy_kib = sum(top) / len(top)
        scale = copy_bytes / (copy_kib * 1024.0)
        names, kvals = pick(vals, kernel)
        mean_kib = sum(kvals) / len(kvals)
        # working dispatches: the ones that moved data (a launch whose
        # matrices have all finished exits at once and reads almost nothing)
        top = max(kvals)
        work = [v for v in kvals if v >= 0.05 * top] if top > 0 else kvals
        wmean = sum(work) / len(work)
        res[name] = {"kernels": names, "dispatches": len(kvals), "mean_kib": mean_kib, "copy_kib": copy_kib,
                     "scale": scale, "bytes_per_dispatch": mean_kib * 1024.0 * scale,
                     "working": len(work), "bytes_per_working_dispatch": wmean * 1024.0 * scale}
    return res


def trace_table(run_dir: str, working_frac: float = 0.05):
    """Markdown table of a `--kernel-trace` run: per kernel, dispatches,
    working dispatches (those lasting at least `working_frac` of the kernel's
    longest: the library launches a fixed number of Newton steps and a
    launch whose matrices have all finished exits at once), total time,
    average per dispatch and per working dispatch, and share of the total."""
    files = glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no kernel_trace.csv under {run_dir}")
    durs = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                ns = float(r["End_Timestamp"]) - float(r["Start_Timestamp"])
                durs.setdefault(r["Kernel_Name"], []).append(ns / 1e6)
    total = sum(sum(v) for v in durs.values())
    rows = []
    for name, v in durs.items():
        top = max(v)
        work = [x for x in v if x >= working_frac * top]
        rows.append((sum(v), name, len(v), len(work), sum(v) / len(v), sum(work) / len(work)))
    rows.sort(reverse=True)
    out = ["| kernel | dispatches | working | total (ms) | avg per dispatch (ms) | avg per working dispatch (ms) | % |",
           "|:--|--:|--:|--:|--:|--:|--:|"]
    for tot, name, n, nw, avg, avgw in rows:
        short = name if len(name) <= 90 else name[:87] + "..."
        out.append(f"| `{short}` | {n} | {nw} | {tot:.3f} | {avg:.4f} | {avgw:.4f} | {100 * tot / total:.2f} |")
    return "\n".join(out)


def mfma_busy(run_dir: str, kernels):
    """Matrix-core busy fraction per kernel: SQ_VALU_MFMA_BUSY_CYCLES per
    GRBM_GUI_ACTIVE cycle, summed over the kernel's dispatches, divided by the
    same ratio of the register-only MFMA loop of the matching precision
    (peak_kernel<K, 0> with K = 0 float32, 1 float64, 2 fp16, 3 int8), which
    keeps every matrix core busy: the counters' own scale (per SIMD or per
    CU) cancels."""
    busy = read_counter(run_dir, "SQ_VALU_MFMA_BUSY_CYCLES")
    active = read_counter(run_dir, "GRBM_GUI_ACTIVE")

    def ratio(needle):
        names, b = pick(busy, needle)
        _, a = pick(active, needle)
        return sum(b) / sum(a), len(b)

    out = {}
    for name, ref in kernels:
        r, n = ratio(name)
        p, _ = ratio(ref)
        out[name] = {"dispatches": n, "busy_per_active": r, "peak_busy_per_active": p, "fraction": r / p}
    return out


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--kernel")
    ap.add_argument("--copy-mib", type=float)
    ap.add_argument("--family", default="quarter", choices=sorted(KERNEL_SOURCES))
    ap.add_argument("--mfma", help="run dir of a SQ_VALU_MFMA_BUSY_CYCLES + GRBM_GUI_ACTIVE pass")
    ap.add_argument("--pair", action="append", default=[],
                    help="KERNEL=PEAK_KERNEL for --mfma (e.g. newton_i8_kernel=\"peak_kernel<3, 0>\")")
    ap.add_argument("--trace", help="run dir of a --kernel-trace run: print the per-kernel table")
    args = ap.parse_args(argv)
    if args.trace:
        print(trace_table(args.trace))
        return 0
    if args.mfma:
        res = mfma_busy(args.mfma, [tuple(x.split("=", 1)) for x in args.pair])
        for name, r in res.items():
            print(f"{name}: dispatches {r['dispatches']}; MFMA busy per active cycle {r['busy_per_active']:.2f} "
                  f"(register-only loop {r['peak_busy_per_active']:.2f}) -> {100 * r['fraction']:.1f}% busy")
        print(f"source_family: {args.family}")
        print(f"source_sha256: {sources_sha256(args.family)}")
        return 0
    if not (args.fetch and args.write and args.kernel and args.copy_mib):
        ap.error("--fetch, --write, --kernel and --copy-mib are required without --mfma")
    res = summarise(args.fetch, args.write, args.kernel, args.copy_mib)
    f, w = res["FETCH_SIZE"], res["WRITE_SIZE"]
    print(f"kernel: {', '.join(f['kernels'])}")
    print(f"dispatches: {f['dispatches']}")
    for name, r in res.items():
        print(f"{name}: mean {r['mean_kib']:.1f} KiB/dispatch; calibration copy of {args.copy_mib:g} MiB "
              f"read {r['copy_kib']:.1f} KiB -> scale {r['scale']:.4f}; {r['bytes_per_dispatch']:.4e} B/dispatch; "
              f"{r['working']} working dispatches: {r['bytes_per_working_dispatch']:.4e} B each")
    print(f"traffic_bytes_per_launch: {f['bytes_per_dispatch'] + w['bytes_per_dispatch']:.6e}")
    print(f"traffic_bytes_per_working_launch: "
          f"{f['bytes_per_working_dispatch'] + w['bytes_per_working_dispatch']:.6e}")
    print(f"source_family: {args.family}")
    print(f"source_sha256: {sources_sha256(args.family)}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
