"""Summarise rocprofv3 CSV output into a short markdown file.

    python3 -m tiled_attention_tileattn_amd.rocprof_summary \
        --trace DIR --fetch DIR --write DIR --sq DIR --copy-fetch DIR --copy-write DIR \
        --out profiles/NAME.md --commands "cmd1" "cmd2" ...

    python3 -m tiled_attention_tileattn_amd.rocprof_summary --generic SPEC_JSON \
        --trace DIR --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \
        --title TITLE --out profiles/NAME.md --commands ...

The first form covers the attention kernel (with the SQ counter pass and the
figures bench.py reads back).  The generic form takes a JSON list of kernels,
each {"key": "sub1&sub2", "label": ..., "flop": F} or {..., "bytes": B}: the
key's substrings must all occur in the kernel name, and F / B is the
algorithmic work of one launch; it prints one table row per kernel.

Each DIR is a ``rocprofv3 -f csv -d DIR -o run`` output directory of one pass
(kernel trace with --stats; then one --pmc pass per counter group).  The copy
passes profile ``bench.py --copy-calibration`` (a plain 256 MiB device copy):
what FETCH_SIZE / WRITE_SIZE read for it gives the factor that turns those
counters into bytes.  The summary ends with a JSON block of the figures that
``bench.py`` reads (it uses them only while the kernel source still has the
hash recorded here).
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import statistics

KERNEL_KEY = "attn_fwd_16_kernel<128, true, false, false, false, false>"
COPY_BYTES = 256 * 1024 * 1024
SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc", "tileattn.hip")
# Sources of the attention kernel that the recorded figures depend on.
KERNEL_SOURCES = (SRC, os.path.join(os.path.dirname(SRC), "attn_common.h"))


def source_hash(*paths: str) -> str:
    """Hash of the kernel sources (default: KERNEL_SOURCES) with comments and
    whitespace removed: the recorded figures stay valid across comment edits
    and go stale with any change to the code itself."""
    h = hashlib.sha256()
    for path in paths or KERNEL_SOURCES:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update("".join(text.split()).encode())
    return h.hexdigest()[:16]


def _csv(d: str, suffix: str):
    paths = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not paths:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    with open(paths[0]) as f:
        return list(csv.DictReader(f))


def counters(d: str, key: str):
    """Mean per-dispatch value of each counter for kernels whose name contains key."""
    acc = {}
    for r in _csv(d, "counter_collection.csv"):
        if key in r["Kernel_Name"]:
            acc.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: statistics.fmean(v) for k, v in acc.items()}


def trace_stats(d: str, key: str):
    for r in _csv(d, "kernel_stats.csv"):
        if _match(key, r["Name"]):
            return {"calls": int(r["Calls"]), "avg_ns": float(r["AverageNs"]),
                    "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"])}
    raise KeyError(key)


def trace_timed(d: str, key: str, last: int):
    """Durations (ns) of the last ``last`` dispatches of the kernel, in
    launch order: the timed steps of a bench.py run, which follow its warmup
    launches."""
    rows = [r for r in _csv(d, "kernel_trace.csv") if _match(key, r["Kernel_Name"])]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    dur = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows[-last:]]
    return {"calls": len(dur), "avg_ns": statistics.fmean(dur), "median_ns": statistics.median(dur),
            "min_ns": float(min(dur)), "max_ns": float(max(dur))}


def _match(key: str, name: str) -> bool:
    return all(part in name for part in key.split("&"))


def counters_matching(d: str, key: str):
    acc = {}
    for r in _csv(d, "counter_collection.csv"):
        if _match(key, r["Kernel_Name"]):
            acc.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: statistics.fmean(v) for k, v in acc.items()}


def copy_scales(copy_fetch: str, copy_write: str):
    cf = counters(copy_fetch, "copyBuffer").get("FETCH_SIZE") or \
        counters(copy_fetch, "elementwise")["FETCH_SIZE"]
    cw = counters(copy_write, "copyBuffer").get("WRITE_SIZE") or \
        counters(copy_write, "elementwise")["WRITE_SIZE"]
    return cf, cw, COPY_BYTES / (cf * 1024.0), COPY_BYTES / (cw * 1024.0)


def generic(a):
    spec = json.loads(a.generic)
    cf, cw, f_scale, w_scale = copy_scales(a.copy_fetch, a.copy_write)
    lines = [f"# rocprofv3: {a.title}", "",
             "Kernel trace (with --stats) and FETCH_SIZE / WRITE_SIZE passes, each a separate run.",
             (f"Times are means over each kernel's last {a.timed} dispatches (the timed steps)."
              if a.timed else "Times are means over every dispatch."),
             f"Counter bytes are scaled by what the counters read for a plain 256 MiB copy "
             f"(FETCH_SIZE x {f_scale:.3f}, WRITE_SIZE x {w_scale:.3f}).", "",
             "| kernel | workload | calls | avg time | algorithmic rate | HBM fetch | HBM write | algorithmic bytes |",
             "|---|---|---|---|---|---|---|---|"]
    figs = []
    for k in spec:
        # With --timed N, the mean over each kernel's last N dispatches (the
        # timed steps after bench.py's warmup); else over all of them.
        tr = trace_timed(a.trace, k["key"], a.timed) if a.timed else trace_stats(a.trace, k["key"])
        fk = counters_matching(a.fetch, k["key"]).get("FETCH_SIZE", float("nan"))
        wk = counters_matching(a.write, k["key"]).get("WRITE_SIZE", float("nan"))
        fb, wb = fk * 1024.0 * f_scale, wk * 1024.0 * w_scale
        avg = tr["avg_ns"] * 1e-9
        if "flop" in k:
            rate = f"{k['flop'] / avg / 1e12:.1f} TFLOP/s"
            algo = k.get("bytes")
        else:
            rate = f"{k['bytes'] / avg / 1e9:.0f} GB/s"
            algo = k["bytes"]
        lines.append(f"| `{k['key'].replace('&', ' ')}` | {k['label']} | {tr['calls']} | {tr['avg_ns']/1e3:.1f} us "
                     f"(min {tr['min_ns']/1e3:.1f}) | {rate} | {fb/2**20:.1f} MiB | {wb/2**20:.1f} MiB | "
                     f"{'%.1f MiB' % (algo / 2**20) if algo else '-'} |")
        figs.append({"key": k["key"], "label": k["label"], "calls": tr["calls"], "avg_kernel_ns": tr["avg_ns"],
                     "fetch_bytes": fb, "write_bytes": wb, **{x: k[x] for x in ("flop", "bytes") if x in k}})
    lines += ["", f"Copy calibration (256 MiB copy): FETCH_SIZE {cf:.0f} KiB, WRITE_SIZE {cw:.0f} KiB.", "",
              "Commands (run from the repository root, `export TMPDIR=/tmp`):", ""]
    lines += [f"    {c}" for c in a.commands] + ["", "```json", json.dumps(figs, indent=1), "```", ""]
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    with open(a.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    for k in ("trace", "fetch", "write", "copy-fetch", "copy-write"):
        ap.add_argument(f"--{k}", required=True)
    ap.add_argument("--sq")
    ap.add_argument("--l2", default=None, help="pass with TCC_HIT_sum and TCC_MISS_sum (L2 hit rate)")
    ap.add_argument("--generic", default=None, help="JSON list of kernels (generic form)")
    ap.add_argument("--title", default="")
    ap.add_argument("--out", required=True)
    ap.add_argument("--workload", default="causal_gqa_bf16 (B=1, Hq=32, Hkv=8, S=8192, D=128)")
    ap.add_argument("--flop", type=float, default=549755813888.0)
    ap.add_argument("--compulsory-bytes", type=float, default=168820736.0)
    ap.add_argument("--commands", nargs="*", default=[])
    ap.add_argument("--timed", type=int, default=None,
                    help="generic form: average each kernel over its last N dispatches")
    ap.add_argument("--bench-log", default=None,
                    help="stdout of the profiled bench.py run (its JSON line)")
    a = ap.parse_args()
    if a.generic:
        generic(a)
        return
    if not a.sq:
        ap.error("--sq is required for the attention summary")

    tr = trace_stats(a.trace, KERNEL_KEY)
    fetch_kib = counters(a.fetch, KERNEL_KEY)["FETCH_SIZE"]
    write_kib = counters(a.write, KERNEL_KEY)["WRITE_SIZE"]
    sq = counters(a.sq, KERNEL_KEY)
    cf = counters(a.copy_fetch, "copyBuffer").get("FETCH_SIZE") or \
        counters(a.copy_fetch, "elementwise")["FETCH_SIZE"]
    cw = counters(a.copy_write, "copyBuffer").get("WRITE_SIZE") or \
        counters(a.copy_write, "elementwise")["WRITE_SIZE"]
    f_scale = COPY_BYTES / (cf * 1024.0)
    w_scale = COPY_BYTES / (cw * 1024.0)
    fetch_b = fetch_kib * 1024.0 * f_scale
    write_b = write_kib * 1024.0 * w_scale
    bench = None
    if a.bench_log:
        for line in open(a.bench_log):
            if line.startswith("{"):
                bench = json.loads(line)
    # The kernel time the figures use: the mean over bench.py's timed steps
    # (the last ``steps`` dispatches), as bench.py's own events measure it;
    # without the bench line, over every dispatch.
    timed = trace_timed(a.trace, KERNEL_KEY, bench["steps"]) if bench else None
    avg_ns = timed["avg_ns"] if timed else tr["avg_ns"]
    avg_s = avg_ns * 1e-9
    gui = sq.get("GRBM_GUI_ACTIVE", float("nan"))
    xcds = 8
    simds = 1024
    mfma_util = sq.get("SQ_VALU_MFMA_BUSY_CYCLES", float("nan")) / (gui / xcds * simds)
    lds_conf = sq.get("SQ_LDS_BANK_CONFLICT", float("nan")) / max(sq.get("SQ_LDS_IDX_ACTIVE", 1.0), 1.0)
    l2 = counters(a.l2, KERNEL_KEY) if a.l2 else {}
    l2_hits, l2_misses = l2.get("TCC_HIT_sum"), l2.get("TCC_MISS_sum")
    l2_rate = l2_hits / (l2_hits + l2_misses) if l2_hits is not None and l2_misses is not None else None
    fig = {
        "kernel": KERNEL_KEY,
        "workload": a.workload,
        "source_sha256_16": source_hash(),
        "avg_kernel_ns": avg_ns,
        "timed_dispatches": timed["calls"] if timed else None,
        "median_kernel_ns": timed["median_ns"] if timed else None,
        "calls": tr["calls"],
        "all_dispatches_avg_ns": tr["avg_ns"],
        "tflops_at_avg": a.flop / avg_s / 1e12,
        "fetch_bytes": fetch_b,
        "write_bytes": write_b,
        "traffic_bytes": fetch_b + write_b,
        "compulsory_bytes": a.compulsory_bytes,
        "fetch_scale": f_scale,
        "write_scale": w_scale,
        "mfma_busy_frac": mfma_util,
        "lds_bank_conflict_per_active": lds_conf,
        "effective_clock_ghz": (gui / xcds) / avg_s / 1e9,
        "valu_insts": sq.get("SQ_INSTS_VALU"),
        "mfma_insts": sq.get("SQ_INSTS_MFMA"),
        "lds_insts": sq.get("SQ_INSTS_LDS"),
        "l2_hit_rate": l2_rate,
        "bench_event_mean_ns": (a.flop / (bench["roofline"]["achieved"] * 1e12) * 1e9) if bench else None,
    }
    lines = [
        f"# rocprofv3: {KERNEL_KEY}, {a.workload}",
        "",
        "Kernel-trace and counter summary of one `bench.py` run (one launch = the whole",
        "attention forward of the workload).  Counter passes are separate runs.",
        "",
        "| figure | value |",
        "|---|---|",
        f"| dispatches profiled | {tr['calls']} |",
        (f"| average kernel time, bench.py's {timed['calls']} timed steps (the last dispatches) | "
         f"{avg_ns/1e3:.1f} us (median {timed['median_ns']/1e3:.1f}, min {timed['min_ns']/1e3:.1f}, "
         f"max {timed['max_ns']/1e3:.1f}) |") if timed else "| timed steps | not identified (no bench line) |",
        f"| average kernel time, all dispatches (warmup included) | {tr['avg_ns']/1e3:.1f} us "
        f"(min {tr['min_ns']/1e3:.1f}, max {tr['max_ns']/1e3:.1f}) |",
        f"| TFLOP/s at the average (counted FLOP {a.flop:.4g}) | {fig['tflops_at_avg']:.1f} |",
        (f"| bench.py's own HIP-event mean in the traced run | {fig['bench_event_mean_ns']/1e3:.1f} us "
         f"(roofline.achieved {bench['roofline']['achieved']:.1f} TFLOP/s) |") if bench else "| bench.py line | not recorded |",
        f"| HBM fetch (FETCH_SIZE x {f_scale:.3f}) | {fetch_b/2**20:.1f} MiB |",
        f"| HBM write (WRITE_SIZE x {w_scale:.3f}) | {write_b/2**20:.1f} MiB |",
        f"| compulsory bytes (Q, K, V read; O, lse written) | {a.compulsory_bytes/2**20:.1f} MiB |",
        f"| MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE/8 x 1024 SIMDs)) | {mfma_util*100:.1f} % |",
        f"| LDS bank conflicts per active LDS cycle | {lds_conf:.4f} |",
        f"| effective engine clock (GRBM_GUI_ACTIVE/8 / kernel time) | {fig['effective_clock_ghz']:.2f} GHz |",
        f"| VALU / MFMA / LDS instructions | {fig['valu_insts']:.3g} / {fig['mfma_insts']:.3g} / {fig['lds_insts']:.3g} |",
        (f"| L2 hit rate (TCC_HIT_sum / (TCC_HIT_sum + TCC_MISS_sum); {l2_hits:.3g} hits, {l2_misses:.3g} misses) "
         f"| {l2_rate*100:.1f} % |") if l2_rate is not None else "| L2 hit rate | not collected |",
        f"| copy calibration (256 MiB copy): FETCH_SIZE / WRITE_SIZE | {cf:.0f} KiB / {cw:.0f} KiB |",
        "",
        "Commands (run from the repository root, `export TMPDIR=/tmp`):",
        "",
    ] + [f"    {c}" for c in a.commands] + [
        "",
        "```json",
        json.dumps(fig, indent=1),
        "```",
        "",
    ]
    os.makedirs(os.path.dirname(os.path.abspath(a.out)), exist_ok=True)
    with open(a.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


if __name__ == "__main__":
    main()
