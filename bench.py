"""Benchmark: attention forward TFLOP/s on the causal GQA 8K workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--all] [--no-cpu]

One step = one launch of the whole hot path (``tileattn_fwd``) on the
causal grouped-query workload B=1, Hq=32, Hkv=8, Sq=Sk=8192, D=128, bf16,
with inputs already resident in HBM.  Prints ONE JSON line on stdout; extra
diagnostics go to stderr.

FLOP per step = 4*B*Hq*Sq*Sk*D, halved for causal.  The roofline object
prices the kernel against MI355X's dense bf16 MFMA peak (2.5 PFLOP/s:
256 CUs x 2048 bf16 FMA/clk x 2 x 2.4 GHz = 2516.6 TFLOP/s), with the
kernel's duration taken from HIP events recorded on the launch stream.
The CPU baseline is the fp64 oracle on a bounded random sample of query
rows of the same workload, scaled by the sampled fraction.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

PEAK_BF16_TFLOPS = 2516.6   # dense bf16 MFMA, MI355X
METRIC = "attention fwd TFLOP/s (bf16) + % of MI355X bf16 MFMA peak, causal GQA S=8K"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def time_workload(ta, w, steps, warmup):
    """Return (ms_per_step wall, mean kernel ms from events, median, min)."""
    from tiled_attention_tileattn_amd.inputs import make_inputs

    q, k, v = make_inputs(w, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        ta.forward(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        ta.forward(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ev = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    del q, k, v, o, lse
    return wall_ms, float(ev.mean()), float(np.median(ev)), float(ev.min())


def cpu_baseline(w, target_s=10.0):
    """Time the fp64 oracle on a random sample of query rows of workload w."""
    import oracle
    from tiled_attention_tileattn_amd.inputs import make_inputs

    q, k, v = make_inputs(w)
    total = w.B * w.Hq * w.Sq
    rng = np.random.default_rng(12345)
    cores = len(os.sched_getaffinity(0))
    n = 2048
    rows = rng.choice(total, size=n, replace=False)
    t0 = time.perf_counter()
    oracle.attention_rows(q, k, v, w.scale, w.causal, rows, threads=cores)
    t_probe = time.perf_counter() - t0
    n = int(min(total, max(n, n * target_s / max(t_probe, 1e-3))))
    rows = rng.choice(total, size=n, replace=False)
    t0 = time.perf_counter()
    oracle.attention_rows(q, k, v, w.scale, w.causal, rows, threads=cores)
    t = time.perf_counter() - t0
    flop = w.flop() * n / total
    return {
        "value": flop / t / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{n} of {total} query rows drawn uniformly (seed 12345), fp64 numpy oracle, "
                  f"{t:.1f} s; FLOP credited = workload FLOP x {n}/{total}",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--all", action="store_true", help="also time every workload (stderr)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import tiled_attention_tileattn_amd as ta
    from tiled_attention_tileattn_amd.inputs import HEADLINE, WORKLOADS

    ta.load_library()
    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}")

    if args.all:
        for name, w in WORKLOADS.items():
            if name == HEADLINE:
                continue
            st = 3 if name == "longctx_gqa_bf16" else args.steps
            wu = 2 if name == "longctx_gqa_bf16" else args.warmup
            wall, mean, med, mn = time_workload(ta, w, st, wu)
            log(f"{name}: median {med*1e3:.1f} us min {mn*1e3:.1f} us "
                f"-> {w.flop()/med/1e9:.1f} TFLOP/s ({w.flop()/med/1e9/PEAK_BF16_TFLOPS*100:.1f}% of bf16 peak)")

    w = WORKLOADS[HEADLINE]
    wall, mean, med, mn = time_workload(ta, w, args.steps, args.warmup)
    flop = w.flop()
    value = flop / (wall * 1e-3) / 1e12
    achieved = flop / (mean * 1e-3) / 1e12
    log(f"{HEADLINE}: wall {wall*1e3:.1f} us/step, kernel mean {mean*1e3:.1f} us "
        f"median {med*1e3:.1f} us min {mn*1e3:.1f} us (no L2 flush between launches)")

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": HEADLINE, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": w.Sq,
                   "Sk": w.Sk, "D": w.D, "causal": w.causal, "scale": "1/sqrt(D)"},
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
