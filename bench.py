"""Benchmark: attention forward TFLOP/s on the causal GQA 8K workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--all] [--no-cpu] [--only matmul]

One step = one launch of the whole hot path (``tileattn_fwd``, called
through its C-ABI mirror with arguments marshalled once) on the causal
grouped-query workload B=1, Hq=32, Hkv=8, Sq=Sk=8192, D=128, bf16, with
inputs already resident in HBM.  Prints ONE JSON line on stdout; extra
diagnostics go to stderr.

The default warmup (100 launches, about 45 ms) outlasts the GPU's power
management transient: after an idle spell the first ~40 launches of this
workload run up to 25% slower than the sustained rate while the engine
clock settles, so the timed steps measure the sustained rate.

FLOP per step = 4*B*Hq*Sq*Sk*D, halved for causal.  The roofline object
prices the kernel against MI355X's dense bf16 MFMA peak (2.5 PFLOP/s:
256 CUs x 2048 bf16 FMA/clk x 2 x 2.4 GHz = 2516.6 TFLOP/s), with the
kernel's mean launch duration taken from one pair of HIP events around the
timed launches on the launch stream (span / steps).
The CPU baseline is the fp64 oracle run on the same workload on the host's
cores.  ``traffic`` is the kernel's HBM bytes per launch from the committed
rocprofv3 counter summary in profiles/ (null when the kernel changed since).

``--all`` also times, on stderr, the bf16 matrix product (tileattn_matmul),
the row softmax and fused GELU (GB/s against the 8 TB/s HBM peak), the other
attention workloads, the biased / block-masked variants and one KV head's
share of the headline; ``--only matmul``, ``--only rowwise`` or ``--only
shard`` (that share, chunked key split) times just those and prints no JSON
line.
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


def raw_launcher(ta, fn, *args):
    """A step that calls one C-ABI mirror with arguments marshalled once (the
    library checks them on every call), so that timed steps carry none of the
    torch wrapper's per-call Python checks: with kernels of ~100 us those can
    outlast the kernel and leave the GPU waiting for the host."""
    def step():
        rc = fn(*args)
        if rc != 0:
            raise ta.TileAttnError(rc, fn.__name__)
    return step


def time_steps(step, steps, warmup, stream=None):
    """Time a launch function: ``warmup`` untimed calls, a pass of min(steps,
    50) calls with events around each one (for the median and minimum), then
    the timed region: ``steps`` calls back to back between one pair of
    events on the launch stream.  Returns (wall ms per call by the host
    clock, mean ms per call by the events' span, median ms, minimum ms).
    Events around every launch add their own packets between the kernels
    (about 7 us a step), so the mean, not the median, prices a launch."""
    stream = stream or torch.cuda.current_stream()
    for _ in range(warmup):
        step()
    n = min(steps, 50)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for i in range(n):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    mean_ms = t_start.elapsed_time(t_end) / steps
    ev = np.array([a.elapsed_time(b) for a, b in zip(starts, ends)])
    return wall_ms, mean_ms, float(np.median(ev)), float(ev.min())


def time_workload(ta, w, steps, warmup, key_chunks=False):
    """Return (ms_per_step wall, mean kernel ms from events, median, min).

    ``key_chunks``: time ``tileattn_fwd_ws`` (the chunked key split where the
    library takes it; its workspace allocated once, outside the timed steps)
    instead of the plain entry point."""
    from tiled_attention_tileattn_amd.inputs import make_inputs

    q, k, v = make_inputs(w, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    # One call through the torch wrapper (its checks), then the timed steps
    # through the same entry point's raw mirror.
    ta.forward(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream)
    fn = {torch.bfloat16: ta.tileattn_fwd, torch.float16: ta.tileattn_fwd_f16,
          torch.float32: ta.tileattn_fwd_f32}[q.dtype]
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.D, w.scale, w.causal)
    if key_chunks:
        n = ta.tileattn_fwd_workspace_size(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.D, w.causal)
        ws = torch.empty(max(n, 16), dtype=torch.uint8, device="cuda")
        step = raw_launcher(ta, ta.tileattn_fwd_ws, *ptrs, None, int(q.dtype == torch.float16), ws.data_ptr(), n,
                            stream.cuda_stream)
    else:
        step = raw_launcher(ta, fn, *ptrs, stream.cuda_stream)
    times = time_steps(step, steps, warmup, stream)
    del q, k, v, o, lse
    return times


def shard_lines(ta, steps, warmup, plain):
    """One GPU's share of the headline if its KV heads were spread over Hkv
    GPUs (head sharding needs no communication): the same call on one KV
    head and its query heads, through tileattn_fwd (if ``plain``) and
    through tileattn_fwd_ws (the chunked key split)."""
    from dataclasses import replace

    from tiled_attention_tileattn_amd.inputs import HEADLINE, WORKLOADS

    w = WORKLOADS[HEADLINE]
    sh = replace(w, name=f"{HEADLINE} head shard", Hq=w.Hq // w.Hkv, Hkv=1)
    for chunks in ((False, True) if plain else (True,)):
        _, mean, med, mn = time_workload(ta, sh, steps, warmup, key_chunks=chunks)
        entry = "tileattn_fwd_ws, chunked key split" if chunks else "tileattn_fwd"
        log(f"{HEADLINE}, one of {w.Hkv} head shards (B={sh.B}, Hq={sh.Hq}, Hkv=1; {entry}): "
            f"mean {mean*1e3:.1f} us (median {med*1e3:.1f}, min {mn*1e3:.1f}) -> {sh.flop()/mean/1e9:.1f} TFLOP/s "
            f"({sh.flop()/mean/1e9/PEAK_BF16_TFLOPS*100:.1f}% of bf16 peak)")


def visible_pairs(mask, Hq, Sq, Sk, causal, block=64):
    """Query-key pairs a block mask [Hm, nq, nk] (and causal) leaves visible, summed over
    the Hq query heads (a single plane is shared by all of them): the counted
    work of a masked workload is 4*D per pair and batch entry."""
    m = mask.to(torch.int64)
    if m.shape[0] == 1:
        m = m * Hq
    total = 0
    for qb in range(m.shape[1]):
        rows = min(block, Sq - qb * block)
        for kb in range(m.shape[2]):
            cols = min(block, Sk - kb * block)
            if causal:
                # pairs (i, j) of the block with j <= i
                i0, j0 = qb * block, kb * block
                if j0 + cols - 1 <= i0:
                    n = rows * cols
                elif j0 > i0 + rows - 1:
                    n = 0
                else:
                    n = sum(max(0, min(cols, i - j0 + 1)) for i in range(i0, i0 + rows))
            else:
                n = rows * cols
            total += int(m[:, qb, kb].sum()) * n
    return total


def time_ext(ta, w, steps, warmup, mask, alibi=True):
    """Time the ALiBi / block-mask entry point on workload w's shape (mask None:
    no block mask; alibi False: no bias)."""
    from tiled_attention_tileattn_amd.inputs import alibi_slopes, make_inputs

    q, k, v = make_inputs(w, device="cuda")
    slopes = alibi_slopes(w.Hq).cuda() if alibi else None
    full = torch.ones(1, -(-w.Sq // 64), -(-w.Sk // 64), dtype=torch.uint8)
    pairs = visible_pairs(full if mask is None else mask, w.Hq, w.Sq, w.Sk, w.causal)
    mask = None if mask is None else mask.cuda()
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    ta.forward(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse, stream=stream,
               alibi_slopes=slopes, block_mask=mask)
    run = raw_launcher(ta, ta.tileattn_fwd_ext, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                       lse.data_ptr(), w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.D, w.scale, w.causal,
                       None if slopes is None else slopes.data_ptr(),
                       None if mask is None else mask.data_ptr(), 1 if mask is None else mask.shape[0],
                       int(q.dtype == torch.float16), stream.cuda_stream)
    _, mean_ms, _, _ = time_steps(run, steps, warmup, stream)
    t = mean_ms * 1e-3
    return t, 4.0 * w.B * w.D * pairs


def time_events(fn, steps, warmup):
    """(mean, median) seconds per call of fn on the current stream: the mean
    over the timed region, the median over a per-launch pass (time_steps)."""
    _, mean_ms, med_ms, _ = time_steps(fn, steps, warmup)
    return mean_ms * 1e-3, med_ms * 1e-3


def matmul_lines(ta, steps, warmup):
    """Time the bf16 matrix product (fp32 and bf16 C) and, for context, the
    library GEMM torch.matmul dispatches to on the same inputs."""
    from tiled_attention_tileattn_amd.inputs import MATMUL_WORKLOADS, random_matrices

    for name, (M, N, K, seed) in MATMUL_WORKLOADS.items():
        a, b = random_matrices(M, N, K, seed, device="cuda")
        flop = 2.0 * M * N * K
        for dt, dname in ((torch.float32, "fp32"), (torch.bfloat16, "bf16")):
            c = torch.empty((M, N), dtype=dt, device="cuda")
            mean, med = time_events(lambda: ta.matmul(a, b, out=c), steps, warmup)
            log(f"{name} (M=N=K={M}, C {dname}): mean {mean*1e6:.1f} us median {med*1e6:.1f} us "
                f"-> {flop/mean/1e12:.1f} TFLOP/s ({flop/mean/1e12/PEAK_BF16_TFLOPS*100:.1f}% of bf16 peak)")
        c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        mean, _ = time_events(lambda: torch.matmul(a, b, out=c), steps, warmup)
        log(f"{name}: torch.matmul (ROCm library GEMM, C bf16, context only): mean {mean*1e6:.1f} us "
            f"-> {flop/mean/1e12:.1f} TFLOP/s")
        del a, b, c


PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, 8 TB/s


def device_peak_line(props) -> str:
    """The dense bf16 MFMA peak recomputed from this device: compute units x
    4096 FLOP/clk x its peak engine clock (hipDeviceAttributeClockRate, kHz,
    read through the HIP runtime that torch and the library already use).
    Printed beside the published figure the metric divides by."""
    import ctypes
    cus = props.multi_processor_count
    try:
        hip = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD)
        khz = ctypes.c_int(0)
        # 5 = hipDeviceAttributeClockRate in hip_runtime_api.h's enum
        if hip.hipDeviceGetAttribute(ctypes.byref(khz), 5, torch.cuda.current_device()) != 0 or khz.value <= 0:
            raise OSError("hipDeviceGetAttribute failed")
        peak = cus * 4096 * khz.value * 1e3 / 1e12
        return (f"CUs={cus}, peak engine clock {khz.value / 1e3:.0f} MHz -> dense bf16 peak "
                f"{peak:.1f} TFLOP/s (the metric uses the published {PEAK_BF16_TFLOPS})")
    except (OSError, RuntimeError) as e:
        return f"CUs={cus}, peak engine clock unavailable ({e}); the metric uses the published {PEAK_BF16_TFLOPS}"


def rowwise_lines(ta, steps, warmup):
    """Time the row softmax and the fused GELU: algorithmic bytes (inputs read
    once, output written once) per launch over the launch time, in GB/s."""
    from tiled_attention_tileattn_amd.inputs import ROWWISE_WORKLOADS, random_gelu_inputs, random_rows

    for name, (kind, dtype, shape, seed) in ROWWISE_WORKLOADS.items():
        esize = 4 if dtype == "fp32" else 2
        if kind == "softmax":
            x = random_rows(*shape, seed=seed, dtype=dtype, device="cuda")
            out = torch.empty_like(x)
            nbytes = 2.0 * x.numel() * esize
            mean, med = time_events(lambda: ta.softmax(x, out=out), steps, warmup)
            bufs = (x, out)
        else:
            x, w, b = random_gelu_inputs(shape[0], seed=seed, dtype=dtype, device="cuda")
            out = torch.empty_like(x)
            nbytes = 4.0 * x.numel() * esize
            mean, med = time_events(lambda: ta.gelu(x, w, b, out=out), steps, warmup)
            bufs = (x, w, b, out)
        log(f"{name}: mean {mean*1e6:.1f} us median {med*1e6:.1f} us -> {nbytes/mean/1e9:.0f} GB/s "
            f"({nbytes/mean/1e9/PEAK_HBM_GBS*100:.1f}% of HBM peak; {nbytes/2**30:.2f} GiB per launch)")
        if kind == "softmax":
            mean, _ = time_events(lambda: torch.softmax(x, dim=1, out=out), steps, warmup)
            log(f"{name}: torch.softmax (context only): mean {mean*1e6:.1f} us -> {nbytes/mean/1e9:.0f} GB/s")
        del bufs, x, out
    # What a plain streaming copy reaches on this device (context for the rates above).
    src = torch.empty(1 << 29, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    mean, _ = time_events(lambda: dst.copy_(src), steps, warmup)
    nbytes = 2.0 * src.numel() * 4
    log(f"device copy 2 GiB -> 2 GiB (torch copy_, context only): mean {mean*1e6:.1f} us -> "
        f"{nbytes/mean/1e9:.0f} GB/s ({nbytes/mean/1e9/PEAK_HBM_GBS*100:.1f}% of HBM peak)")
    del src, dst


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), or 'unknown CPU'."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline(w, sample_rows=None, min_seconds=10.0):
    """Time the fp64 oracle on workload w on this host's cores.

    The oracle forms every head's full Sq x Sk score block (causal entries
    masked, not skipped), so it does twice the counted FLOP of a causal
    workload; the rate reported is the counted FLOP over its time.  A whole
    workload that takes less than ``min_seconds`` is run again until that
    much time has passed, and the rate is the mean over the passes.  With
    ``sample_rows`` it times that many seeded random query rows (each costs
    the same Sk-key row of work) and extrapolates linearly to every row, and
    the sample string says so.
    """
    import oracle
    from tiled_attention_tileattn_amd.inputs import make_inputs

    q, k, v = make_inputs(w)
    cores = len(os.sched_getaffinity(0))
    cpu = cpu_model()
    n_rows = w.B * w.Hq * w.Sq
    t0 = time.perf_counter()
    if sample_rows is None:
        passes = 0
        while True:
            oracle.attention(q, k, v, w.scale, w.causal, threads=cores)
            passes += 1
            t = time.perf_counter() - t0
            if t >= min_seconds:
                break
        t_all = t / passes
        per_pass = f"{t_all * 1e3:.1f} ms" if t_all < 1 else f"{t_all:.2f} s"
        sample = f"the whole workload ({n_rows} query rows), {passes} pass{'es' if passes > 1 else ''} of {per_pass}"
    else:
        rows = np.random.default_rng(w.seed + 7).choice(n_rows, sample_rows, replace=False)
        oracle.attention_rows(q, k, v, w.scale, w.causal, rows, threads=cores)
        t = time.perf_counter() - t0
        t_all = t * n_rows / sample_rows
        sample = (f"{sample_rows} random query rows of {n_rows}, extrapolated linearly to all rows "
                  f"({t_all:.0f} s)")
    return {
        "value": w.flop() / t_all / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{sample}, fp64 numpy oracle with one BLAS thread per worker thread, {t:.1f} s, on {cpu}",
    }


PROFILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                       "attn_fwd_bf16_causal_gqa_8k.md")


def profiled_traffic():
    """HBM bytes per launch from the committed rocprofv3 summary, or None.

    The counters were taken on one kernel build; they are reported only while
    the kernel source still has the hash recorded with them.
    """
    try:
        from tiled_attention_tileattn_amd.rocprof_summary import source_hash

        text = open(PROFILE).read()
        fig = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
        if fig.get("source_sha256_16") != source_hash():
            return None
        return int(round(fig["traffic_bytes"]))
    except (OSError, IndexError, KeyError, ValueError):
        return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--all", action="store_true", help="also time every workload (stderr)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", choices=["matmul", "rowwise", "shard"],
                    help="time only those kernels (stderr) and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (calibrates the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import tiled_attention_tileattn_amd as ta
    from tiled_attention_tileattn_amd.inputs import HEADLINE, WORKLOADS

    torch.cuda.set_device(0)
    if args.copy_calibration:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE per dispatch
        # (256 MiB each way) gives the scale factor of those counters.
        src = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {src.numel() * 4} bytes x5")
        return
    ta.load_library()
    props = torch.cuda.get_device_properties(0)
    log(f"device: {props.name} {getattr(props, 'gcnArchName', '')} {device_peak_line(props)}")

    if args.only == "matmul":
        matmul_lines(ta, args.steps, args.warmup)
        return
    if args.only == "rowwise":
        rowwise_lines(ta, args.steps, args.warmup)
        return
    if args.only == "shard":
        shard_lines(ta, args.steps, args.warmup, plain=False)
        return

    if args.all:
        matmul_lines(ta, args.steps, args.warmup)
        rowwise_lines(ta, args.steps, args.warmup)
        for name, w in WORKLOADS.items():
            if name == HEADLINE:
                continue
            st = 3 if name == "longctx_gqa_bf16" else args.steps
            wu = 2 if name == "longctx_gqa_bf16" else args.warmup
            wall, mean, med, mn = time_workload(ta, w, st, wu)
            log(f"{name}: mean {mean*1e3:.1f} us (median {med*1e3:.1f}, min {mn*1e3:.1f}) "
                f"-> {w.flop()/mean/1e9:.1f} TFLOP/s ({w.flop()/mean/1e9/PEAK_BF16_TFLOPS*100:.1f}% of bf16 peak)")
            if not args.no_cpu:
                cb = cpu_baseline(w, sample_rows=256 if name == "longctx_gqa_bf16" else None)
                log(f"{name}: CPU oracle {cb['value']:.3g} TFLOP/s on {cb['cores']} cores ({cb['sample']})")

        # ALiBi bias + block masks on the headline shape; work counted over
        # the visible query-key pairs only.
        from tiled_attention_tileattn_amd.inputs import random_block_mask, window_block_mask

        w = WORKLOADS[HEADLINE]
        rnd = random_block_mask(w.Hq, w.Sq, w.Sk, seed=w.seed + 100, p_visible=0.5)
        win = window_block_mask(w.Sq, w.Sk, 16)
        cases = [("ALiBi", None, True),
                 ("random 50% per-head block mask", rnd, False),
                 ("ALiBi + random 50% per-head block mask", rnd, True),
                 ("ALiBi + 1024-key local window + sink block", win, True)]
        for what, mask, alibi in cases:
            t, flop = time_ext(ta, w, args.steps, args.warmup, mask, alibi)
            log(f"{HEADLINE} + {what}: mean {t*1e6:.1f} us -> {flop/t/1e12:.1f} TFLOP/s "
                f"on visible pairs ({flop/t/1e12/PEAK_BF16_TFLOPS*100:.1f}% of bf16 peak)")

        shard_lines(ta, args.steps, args.warmup, plain=True)

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
            "traffic": profiled_traffic(),   # HBM bytes per launch (rocprofv3 counters)
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
