#!/usr/bin/env python3
"""Benchmark of the varlen attention hot path on one MI355X.

Prints ONE JSON line.  A step is one pass of the hot path over the headline
workload, the ModernBERT-base global layer at long context (8 packed
sequences of U[4096,8192] tokens, 52277 in all, 12 heads, head width 64,
full bidirectional attention, RoPE theta 1.6e5), inputs resident in HBM:
the in-place RoPE prologue (kattn_rope_prologue), then the attention forward
(kattn_varlen_fwd: the tile planner, then the FP32-MFMA tile kernel).  The
fused form of the same step (kattn_varlen_fwd_rope, RoPE inside the tile
loads) is timed beside it.  The same line carries the other workloads of the
path, each timed per call with HIP events on the stream it runs on and the
L2/MALL flushed between calls, after a 100 ms pre-roll of its own untimed
calls (the GPU idles while a part builds its inputs on the host, and the first
calls after that run below full clock); the two-pass prefill attention and the
decode step are also timed from a flushed loop without event pairs:

  prefill_local_w128    ModernBERT local layer, 64 x U[16,512], window 128
  prefill_global_long   the headline workload's fused and binary16-output forms
  prefill_causal_1142   SmolLM2 causal GQA prefill, one 1142-token sequence
  prefill_causal_16x2048 SmolLM2 causal GQA prefill, 16 x 2048
  prefill_causal_1142_plus_16x2048  both in one call
  decode_b64            SmolLM2 decode, 64 sequences, caches [64][3][8192][64]
  chunked_prefill_b16   SmolLM2 prefill continuing from filled caches, 16 chunks

`roofline` is for the headline step's dominant kernel (the attention tile
kernel): algorithmic FLOPs per launch over its mean launch time, from one HIP
event pair around every timed attention call on the stream it is queued on.
`traffic` comes from rocprofv3 PMC counters taken offline (profiles/), or is
null when the kernel source changed since.  `cpu_baseline` times the FP64 CPU
oracle on a bounded random sample of the headline workload's rows.
`pages_cpu_context` quotes the CPU figures the pages print (other hardware,
other work: context, not a target).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense FP32 matrix
PEAK_HBM_GBS = 8000.0           # MI355X HBM3E

HEADLINE = "2"
PARTS = {"1": "prefill_local_w128", "2": "prefill_global_long", "3a": "prefill_causal_1142",
         "3b": "prefill_causal_16x2048", "3c": "prefill_causal_1142_plus_16x2048",
         "4": "decode_b64", "5": "chunked_prefill_b16"}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the timed region is about 0.4 s of headline steps (8.2 ms each)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--preroll-ms", type=float, default=300.0,
                    help="after the warmup steps, further untimed steps until this much wall "
                         "time has passed, so the timed steps start at full clock (reported)")
    ap.add_argument("--part-preroll-ms", type=float, default=100.0,
                    help="before each part's timed calls, untimed calls of it (each after a cache "
                         "flush) for this much wall time (reported per part)")
    ap.add_argument("--parts", default="1,2,3a,3b,3c,4,5",
                    help="comma list of extra workloads to time, or 'none'")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="budget for the CPU oracle baseline (0 disables)")
    ap.add_argument("--only", default=None,
                    help="run only this workload's loop (for profiling): 1, 2, 3a, 3b, 3c, 4 or 5")
    ap.add_argument("--fused", action="store_true",
                    help="with --only: loop the fused-RoPE step instead of prologue + attention")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="with --only: also run one plain device copy of this many MiB, the "
                         "known-size kernel that scales PMC byte counters")
    return ap.parse_args()


class Flusher:
    """Reads a buffer larger than L2 + MALL so the next call starts cold.

    A read pass leaves clean lines behind; a write pass would leave dirty lines
    that the timed call then pays to write back."""

    def __init__(self, torch, nbytes=1 << 30):
        self.buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        self.sink = torch.empty((), dtype=torch.float32, device="cuda")

    def __call__(self):
        torch_sum = self.buf.sum
        self.sink.copy_(torch_sum())


def time_calls(torch, fn, steps, warmup, flush=None):
    """Mean and min ms of `fn` per call, from events recorded around each call on the current
    stream.  Every call (and the cache flush before it) is queued without a host
    synchronisation in between, so an event pair brackets GPU work only.  Each pair still
    drains the GPU before the call and waits for its last kernel, so a short call measured
    this way (decode) takes a few us longer than the same call inside a loop of steps."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        if flush is not None:
            flush()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) for a, b in evs]
    time_calls.median = float(np.median(times))
    return float(np.mean(times)), float(np.min(times))


def preroll(torch, fn, flush, ms):
    """Untimed calls of `fn` (each after a cache flush, as in the timed loop) until `ms` of wall
    time have passed, so a part is timed at the clock its own work holds rather than the one the
    previous part left.  Returns (calls, ms)."""
    n = 0
    torch.cuda.synchronize()
    t = time.perf_counter()
    while (time.perf_counter() - t) * 1e3 < ms:
        if flush is not None:
            flush()
        fn()
        torch.cuda.synchronize()
        n += 1
    return {"calls": n, "ms": round((time.perf_counter() - t) * 1e3, 1)}


def flushed_loop_ms(torch, fn, flush, n, reps=5):
    """Per call with the caches flushed before it, without an event pair around it: a loop of n
    (flush, call) pairs less a loop of n flushes alone, both queued with no host wait inside
    (the flush reads 1 GiB, so the host stays ahead of the GPU), wall clock.  The two loops
    alternate `reps` times and the median difference is returned (one pair of loops varies by
    a few us per call, which is a tenth of a call of tens of us)."""
    def loop_wall(f):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            f()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n

    diffs = [loop_wall(lambda: (flush(), fn())) - loop_wall(flush) for _ in range(reps)]
    return float(np.median(diffs))


def prefill_part(torch, key, steps, warmup, flush, preroll_ms=0.0):
    from transformer_attention_varlen_amd import metrics, workloads as wl
    from transformer_attention_varlen_amd.session import PrefillRun
    case = wl.build(key)
    run = PrefillRun(case)
    # fused first, on the unrotated inputs; then the prologue and the two-pass attention
    pre = preroll(torch, run.attention_rope, flush, preroll_ms)
    fused_ms, _ = time_calls(torch, run.attention_rope, steps, warmup, flush)
    out16 = torch.empty((case.T, case.H * 64), dtype=torch.float16, device="cuda")
    f16_ms, _ = time_calls(torch, lambda: run.attention_f16(out16, fused=True),
                           max(3, steps // 2), 1, flush)
    del out16
    run.rope()
    mean_ms, min_ms = time_calls(torch, run.attention, steps, warmup, flush)
    median_ms = time_calls.median
    # the same call without the event pair (which adds a few us to a call of tens of us)
    loop_ms = flushed_loop_ms(torch, run.attention, flush, max(steps, 100) if key != "2" else 20)
    rope_ms, _ = time_calls(torch, run.rope, max(3, steps // 4), 1, flush)
    flops = metrics.prefill_flops(case.lengths, case.H, case.window, case.causal)
    tflops = flops / (mean_ms * 1e-3) / 1e12
    rb = metrics.rope_bytes(case.T, case.H, case.G)
    res = {"workload": wl.WORKLOADS[key].name, "tokens": case.T, "seqs": case.S,
           "heads": case.H, "kv_heads": case.G, "window": case.window, "causal": case.causal,
           "attn_ms": round(mean_ms, 4), "attn_ms_min": round(min_ms, 4),
           "attn_ms_median": round(median_ms, 4),
           "mtok_s": round(case.T / (mean_ms * 1e-3) / 1e6, 3),
           "algorithmic_gflop": round(flops / 1e9, 3), "tflops": round(tflops, 2),
           "frac_fp32_mfma": round(tflops / PEAK_FP32_MFMA_TFLOPS, 4),
           "flushed_loop_ms": round(loop_ms, 4),
           "flushed_loop_frac_fp32_mfma": round(flops / (loop_ms * 1e-3) / 1e12
                                                / PEAK_FP32_MFMA_TFLOPS, 4),
           "rope_ms": round(rope_ms, 4),
           "rope_gbs": round(rb / (rope_ms * 1e-3) / 1e9, 1),
           "fused_rope_attn_ms": round(fused_ms, 4),
           "fused_tflops": round(flops / (fused_ms * 1e-3) / 1e12, 2),
           "fused_f16_out_ms": round(f16_ms, 4), "preroll": pre,
           "traffic": part_traffic(wl.WORKLOADS[key].name, "prefill.hip")}
    del run
    torch.cuda.empty_cache()
    return res


def decode_part(torch, steps, warmup, flush, preroll_ms=0.0):
    from transformer_attention_varlen_amd import metrics, workloads as wl
    from transformer_attention_varlen_amd.session import DecodeRun
    case = wl.build("4")
    run = DecodeRun(case, rotate=True)
    pre = preroll(torch, run.step, flush, preroll_ms)
    mean_ms, min_ms = time_calls(torch, run.step, steps, warmup, flush)
    median_ms = time_calls.median
    # a serving loop: steps back to back (no flush), wall clock over all of them, after a few
    # untimed steps of its own (the per-call timing above ends on a drained GPU)
    loop_steps = max(steps, 200)
    for _ in range(20):
        run.step()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(loop_steps):
        run.step()
    torch.cuda.synchronize()
    loop_ms = (time.perf_counter() - t) * 1e3 / loop_steps
    n_fl = max(steps, 100)
    flushed_ms = flushed_loop_ms(torch, run.step, flush, n_fl)
    # the same step captured once in a HIP graph and replayed (fixed shape, device counts)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run.step()
    graph_ms, _ = time_calls(torch, graph.replay, steps, warmup, flush)
    del graph
    nbytes = metrics.decode_bytes(case.used, case.H, case.G)
    gbs = nbytes / (mean_ms * 1e-3) / 1e9
    res = {"workload": wl.WORKLOADS["4"].name, "seqs": case.B, "heads": case.H,
           "kv_heads": case.G, "cap": case.cap, "sum_used": int(case.used.sum()),
           "decode_ms": round(mean_ms, 4), "decode_ms_min": round(min_ms, 4),
           "decode_ms_median": round(median_ms, 4),
           "frac_hbm_best_call": round(nbytes / (min_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "back_to_back_ms": round(loop_ms, 4),
           "back_to_back_frac_hbm": round(nbytes / (loop_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "flushed_loop_ms": round(flushed_ms, 4),
           "flushed_loop_frac_hbm": round(nbytes / (flushed_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
           "flushed_loop_how": f"{n_fl} (flush, step) pairs less {n_fl} flushes, wall clock, "
                               "median of 5 alternating repetitions",
           "graph_replay_ms": round(graph_ms, 4), "preroll": pre,
           "algorithmic_mb": round(nbytes / 1e6, 2), "gbs": round(gbs, 1),
           "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
           "traffic": part_traffic(wl.WORKLOADS["4"].name, "decode.hip")}
    del run
    torch.cuda.empty_cache()
    return res


def chunk_part(torch, steps, warmup, flush, preroll_ms=0.0):
    from transformer_attention_varlen_amd import metrics, workloads as wl
    from transformer_attention_varlen_amd.session import ChunkRun
    case = wl.build("5")
    run = ChunkRun(case, rotate=True)
    # every call appends the same chunk at the same rows, so repeated calls do equal work
    pre = preroll(torch, run.step, flush, preroll_ms)
    mean_ms, min_ms = time_calls(torch, run.step, steps, warmup, flush)
    median_ms = time_calls.median
    flops = metrics.chunk_flops(case.lengths, case.offsets, case.H)
    tflops = flops / (mean_ms * 1e-3) / 1e12
    res = {"workload": wl.WORKLOADS["5"].name, "seqs": case.B, "chunk_tokens": case.T,
           "heads": case.H, "kv_heads": case.G, "cap": case.cap, "max_ctx": case.max_ctx,
           "ms": round(mean_ms, 4), "ms_min": round(min_ms, 4), "ms_median": round(median_ms, 4),
           "mtok_s": round(case.T / (mean_ms * 1e-3) / 1e6, 3),
           "algorithmic_gflop": round(flops / 1e9, 3), "tflops": round(tflops, 2),
           "frac_fp32_mfma": round(tflops / PEAK_FP32_MFMA_TFLOPS, 4), "preroll": pre}
    del run
    torch.cuda.empty_cache()
    return res


def traffic_record(workload: str, kernel_source: str):
    """The rocprofv3 PMC record of a workload's dominant kernel (profiles/traffic.json: HBM
    bytes fetched and written per launch, scaled by a copy of known size), or None when there
    is none or the kernel source has changed since the counters were taken."""
    import hashlib
    from pathlib import Path
    root = Path(__file__).resolve().parent
    try:
        rec = json.loads((root / "profiles" / "traffic.json").read_text())[workload]
    except (OSError, KeyError, ValueError):
        return None
    src = root / "transformer_attention_varlen_amd" / "csrc" / kernel_source
    if hashlib.sha256(src.read_bytes()).hexdigest() != rec.get("source_sha256"):
        return None
    return rec


def traffic_from_profiles(workload: str, kernel_source: str):
    """HBM bytes per launch (PMC), or None (see traffic_record)."""
    rec = traffic_record(workload, kernel_source)
    return None if rec is None else rec["traffic_bytes"]


def part_traffic(workload: str, kernel_source: str):
    """The PMC traffic of a part's kernel, with the kernel (and form) it was measured on."""
    rec = traffic_record(workload, kernel_source)
    if rec is None:
        return None
    return {"bytes_per_launch": rec["traffic_bytes"], "fetch": rec["fetch_bytes"],
            "write": rec["write_bytes"], "kernel": rec["kernel"]}


def measure_ceilings(torch):
    """Reference rates of library kernels on this GPU: a cold 1 GiB read (torch's sum) and a
    copy for HBM, a large FP32 GEMM (torch.mm) for the FP32 matrix units."""
    buf = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(buf)
    other = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")

    def best_ms(fn, reps=5):
        out = []
        for _ in range(reps):
            sink.copy_(other.sum())  # evict buf from L2 / MALL
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            out.append(a.elapsed_time(b))
        return min(out)

    read_ms = best_ms(lambda: sink.copy_(buf.sum()))
    copy_ms = best_ms(lambda: dst.copy_(buf))
    n = 8192
    A = torch.randn(n, n, device="cuda")
    Bm = torch.randn(n, n, device="cuda")
    C = torch.empty(n, n, device="cuda")
    torch.mm(A, Bm, out=C)
    gemm_ms = best_ms(lambda: torch.mm(A, Bm, out=C), reps=3)
    res = {"torch_sum_read_gbs": round(buf.numel() * 4 / (read_ms * 1e-3) / 1e9, 1),
           "hbm_copy_gbs": round(2 * buf.numel() * 4 / (copy_ms * 1e-3) / 1e9, 1),
           "fp32_gemm_tflops": round(2 * n ** 3 / (gemm_ms * 1e-3) / 1e12, 2),
           "how": "best of a few: torch sum over 1 GiB (cold; a library reduction, below what "
                  "streaming reads reach), torch copy of 1 GiB (read + write bytes), "
                  "torch.mm 8192^3 FP32"}
    del buf, dst, other, A, Bm, C
    torch.cuda.empty_cache()
    return res


def visible_pairs(case, rows):
    """Keys visible to the given packed rows, summed (per head)."""
    seq = np.searchsorted(case.cu, rows, side="right") - 1
    pos = rows - case.cu[seq]
    n = case.lengths[seq].astype(np.int64)
    lo = np.zeros_like(n)
    hi = n - 1
    if case.causal:
        hi = np.minimum(hi, pos)
    if case.window >= 0:
        hw = case.window // 2
        lo = np.maximum(lo, pos - hw)
        hi = np.minimum(hi, pos + hw)
    return int(np.sum(hi - lo + 1))


def cpu_model():
    """The host CPU as /proc/cpuinfo names it: model name, family, model, stepping, and the
    number of logical CPUs it lists."""
    info = {}
    n = 0
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if ":" not in line:
                    continue
                k, v = (x.strip() for x in line.split(":", 1))
                if k == "processor":
                    n += 1
                elif k in ("model name", "cpu family", "model", "stepping") and k not in info:
                    info[k] = v
    except OSError:
        return "unknown"
    return (f"{info.get('model name', 'unknown')} (family {info.get('cpu family', '?')}, "
            f"model {info.get('model', '?')}, stepping {info.get('stepping', '?')}; "
            f"{n} logical CPUs listed)")


def oracle_threads():
    """Threads the oracle runs with: OMP_NUM_THREADS when set (a GPU machine sets it to the CPU
    share of one GPU), else every CPU the process may use."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(case, budget_s):
    """The oracle, untuned, on random samples of the workload's rows (all heads each),
    repeated until the time budget is spent."""
    import oracle
    threads = oracle_threads()
    tables = oracle.rope_tables(case.theta, max(int(case.lengths.max()), 1))
    rng = np.random.default_rng(0)
    n = 64
    spent = 0.0
    done = 0
    pairs = 0
    while spent < budget_s:
        rows = np.sort(rng.integers(0, case.T, n)).astype(np.int32)
        pairs += visible_pairs(case, rows)
        t0 = time.perf_counter()
        oracle.varlen_attention(case.q, case.k, case.v, case.cu, case.H, case.G, case.window,
                                case.causal, tables=tables, rows=rows, threads=threads)
        dt = time.perf_counter() - t0
        spent += dt
        done += n
        per_row = dt / n
        n = int(min(max(1, (budget_s - spent) / max(per_row, 1e-9)), 4 * n, case.T))
    return {"value": round(done / spent / 1e6, 6), "unit": "Mtok/s", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "fp64_gflops": round(4 * 64 * case.H * pairs / spent / 1e9, 3),
            "sample": f"{done} query rows drawn uniformly (with replacement) from the headline "
                      f"workload, all {case.H} heads each (RoPE, -inf mask, two-pass softmax in "
                      f"FP64), {spent:.1f} s on {threads} OpenMP threads"}


def pages_cpu_context():
    """The CPU figures the pages print for this method, quoted as context: an unnamed CPU, FP32,
    the SmolLM2-135M tower at its 1142-token caption prompt.  Other hardware and other work,
    so no ratio is taken against them."""
    where = "ffai-argus 0.7.3 src/text.rs"
    return {
        "hardware": "unnamed CPU (candle's CPU backend), FP32",
        "workload": "SmolLM2-135M text tower, 9 q heads / 3 kv heads, head width 64, "
                    "1142-token caption prompt and the decode steps after it",
        "masked_fill_ms_per_layer": {"value": 114.13, "gbs": 0.8,
                                     "what": "writing -inf into the causal upper triangle of "
                                             "the (9, 1142, 1142) score matrix",
                                     "cite": f"{where}, module docs, per-layer table"},
        "scale_ms_per_layer": {"value": 19.39, "cite": f"{where}, module docs, per-layer table"},
        "softmax_ms_per_layer": {"value": 5.95, "cite": f"{where}, module docs, per-layer table"},
        "matmul_gflops": {"value": [516, 591], "what": "candle matmuls at the tower's shapes",
                          "cite": f"{where}, module docs"},
        "kv_cat_ms_per_decode_token": {"value": 14.0, "mb_per_token": 52.7,
                                       "what": "recopying both caches at full length for every "
                                               "decode token, 30 layers",
                                       "cite": f"{where}, doc comment of KvAppend"},
        "here": "this library skips the masked tiles (no mask is written), folds the scale "
                "into q and appends in place; see parts.prefill_causal_1142 (one layer's "
                "attention at the same shape) and parts.decode_b64",
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by sequence or head with no exchange; see DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from transformer_attention_varlen_amd import kattn, metrics, workloads as wl
    from transformer_attention_varlen_amd.session import PrefillRun

    kattn.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)

    if args.only is not None:
        # profiling mode: just the named workload's loop, nothing else
        if args.only == "4":
            from transformer_attention_varlen_amd.session import DecodeRun
            run = DecodeRun(wl.build("4"), rotate=True)
            fn = run.step
        elif args.only == "5":
            from transformer_attention_varlen_amd.session import ChunkRun
            run = ChunkRun(wl.build("5"), rotate=True)
            fn = run.step
        else:
            run = PrefillRun(wl.build(args.only))
            fn = run.step_fused if args.fused else run.step
        for _ in range(args.warmup + args.steps):
            fn()
        torch.cuda.synchronize()
        if args.calib_copy_mib > 0:
            n = args.calib_copy_mib * (1 << 20) // 4
            src = torch.ones(n, dtype=torch.float32, device="cuda")
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            dst.copy_(src)
            torch.cuda.synchronize()
        print(json.dumps({"only": args.only, "steps": args.steps, "warmup": args.warmup,
                          "calib_copy_mib": args.calib_copy_mib}))
        return

    case = wl.build(HEADLINE)
    run = PrefillRun(case)
    # W warmup steps, then a pre-roll: further untimed steps until --preroll-ms of wall time
    # has passed, so that the timed steps run at full clock whatever W is
    for _ in range(args.warmup):
        run.step()
    torch.cuda.synchronize()
    t_pre = time.perf_counter()
    preroll_steps = 0
    while (time.perf_counter() - t_pre) * 1e3 < args.preroll_ms:
        run.step()
        preroll_steps += 1
        torch.cuda.synchronize()
    preroll_ms = (time.perf_counter() - t_pre) * 1e3
    # K timed steps bracketed by synchronisation.  In each, an event pair on the stream the
    # launches are queued on (torch's current stream) brackets the attention call (the
    # planner and the tile kernel); the prologue runs between the pairs.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        run.rope()
        a.record()
        run.attention()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    attn_times = [a.elapsed_time(b) for a, b in evs]
    attn_ms = float(np.mean(attn_times))
    ms_per_step = wall * 1e3 / args.steps
    # the fused form of the same step: RoPE inside the tile loads (q and k read-only)
    run.reset_inputs()
    for _ in range(2):
        run.step_fused()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        run.step_fused()
    torch.cuda.synchronize()
    fused_ms = (time.perf_counter() - t1) * 1e3 / args.steps
    # the two-pass step captured once in a HIP graph and replayed back to back
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run.step()
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t2) * 1e3 / args.steps
    del graph
    flops = metrics.prefill_flops(case.lengths, case.H, case.window, case.causal)
    achieved = flops / (attn_ms * 1e-3) / 1e12
    value = case.T / (ms_per_step * 1e-3) / 1e6

    out = {
        "metric": "varlen attention Mtok/s + % FP32-MFMA peak; decode KV GB/s (% HBM)",
        "value": round(value, 4), "unit": "Mtok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.WORKLOADS[HEADLINE].name, "tokens": case.T, "seqs": case.S,
                   "heads": case.H, "kv_heads": case.G, "head_dim": 64, "window": case.window,
                   "causal": case.causal, "rope_theta": case.theta,
                   "seed": wl.WORKLOADS[HEADLINE].seed,
                   "step": "RoPE prologue (in place on q and k), then the attention forward",
                   "preroll": {"steps": preroll_steps, "ms": round(preroll_ms, 1)},
                   "fused_rope_ms_per_step": round(fused_ms, 4),
                   "graph_replay_ms_per_step": round(graph_ms, 4)},
        "roofline": {"bound": "mfma",
                     "kernel": "fwd_kernel<1, 4, 64, 0, false> (FP32-MFMA tile kernel) with "
                               "plan_kernel (about 5 us) ahead of it: one event pair around each "
                               "timed kattn_varlen_fwd call",
                     "achieved": round(achieved, 3), "peak": PEAK_FP32_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_MFMA_TFLOPS, 4),
                     "traffic": traffic_from_profiles(wl.WORKLOADS[HEADLINE].name, "prefill.hip"),
                     "algorithmic_bytes_per_launch": metrics.prefill_bytes(case.T, case.H,
                                                                           case.G),
                     "mean_launch_ms": round(attn_ms, 4),
                     "median_launch_ms": round(float(np.median(attn_times)), 4),
                     "algorithmic_gflop_per_launch": round(flops / 1e9, 4)},
    }
    del run
    torch.cuda.empty_cache()

    parts = {}
    keys = [] if args.parts == "none" else [k for k in args.parts.split(",") if k]
    if keys:
        flush = Flusher(torch)
        for k in keys:
            psteps, pwarm = max(5, args.steps // 2), 2
            pms = args.part_preroll_ms
            if k == "4":
                parts[PARTS[k]] = decode_part(torch, max(psteps, 20), pwarm, flush, pms)
            elif k == "5":
                parts[PARTS[k]] = chunk_part(torch, psteps, pwarm, flush, pms)
            else:
                parts[PARTS[k]] = prefill_part(torch, k, max(3, psteps // 4) if k == "2" else psteps,
                                               pwarm, flush, pms)
        del flush
    out["parts"] = parts
    out["ceilings"] = measure_ceilings(torch) if args.parts != "none" else None
    if out["ceilings"] is not None:
        # the same rates against what the library kernels of this GPU reach (besides the
        # nominal peaks): a large FP32 GEMM for the MFMA-bound parts, a device copy for decode
        gemm = out["ceilings"]["fp32_gemm_tflops"]
        copy = out["ceilings"]["hbm_copy_gbs"]
        out["roofline"]["frac_of_measured_fp32_gemm"] = round(achieved / gemm, 4)
        for part in parts.values():
            if "tflops" in part:
                part["frac_of_measured_fp32_gemm"] = round(part["tflops"] / gemm, 4)
            if "gbs" in part:
                part["frac_of_measured_copy"] = round(part["gbs"] / copy, 4)
    if args.cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    out["pages_cpu_context"] = pages_cpu_context()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
