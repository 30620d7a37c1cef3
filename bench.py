"""Benchmark of the KDA chunked forward pass on one MI355X.

One step = one forward call over the whole workload (every stage of the
forward pass runs inside it), inputs already resident in HBM: ``kda_fwd``,
or for workloads with few chains the segmented form ``kda_fwd_scan``
(``--segment-chunks``; its three launches together make the step).
``kda_fwd`` runs the pipelined chunked kernel, or for decode-shaped
workloads (at most 16 tokens per sequence) the recurrent or single-chunk
one; ``config.kernel`` names it.

The headline workload is the large throughput case: B=8, T=16384, H=32,
K=V=128, lower_bound=-5, scale=1/sqrt(128), fp32 final_state written, no
initial state, timed back to back.  By default the same run also measures
the four other configured workloads (tiny B1 T64 H2, small B2 T128 H8, long
B1 T8192 H16 with fp32 states, packed varlen N8 H32 with bf16 states), each
with the cache flushed before every launch (they fit in, or overlap, the
256 MiB MALL), and reports them under ``configs``.  Order: those four first,
then the headline (its --warmup steps, then its --steps timed steps), then
every CPU-oracle baseline, so that all GPU timing happens under steady load
(from idle, the clocks take about 25 launches of the headline to ramp up).
Prints one JSON line:

  value     head-tokens/s of the whole job (B*T*H per step / seconds per step)
  roofline  the kernel against HBM: algorithmic bytes per launch (inputs read
            once, outputs written once) / average launch time (HIP events on
            the launch stream), against 8 TB/s
  cpu_baseline  the fp64 CPU oracle timed on this host on a bounded sample of
            the same workload (whole sequences of two batch rows), and on one
            thread over two chains
  configs   per other workload: kernel ms, roofline fraction, head-tokens/s
            and the oracle's head-tokens/s on the same inputs (all chains)
  copy_gbs  a plain 1 GiB device-to-device copy on the same GPU, for context
  launch_ms_stats  the spread of the timed launches (first, min, median, max,
            first and last quarter means)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--headline-only] [--segment-chunks auto|off|N]
                       [--flush-cache] [--kernel K] [--inverse I] [--sigmoid S]

--flush-cache reads a 512 MiB buffer before every launch of the headline
(outside its HIP events), so that no launch finds its inputs in L2 or the
256 MiB MALL (a read leaves clean lines, so the launch pays no write-back for
the flush); the step time is then the mean of the per-launch event times
instead of the wall clock over the timed steps.  The other configs are always
measured this way.  --kernel, --inverse and --sigmoid pass the library's
options (the kernel and the two ablations) for the headline workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA
# Algorithmic flops per head-token of the chunked method (multiply-add = 2):
# per 16-token chunk and head 6 C K V (W S, Qt S, Kbar^T U) + 2 C^2 (3K + 2V)
# (A, P, W, U~, P U) + K V (decay) + C^3 (inverse) = 1,921,024.
FLOPS_PER_HEAD_TOKEN = 1921024 / 16
PROFILES = os.path.join(HERE, "profiles")
HEADLINE = "large_b8_t16384_h32"
OTHER_CONFIGS = ("tiny_b1_t64_h2", "small_b2_t128_h8", "long_b1_t8192_h16_state",
                 "varlen_n8_h32_bf16state")
# Host threads for the oracle: the host share of one GPU on this machine
# (16 cores), whatever the affinity mask shows.
ORACLE_THREADS_MAX = 16


def source_digest() -> str:
    """sha256 over the kernel sources, to tell whether stored counters apply."""
    csrc = os.path.join(HERE, "gated_delta_rule_36_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".cpp", ".h")):
            with open(os.path.join(csrc, name), "rb") as fh:
                h.update(name.encode() + b"\0" + fh.read())
    return h.hexdigest()


def algorithmic_bytes(x, final_dtype) -> int:
    """Bytes the method must move once: q, k, v, g, beta and out in bf16,
    A_log and dt_bias, the states, cu_seqlens."""
    B, T, H, K = x.q.shape
    rows = B * T * H
    n = rows * K * 2 * 4 + rows * 2 + rows * 128 * 2
    n += (H * 4 if x.A_log is not None else 0) + (H * K * 4 if x.dt_bias is not None else 0)
    chains = x.num_seqs * H
    if x.initial_state is not None:
        n += chains * 128 * 128 * x.initial_state.element_size()
    if final_dtype is not None:
        n += chains * 128 * 128 * (2 if str(final_dtype).endswith("bfloat16") else 4)
    if x.cu_seqlens is not None:
        n += x.cu_seqlens.numel() * 8
    return n


def stored_traffic(workload: str, kernel: str):
    """HBM bytes per launch of this workload from committed rocprofv3
    counters (profiles/traffic_<workload>.json), if they were taken on the
    current kernel sources and the same kernel; else None."""
    try:
        with open(os.path.join(PROFILES, f"traffic_{workload}.json")) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != source_digest() or rec.get("kernel_choice") != kernel:
        return None
    return rec.get("hbm_bytes_per_launch")


def oracle_threads() -> int:
    return min(ORACLE_THREADS_MAX, len(os.sched_getaffinity(0)))


def cpu_baseline(x, rows=None, one_thread=True):
    """Time the oracle on whole sequences: every sequence (rows=None) or the
    first `rows` batch rows; all heads."""
    from oracle import kda_oracle
    B, T, H, _ = x.q.shape
    if x.cu_seqlens is not None or rows is None:
        rows = B
    rows = min(rows, B)
    cores = oracle_threads()
    sl = slice(0, rows)
    cpu = lambda t: None if t is None else t.cpu()
    q, k, v, g, beta = (cpu(t[sl]) for t in (x.q, x.k, x.v, x.g, x.beta))
    init = None if x.initial_state is None else cpu(x.initial_state[sl] if x.cu_seqlens is None
                                                    else x.initial_state)
    cu = cpu(x.cu_seqlens)
    N = rows if cu is None else cu.numel() - 1
    chains = [(n, h) for n in range(N) for h in range(H)]
    args = (q, k, v, g, beta, x.scale, cpu(x.A_log), cpu(x.dt_bias), x.lower_bound)
    t0 = time.perf_counter()
    kda_oracle(*args, initial_state=init, cu_seqlens=cu, chains=chains, threads=cores)
    dt = time.perf_counter() - t0
    head_tokens = rows * T * H
    res = {"value": head_tokens / dt, "unit": "head-tokens/s", "cores": cores, "kind": "oracle",
           "affinity_cores": len(os.sched_getaffinity(0)),
           "sample": f"{len(chains)} whole (sequence, head) chains = {head_tokens} head-tokens "
                     f"({rows} of {B} batch rows, all {H} heads), fp64 token loop on {cores} "
                     f"threads, {dt:.2f} s wall"}
    if one_thread:
        t0 = time.perf_counter()
        kda_oracle(*args, initial_state=init, cu_seqlens=cu, chains=chains[:2], threads=1)
        dt1 = time.perf_counter() - t0
        seq_len = T if cu is None else int(cu[1] - cu[0])
        res["value_1thread"] = 2 * seq_len / dt1
        res["sample_1thread"] = (f"chains (0,0), (0,1) = {2 * seq_len} head-tokens on one thread, "
                                 f"{dt1:.2f} s wall")
    return res


def measure(kda, x, final_dtype, steps, warmup, flush, seg, opts):
    """Warm up, then time `steps` calls; returns (ms_per_step, mean launch ms,
    the per-launch ms in order).

    Per-launch HIP events on the launch stream give the kernel time.  With
    `flush` (a 512 MiB device buffer) it is read before every launch, outside
    the events, and the step time is the mean launch time; otherwise the
    steps run back to back and the step time is the wall clock over them."""
    import torch
    H = x.q.shape[2]
    out = torch.empty_like(x.v)
    final = None
    if final_dtype is not None:
        final = torch.empty(x.num_seqs, H, 128, 128, dtype=final_dtype, device="cuda")

    def step():
        kda.fwd(x.q, x.k, x.v, x.g, x.beta, x.scale, out, x.A_log, x.dt_bias, x.lower_bound,
                initial_state=x.initial_state, final_state=final, cu_seqlens=x.cu_seqlens,
                check_cu_seqlens=False, segment_chunks=seg, **opts)

    for _ in range(warmup):
        if flush is not None:
            flush.max()
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s, e in ev:
        if flush is not None:
            flush.max()
        s.record(stream)
        step()
        e.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [s.elapsed_time(e) for s, e in ev]
    mean_launch = sum(launch_ms) / len(launch_ms)
    # with cache flushes in between, the wall clock would count them: use the launches
    ms_per_step = mean_launch if flush is not None else wall * 1e3 / steps
    return ms_per_step, mean_launch, launch_ms


def launch_stats(launch_ms):
    """The timed launches' spread: from idle the engine clock needs some 25
    launches of the large workload to settle, so early and late launches
    differ (the mean is what `value` and `roofline` use)."""
    xs = sorted(launch_ms)
    q = max(1, len(launch_ms) // 4)
    return {"first": round(launch_ms[0], 4), "min": round(xs[0], 4),
            "median": round(xs[len(xs) // 2], 4), "max": round(xs[-1], 4),
            "first_quarter_mean": round(sum(launch_ms[:q]) / q, 4),
            "last_quarter_mean": round(sum(launch_ms[-q:]) / q, 4)}


def roofline_of(x, final_dtype, launch_ms, traffic=None):
    B, T, H, _ = x.q.shape
    launch_bytes = algorithmic_bytes(x, final_dtype)
    achieved = launch_bytes / (launch_ms / 1e3) / 1e9
    flops = B * T * H * FLOPS_PER_HEAD_TOKEN
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel_ms": round(launch_ms, 4), "bytes_per_launch": launch_bytes,
            "flops_per_launch": round(flops),
            "mfma_frac": round(flops / (launch_ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}


def segment_choice(kda, x, arg):
    if arg == "auto":
        return kda.auto_segment_chunks(x.num_seqs * x.q.shape[2], x.q.shape[1])
    return None if arg == "off" else int(arg)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the clocks take some 25 launches (about 40 ms) to settle under this load
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--headline-only", action="store_true",
                    help="measure only --workload (no other configs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--segment-chunks", default="auto",
                    help="segmented form: 'auto' (used only for workloads with few chains), "
                         "'off', or a segment length in 16-token chunks")
    ap.add_argument("--flush-cache", action="store_true",
                    help="read a 512 MiB buffer before every launch of --workload (outside "
                         "its timing)")
    ap.add_argument("--kernel", default=None, help="kda options: auto, mfma, recurrent, single")
    ap.add_argument("--inverse", default=None, help="kda options: substitution, neumann")
    ap.add_argument("--sigmoid", default=None, help="kda options: exp2, tanh")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="before warm-up, run one plain device-to-device copy of this many "
                         "bytes (untimed), as a known-size reference for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; this path runs on one GPU "
              "(every (sequence, head) chain is independent, see the design notes on "
              "sharding)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_36_amd as kda
    from gated_delta_rule_36_amd import synth

    torch.cuda.set_device(0)
    opts = {k: v for k, v in (("kernel", args.kernel), ("inverse", args.inverse),
                              ("sigmoid", args.sigmoid)) if v is not None}
    print(f"[bench] drawing {args.workload} on the GPU", file=sys.stderr, flush=True)
    x = synth.workload(args.workload, device="cuda")
    B, T, H, K = x.q.shape
    final_dtype = x.final_dtype
    torch.cuda.synchronize()
    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # context: a plain device-to-device copy of 1 GiB (read + write), best of 4
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    best = None
    for _ in range(4):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    copy_gbs = 2 * (1 << 30) / (best / 1e3) / 1e9
    del src, dst
    flush_buf = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")

    # The four other configured workloads first (GPU timing only; their CPU
    # baselines come after all GPU work): every launch is measured with the
    # cache flushed before it, and the GPU is under steady load when the
    # headline's own warm-up starts (from idle, the clocks take about 25
    # launches of the headline workload to ramp up).
    configs = {}
    others = [] if args.headline_only else [n for n in OTHER_CONFIGS if n != args.workload]
    drawn = {}
    for name in others:
        y = synth.workload(name, device="cuda")
        yB, yT, yH, _ = y.q.shape
        yseg = segment_choice(kda, y, "auto")
        step_ms, lms, _ = measure(kda, y, y.final_dtype, args.steps, args.warmup, flush_buf, yseg, {})
        rl = roofline_of(y, y.final_dtype, lms)
        ht = yB * yT * yH
        configs[name] = {
            "workload": name, "B": yB, "T": yT, "H": yH, "lower_bound": y.lower_bound,
            "varlen": y.cu_seqlens is not None,
            "initial_state": None if y.initial_state is None else str(y.initial_state.dtype),
            "final_state": None if y.final_dtype is None else str(y.final_dtype),
            "kernel": "mfma (segmented)" if yseg else kda.fwd_kernel(yT, y.cu_seqlens is not None),
            "segment_chunks": yseg, "cache_flushed": True, "head_tokens": ht,
            "ms_per_step": round(step_ms, 4), "head_tokens_per_s": ht / (step_ms / 1e3),
            "kernel_ms": rl["kernel_ms"], "frac": rl["frac"], "achieved_gbs": rl["achieved"],
            "bytes_per_launch": rl["bytes_per_launch"]}
        print(f"[bench] {name}: {step_ms:.4f} ms/step, frac {rl['frac']}", file=sys.stderr, flush=True)
        drawn[name] = y.to("cpu")  # inputs for the CPU baseline, off the GPU
        del y

    seg = segment_choice(kda, x, args.segment_chunks)
    ms_per_step, launch_ms, per_launch = measure(kda, x, final_dtype, args.steps, args.warmup,
                                                 flush_buf if args.flush_cache else None, seg, opts)
    head_tokens = B * T * H
    print(f"[bench] {args.workload}: {args.warmup} warm-up + {args.steps} timed steps, "
          f"{ms_per_step:.4f} ms/step", file=sys.stderr, flush=True)
    kernel = "mfma (segmented)" if seg else kda.fwd_kernel(T, x.cu_seqlens is not None, **opts)
    roofline = roofline_of(x, final_dtype, launch_ms,
                           None if opts else stored_traffic(args.workload, kernel))

    result = {
        "metric": "KDA fwd head-tokens/sec (K=V=128); % of HBM/MFMA roofline",
        "value": head_tokens / (ms_per_step / 1e3),
        "unit": "head-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",  # bf16 MFMA operands, fp32 accumulation and state
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "T": T, "H": H, "K": K, "V": 128,
                   "lower_bound": x.lower_bound, "varlen": x.cu_seqlens is not None,
                   "initial_state": None if x.initial_state is None else str(x.initial_state.dtype),
                   "final_state": None if final_dtype is None else str(final_dtype),
                   "segment_chunks": seg, "kernel": kernel, **opts},
        "roofline": roofline,
        "launch_ms_stats": launch_stats(per_launch),
        "copy_gbs": round(copy_gbs, 1),
        "cache_flushed": bool(args.flush_cache),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(x, rows=2)
        for name, y in drawn.items():
            configs[name]["cpu_baseline"] = cpu_baseline(y, rows=None, one_thread=False)
    if configs:
        result["configs"] = configs
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
