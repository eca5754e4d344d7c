#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-cpu-baseline] [--mode bench|copy|fwd-only|bwd-only]
                    [--splits S] [--mask lengths|random|blocks|all]
                    [--kv-heads G] [--dropout P]

Default workload: causal fp16 attention forward, B=1 H=32 N=8192 D=128 (the
headline metric: causal forward TFLOP/s and its fraction of the dense fp16
MFMA peak).  A timed step is one fa_fwd call over the whole batch; inputs are
seeded synthetic tensors already resident in HBM.  The same run also times
the backward (fa_bwd on the same shapes) and reports it under "bwd".

Prints ONE JSON line.  Timing uses torch.cuda events on the stream the
library launches on (torch's current stream); `value` is K calls between
two events.  After that region, "timing" adds the median and p95 of single
calls, the median of 7 group means of back-to-back calls, and for workloads
that fit the last-level cache the median of cold calls (each after
overwriting 512 MB).  The cpu_baseline leg times the float64 CPU oracle on a
bounded sample of the same workload.

--mode copy runs only a plain device copy of known size; it exists so that
rocprofv3 FETCH_SIZE / WRITE_SIZE counters can be calibrated against a
kernel whose HBM traffic is known.
--mode fwd-only / bwd-only launch just that pass K times (for profiling).
--splits S times the split-K/V forward (fa_fwd_ex, fa_options.num_splits = S) instead of fa_fwd (S = auto:
the count fa_fwd_splitkv_num_splits picks for the workload).
--kv-heads G gives K and V only G heads (grouped-query attention).
--dropout P times fa_fwd_ex / fa_bwd_ex with dropout (seed 1234, offset 0);
with --mask too, with both options.
--mask KIND times fa_fwd_ex / fa_bwd_ex with a seeded key-padding
mask (lengths / random / blocks / all); TFLOP/s then count only the visible
(query, key) pairs, and the one-off tile-table build is reported apart.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "causal attn fwd TFLOP/s + % MFMA peak, B1 H32 D128 N=8192 fp16"
PEAK_TFLOPS_FP16 = 2516.6   # MI355X dense fp16/bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# The pages' own figure for exactly this workload (causal fp16, B1 H32 D128,
# N=8192): 25.854 ms on an RTX 3060 Laptop GPU with PyTorch's FlashAttention
# backend ("CUDA FlashAttention: from online softmax to the long-sequence IO
# limit", §8) = 2*1*32*8192^2*128 FLOP / 25.854 ms = 21.26 TFLOP/s.
PAGE_BASELINE_TFLOPS = 2 * 32 * 8192 ** 2 * 128 / 25.854e-3 / 1e12

FWD_SOURCES = ["exact_attention_25_amd/csrc/fa_fwd.hip", "exact_attention_25_amd/csrc/fa_fwd_d128.hip",
               "exact_attention_25_amd/csrc/fa_fwd_short.hip", "exact_attention_25_amd/csrc/fa_common.hpp"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_causal_b1h32n8192d128_fp16_traffic.json")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default=None)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--mode", default="bench", choices=["bench", "copy", "fwd-only", "bwd-only"])
    p.add_argument("--splits", default="0",
                   help="time the split-K/V forward with this many key splits (split pass + merge) instead of fa_fwd; "
                        "'auto': the count fa_fwd_splitkv_num_splits picks")
    p.add_argument("--dropout", type=float, default=0.0,
                   help="time fa_fwd_ex / fa_bwd_ex with dropout of this probability (seed 1234, offset 0)")
    p.add_argument("--kv-heads", type=int, default=0,
                   help="grouped heads: K and V get this many heads (must divide H); 0 = H")
    p.add_argument("--mask", default=None, choices=["lengths", "random", "blocks", "all"],
                   help="time fa_fwd_ex / fa_bwd_ex with a seeded key-padding mask of this kind; "
                        "FLOPs then count only visible (query, key) pairs")
    return p.parse_args()


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload_name, launches_per_step=1):
    """HBM bytes per launch measured by rocprofv3 counters, if they were taken
    on the current forward-kernel sources; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("workload") != workload_name or t.get("source_hash") != source_hash(FWD_SOURCES):
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, seconds):
    """Time the float64 oracle on whole heads of the workload until about
    `seconds` have passed; report algorithmic TFLOP/s on that sample.  For a
    forward+backward workload the oracle's backward is timed the same way
    (its own heads, its own time budget) and reported under "bwd"."""
    import numpy as np
    from exact_attention_25_amd.inputs import make_inputs
    from oracle import attention_backward, attention_forward
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        pools = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in pools] or [1])
        blas = ",".join(sorted({i.get("internal_api", "?") for i in pools})) or "none"
    except Exception:
        threads = len(os.sched_getaffinity(0))
    order = [(b, h) for b in range(w.B) for h in range(w.H)]

    def time_heads(fn, flops_per_head, with_dout):
        heads_done, t_total = 0, 0.0
        for b, h in order:
            inp = make_inputs(w.B, w.H, w.N, w.D, w.dtype, seed=w.seed, spiky_keys=w.spiky_keys, heads=[(b, h)],
                              with_dout=with_dout)
            args = [inp[n][None] for n in (("q", "k", "v", "do") if with_dout else ("q", "k", "v"))]
            t0 = time.perf_counter()
            fn(*args)
            t_total += time.perf_counter() - t0
            heads_done += 1
            if t_total >= seconds:
                break
        return heads_done * flops_per_head / t_total / 1e12, heads_done, t_total

    value, heads_done, t_total = time_heads(lambda q, k, v: attention_forward(q, k, v, w.causal, w.scale),
                                            w.fwd_flops() / (w.B * w.H), False)
    rec = {
        "value": value,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "%d of %d heads of %s, float64 numpy (BLAS %s, %d host CPUs available), %.1f s" % (
            heads_done, len(order), w.name, blas, len(os.sched_getaffinity(0)), t_total),
    }
    if w.backward:
        value, heads_done, t_total = time_heads(
            lambda q, k, v, do: attention_backward(q, k, v, do, w.causal, w.scale), w.bwd_flops() / (w.B * w.H), True)
        rec["bwd"] = {
            "value": value,
            "unit": "TFLOP/s",
            "cores": threads,
            "kind": "oracle",
            "flops_counted": "10*B*H*N^2*D (causal: half), the GPU backward's count",
            "sample": "attention_backward on %d of %d heads of %s, float64 numpy (BLAS %s), %.1f s" % (
                heads_done, len(order), w.name, blas, t_total),
        }
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested; run with --gpus 1)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import exact_attention_25_amd as fa
    from exact_attention_25_amd import workloads
    from exact_attention_25_amd.inputs import make_inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.mode == "copy":
        n = 1 << 30
        src = torch.ones(n // 2, dtype=torch.float16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"mode": "copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                          "launches": args.warmup + args.steps}), flush=True)
        return

    w = workloads.HEADLINE
    if args.workload:
        named = {x.name: x for x in workloads.ALL}
        if args.workload not in named:
            sys.exit("unknown workload %s; choose from %s" % (args.workload, ", ".join(named)))
        w = named[args.workload]

    if args.splits == "auto":
        args.splits = fa.splitkv_num_splits(w.B, w.H, w.N, w.D, w.causal)
    else:
        args.splits = int(args.splits)

    tdt = torch.float16 if w.dtype == "fp16" else torch.bfloat16
    inp = make_inputs(w.B, w.H, w.N, w.D, w.dtype, seed=w.seed, spiky_keys=w.spiky_keys, with_dout=True)
    q, k, v, do = (torch.from_numpy(inp[n]).to(dev).to(tdt).contiguous() for n in ("q", "k", "v", "do"))
    del inp
    hkv = args.kv_heads or w.H
    if w.H % hkv:
        sys.exit("--kv-heads %d does not divide H=%d" % (hkv, w.H))
    if hkv != w.H:  # the first hkv heads of the drawn K and V serve as the shared heads
        k, v = k[:, :hkv].contiguous(), v[:, :hkv].contiguous()
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.N, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    tiles = None
    flop_fraction = 1.0  # visible (query, key) pairs / pairs of the unmasked workload
    mask_ms = None
    if args.mask:
        from exact_attention_25_amd.inputs import make_key_mask
        m = make_key_mask(w.B, w.N, args.mask, seed=w.seed, p=0.5)
        vis = m.astype(np.int64)
        if w.causal:
            pairs = int(np.cumsum(vis, axis=1).sum())  # row i sees visible keys j <= i
            full = w.B * w.N * (w.N + 1) // 2
        else:
            pairs = int(vis.sum()) * w.N
            full = w.B * w.N * w.N
        flop_fraction = pairs / full
        mask_dev = torch.from_numpy(m).to(dev)
        tiles = fa.mask_tiles(mask_dev)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(10):
            fa.mask_tiles(mask_dev)
        torch.cuda.synchronize()
        mask_ms = (time.perf_counter() - t0) / 10 * 1e3

    if args.dropout:  # with --mask as well: both options
        def run_fwd():
            fa.fwd_dropout(q, k, v, args.dropout, 1234, 0, causal=w.causal, scale=w.scale, out=o, lse=lse,
                           tiles=tiles)
    elif args.mask:
        def run_fwd():
            fa.fwd_masked(q, k, v, tiles, causal=w.causal, scale=w.scale, out=o, lse=lse)
    elif args.splits > 0:
        split_ws = torch.empty(max(256, fa.fwd_ex_workspace_bytes(
            w.B, w.H, w.N, w.D, w.causal, 0 if w.dtype == "fp16" else 1, fa.options(num_splits=args.splits))),
            dtype=torch.uint8, device=dev)

        def run_fwd():
            fa.fwd_splitkv(q, k, v, args.splits, causal=w.causal, scale=w.scale, out=o, lse=lse, workspace=split_ws)
    else:
        def run_fwd():
            fa.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)

    ws = torch.empty(max(256, fa.bwd_ex_workspace_bytes(w.B, w.H, w.N, w.D, w.causal, 0 if w.dtype == "fp16" else 1,
                                                        fa.options(h_kv=hkv))),
                     dtype=torch.uint8, device=dev)

    def run_bwd():
        if args.dropout:
            return fa.bwd_dropout(q, k, v, o, lse, do, args.dropout, 1234, 0, causal=w.causal, scale=w.scale,
                                  workspace=ws, tiles=tiles)
        if args.mask:
            return fa.bwd_masked(q, k, v, o, lse, do, tiles, causal=w.causal, scale=w.scale, workspace=ws)
        return fa.bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale, workspace=ws)

    if args.mode in ("fwd-only", "bwd-only"):
        run_fwd()
        fn = run_fwd if args.mode == "fwd-only" else run_bwd
        for _ in range(args.warmup + args.steps):
            fn()
        torch.cuda.synchronize()
        print(json.dumps({"mode": args.mode, "workload": w.name, "launches": args.warmup + args.steps}), flush=True)
        return

    def timed(fn, steps, warmup):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps  # ms per call

    ms = timed(run_fwd, args.steps, args.warmup)
    tflops = flop_fraction * w.fwd_flops() / (ms * 1e-3) / 1e12

    # Per-call statistics of the same forward, after the timed region (they
    # do not enter `value`): median and p95 of single calls, each between its
    # own events; the median of 7 group means of back-to-back calls (the
    # protocol for kernels of a few microseconds); and, for workloads whose
    # compulsory bytes fit the 256 MB last-level cache, the median of single
    # calls each preceded by overwriting a 512 MB buffer (cold caches).
    def per_call(fn, n, flush=None):
        ev = []
        for _ in range(n):
            if flush is not None:
                flush()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            ev.append((a, b))
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in ev)

    def group_median(fn, groups, k):
        means = []
        for _ in range(groups):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(k):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            means.append(a.elapsed_time(b) / k)
        return float(np.median(means))

    calls = per_call(run_fwd, args.steps)
    timing = {"per_call_median_ms": round(float(np.median(calls)), 4),
              "per_call_p95_ms": round(float(np.percentile(calls, 95)), 4),
              "groups_median_ms": round(group_median(run_fwd, 7, max(1, args.steps // 7)), 4)}
    if w.io_bytes_fwd() < 256e6:
        flush_buf = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
        cold = per_call(run_fwd, min(args.steps, 20), flush=flush_buf.zero_)
        timing["cold_median_ms"] = round(float(np.median(cold)), 4)
        del flush_buf
    bwd_ms = timed(run_bwd, max(1, args.steps // 2), max(1, args.warmup // 2))
    bwd_tflops = flop_fraction * w.bwd_flops() / (bwd_ms * 1e-3) / 1e12

    traffic = load_traffic(w.name) if args.splits == 0 and not args.mask and hkv == w.H and not args.dropout else None
    if args.dropout:
        kernel = "fwd_kernel<%d,%s,%sdropout %g>" % (w.D, "causal" if w.causal else "full",
                                                       "key mask," if args.mask else "", args.dropout)
    elif args.mask:
        kernel = "fwd_kernel<%d,%s,key mask>" % (w.D, "causal" if w.causal else "full")
    elif args.splits > 0:
        kernel = "fwd_kernel<%d,%s> split x%d + merge_kernel" % (w.D, "causal" if w.causal else "full", args.splits)
    else:
        kernel = "%s<%d,%s,%s>" % (fa.fwd_kernel_name(w.B, w.H, w.N, w.D, w.causal), w.D,
                                   "causal" if w.causal else "full", w.dtype)
    rec = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(tflops / PAGE_BASELINE_TFLOPS, 2) if w is workloads.HEADLINE else None,
        "vs_baseline_ref": "RTX 3060 Laptop, PyTorch FlashAttention backend, 25.854 ms = 21.26 TFLOP/s "
                           "(another machine: context only)" if w is workloads.HEADLINE else None,
        "dtype": w.dtype,
        "data": "synthetic: seeded i.i.d. N(0,1) rounded to %s (seed %d)" % (w.dtype, w.seed),
        "config": {"workload": w.name, "B": w.B, "H": w.H, "H_kv": hkv, "N": w.N, "D": w.D, "causal": w.causal,
                   "scale": w.scale},
        "pct_mfma_peak": round(100 * tflops / PEAK_TFLOPS_FP16, 2),
        "roofline": {
            "bound": "mfma",
            "kernel": kernel,
            "achieved": round(tflops, 2),
            "peak": PEAK_TFLOPS_FP16,
            "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_TFLOPS_FP16, 4),
            "traffic": traffic,
        },
        "hbm_compulsory_gbs": round(w.io_bytes_fwd() / (ms * 1e-3) / 1e9, 1),
        "timing": timing,
        "bwd": {
            "ms_per_call": round(bwd_ms, 4),
            "tflops": round(bwd_tflops, 2),
            "frac_mfma_peak": round(bwd_tflops / PEAK_TFLOPS_FP16, 4),
            "flops_counted": "10*B*H*N^2*D (causal: half): five N x N x D products",
        },
    }
    if args.dropout:
        rec["dropout"] = {"p": args.dropout, "seed": 1234, "offset": 0}
    if hkv != w.H or args.dropout:  # a different workload from the one the page's number is for
        rec["vs_baseline"] = None
        rec["vs_baseline_ref"] = None
    if args.mask:
        rec["mask"] = {"kind": args.mask, "visible_pair_fraction": round(flop_fraction, 4),
                       "mask_tiles_ms": round(mask_ms, 4),
                       "flops_counted": "visible (query, key) pairs only"}
        rec["vs_baseline"] = None
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
