#!/usr/bin/env python3
"""Benchmark of the fused gated activation on one MI355X.

One step = one pass of the whole path over one batch: the SwiGLU forward
y = silu(a) * b out of place, then the backward in place (da over a, db over
b), bf16, a, b, dy of shape (4096, 14336).  Inputs are seeded synthetic data
(a ~ N(0, 2^2), b, dy ~ N(0, 1), rounded to bf16), resident in HBM before the
timed region.  Several buffer sets are rotated so consecutive steps touch
disjoint memory (well over the last-level cache), i.e. the numbers are HBM
numbers, not cache numbers.

Metric: achieved HBM GB/s = algorithmic bytes / time, algorithmic bytes =
forward 3*N*2 + backward 5*N*2 = 939,524,096 B per step (N = 4096*14336).

Prints one JSON line (see the keys below).  `--gpus N` with N > 1 exits with
a message: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "achieved HBM GB/s (% of peak) for bf16 silu(a)*b fwd+bwd at 4096x14336"
PEAK_HBM_GBS = 8000.0
ROWS, COLS = 4096, 14336
N = ROWS * COLS
ES = 2
FWD_BYTES = 3 * N * ES          # read a, b; write y
BWD_BYTES = 5 * N * ES          # read a, b, dy; write da, db
STEP_BYTES = FWD_BYTES + BWD_BYTES
KERNEL_SOURCES = ["mlp_gated_activation_amd/csrc/glu_kernels.hip",
                  "mlp_gated_activation_amd/csrc/glu_act.h",
                  "mlp_gated_activation_amd/csrc/glu_internal.h",
                  "mlp_gated_activation_amd/csrc/glu_taylor.h",
                  "mlp_gated_activation_amd/csrc/glu_erfc.h"]
PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_glu_swiglu_bf16_4096x14336.md")
TILE_PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_glu_tile_swiglu_bf16_4096x14336_dyT.md")
GEMM_SOURCES = ["mlp_gated_activation_amd/csrc/gemm_kernels.hip",
                "mlp_gated_activation_amd/csrc/gemm_internal.h",
                "mlp_gated_activation_amd/csrc/glu_act.h",
                "mlp_gated_activation_amd/csrc/glu_internal.h",
                "mlp_gated_activation_amd/csrc/glu_taylor.h",
                "mlp_gated_activation_amd/csrc/glu_erfc.h"]
GEMM_PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_gemm_glu_swiglu_bf16_4096x4096x14336.md")
RMS_SOURCES = ["mlp_gated_activation_amd/csrc/rmsnorm_kernels.hip", "mlp_gated_activation_amd/csrc/rmsnorm_internal.h"]
RMS_PMC_SUMMARY = os.path.join(ROOT, "profiles", "pmc_add_rmsnorm_bf16_4096x{h}.md")


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for p in sources:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(path=PMC_SUMMARY, key="bwd_traffic_bytes", sources=KERNEL_SOURCES):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    try:
        text = open(path).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("source_hash") != kernel_source_hash(sources):
        return None
    return d.get(key)


def cpu_baseline(a, b, dy, bwd_only=False):
    """The fp64 oracle, as it stands, on the same inputs: fwd then bwd (or
    the bwd alone) over the whole (4096, 14336) batch.  The oracle sees the
    logical values, whatever layout the GPU operands have.

    fwd and bwd are timed separately on all the host's OpenMP threads (best
    of up to 5 runs within ~10 s) and once each on one thread; `value` is
    the all-thread rate of the timed work."""
    import torch
    import oracle
    fa = a.to(torch.float64).numpy()
    fb = b.to(torch.float64).numpy()
    fdy = dy.to(torch.float64).numpy()
    oracle.fwd("silu", fa[:8], fb[:8])          # load/compile outside the timing
    run_fwd = lambda: oracle.fwd("silu", fa, fb)
    run_bwd = lambda: oracle.bwd("silu", fa, fb, fdy)
    S = 512                                       # rows of the one-thread sample
    run1_fwd = lambda: oracle.fwd("silu", fa[:S], fb[:S])
    run1_bwd = lambda: oracle.bwd("silu", fa[:S], fb[:S], fdy[:S])

    def best(fn, budget_s):
        times = []
        t_all = time.perf_counter()
        while True:
            t0 = time.perf_counter()
            fn()
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_all > budget_s or len(times) >= 5:
                return min(times), len(times)

    threads = oracle.num_threads()
    t_fwd, n_fwd = (None, 0) if bwd_only else best(run_fwd, 5.0)
    t_bwd, n_bwd = best(run_bwd, 5.0)
    oracle.set_num_threads(1)
    try:
        t1_fwd = None if bwd_only else best(run1_fwd, 0.0)[0] * ROWS / S
        t1_bwd = best(run1_bwd, 0.0)[0] * ROWS / S
    finally:
        oracle.set_num_threads(threads)
    del fa, fb, fdy
    gbs = lambda nbytes, t: None if t is None else round(nbytes / t / 1e9, 3)
    t_all_threads = t_bwd if bwd_only else t_fwd + t_bwd
    what = "bwd" if bwd_only else "fwd+bwd"
    return {
        "value": gbs(BWD_BYTES if bwd_only else STEP_BYTES, t_all_threads),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"full workload, {what} over {ROWS}x{COLS} (fp64 scalar C, OpenMP), fwd and bwd each "
                  f"best of {max(n_fwd, n_bwd)}; the one-thread figures from the first {S} rows, once",
        "elements_per_s": round(N / t_all_threads, 1),
        "seconds_per_step": round(t_all_threads, 4),
        "by_pass": {
            "all_threads": {"threads": threads, "fwd_GBps": gbs(FWD_BYTES, t_fwd), "bwd_GBps": gbs(BWD_BYTES, t_bwd)},
            "one_thread": {"threads": 1, "fwd_GBps": gbs(FWD_BYTES, t1_fwd), "bwd_GBps": gbs(BWD_BYTES, t1_bwd)},
        },
    }


def event_ms(torch, stream, fn, n, warmup=0):
    """Average milliseconds per call of fn(0) .. fn(n - 1), launched back to
    back and bracketed by HIP events recorded on `stream`, the stream the
    library launches on (torch.cuda.Event on another stream would not see
    them); `warmup` untimed calls go first."""
    for i in range(warmup):
        fn(i)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(n):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def batched_ms(torch, stream, fn, n, batch, restore):
    """Total milliseconds of fn(0) .. fn(n - 1), timed in batches of `batch`
    back-to-back calls, each batch bracketed by HIP events on `stream`.
    restore() runs after every batch, outside the timed intervals: it puts
    back the inputs an in-place call overwrote, so every timed call reads the
    stated input values."""
    pairs = []
    torch.cuda.synchronize()
    for s0 in range(0, n, batch):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(s0, min(n, s0 + batch)):
            fn(i)
        e1.record(stream)
        restore()
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    return sum(e0.elapsed_time(e1) for e0, e1 in pairs)


def attainable(torch, stream, sets, n, restore):
    """Same-run ceilings: the data-movement reference kernels (the streaming
    kernels' access pattern and launch shape, no arithmetic) over the same
    rotating buffer sets, average ms per launch of the forward's 2:1 mix,
    the backward's 3:2 mix (in place, like the backward) and a plain copy."""
    from mlp_gated_activation_amd import stream_ref

    def fwd_mix(i):
        a, b, dy, y = sets[i % len(sets)]
        stream_ref.fwd_mix(a, b, y)

    def bwd_mix(i):
        a, b, dy, y = sets[i % len(sets)]
        stream_ref.bwd_mix(a, b, dy, a, b)

    def copy(i):
        a, b, dy, y = sets[i % len(sets)]
        stream_ref.copy(a, y)

    for i in range(len(sets)):
        fwd_mix(i)
        bwd_mix(i)
        copy(i)
    t_f = event_ms(torch, stream, fwd_mix, n)
    t_b = event_ms(torch, stream, bwd_mix, n)
    t_c = event_ms(torch, stream, copy, n)
    restore()
    torch.cuda.synchronize()
    return t_f, t_b, t_c


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--op", choices=["glu", "add_rmsnorm", "glu_strided", "gemm_glu", "providers", "mlp", "configs"],
                    default="glu",
                    help="glu: the SwiGLU fwd+bwd step (default); add_rmsnorm: the fused residual "
                         "add + RMSNorm forward, bf16, 4096 rows; glu_strided: the SwiGLU backward "
                         "with a transposed incoming gradient (LDS-tiled kernel) and related layouts; "
                         "gemm_glu: the gate/up projection with the activation fused into its epilogue "
                         "(bf16, 4096 tokens, hidden 4096, I 14336); providers: the SwiGLU op at "
                         "4096 x H, H = 1024 .. 16384, against torch eager and torch.compile; mlp: a whole "
                         "SwiGLU MLP training step (4096 tokens, 4096 -> 14336, bf16), GatedMLP against the "
                         "same network in torch, time and peak memory; configs: every workload configuration "
                         "and kind, forward and backward per kernel")
    ap.add_argument("--hidden", type=int, default=4096, help="add_rmsnorm only: row width")
    ap.add_argument("--gemm-shapes", action="store_true",
                    help="gemm_glu only: also time the fused and unfused paths at 1 .. 256 tokens over other "
                         "MLP shapes (hidden x intermediate), with the choice GatedMLP's default makes")
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--sets", type=int, default=6, help="rotating buffer sets (470 MB each)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-torch-eager", dest="torch_eager", action="store_false",
                    help="skip the torch eager comparison")
    ap.add_argument("--torch-compile", action="store_true",
                    help="also time torch.compile of the same step (context; compiles on first use)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported. The op shards with no communication (rows or matched column slices), "
              "so one GPU's throughput is the per-GPU figure.", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    from mlp_gated_activation_amd import build as _build
    if not os.path.exists(_build.LIB) or not os.path.exists(_build.REF_LIB):
        _build.build()
    from mlp_gated_activation_amd import glu, inputs

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.op == "add_rmsnorm":
        return bench_add_rmsnorm(args, torch, glu, inputs, dev)
    if args.op == "glu_strided":
        return bench_strided(args, torch, glu, inputs, dev)
    if args.op == "gemm_glu":
        return bench_gemm(args, torch, glu, inputs, dev)
    if args.op == "providers":
        return bench_providers(args, torch, glu, inputs, dev)
    if args.op == "mlp":
        return bench_mlp(args, torch, dev)
    if args.op == "configs":
        return bench_configs(args, torch, glu, inputs, dev)
    w = inputs.WORKLOADS["swiglu_bf16_4096x14336"]
    a_h, b_h, dy_h = w.make(seed=0)
    # pristine device copies of the operands the in-place backward overwrites
    a_p, b_p = a_h.to(dev), b_h.to(dev)
    sets = []
    for _ in range(args.sets):
        sets.append([a_p.clone(), b_p.clone(), dy_h.to(dev), torch.empty(ROWS, COLS, dtype=torch.bfloat16, device=dev)])
    stream = torch.cuda.current_stream(dev)

    def restore():
        for s_ in sets:
            s_[0].copy_(a_p)
            s_[1].copy_(b_p)

    def step(i):
        a, b, dy, y = sets[i % len(sets)]
        glu.glu_fwd("silu", "separate", a, b, y)
        glu.glu_bwd("silu", "separate", a, b, dy, inplace=True)

    nb = len(sets)
    for i in range(args.warmup):
        step(i)
        if i % nb == nb - 1:
            restore()
    restore()
    torch.cuda.synchronize()

    # Headline: K whole steps in batches of one pass over the buffer sets;
    # each batch is timed between HIP events with nothing else between its
    # launches, and the in-place inputs are restored between batches.
    wall0 = time.perf_counter()
    total_ms = batched_ms(torch, stream, step, args.steps, nb, restore)
    wall = time.perf_counter() - wall0
    ms_per_step = total_ms / args.steps
    value = STEP_BYTES / (ms_per_step * 1e-3) / 1e9

    # Per-kernel average launch durations: K launches of each kernel alone
    # (rotating buffer sets, so every launch streams cold memory).
    def fwd_only(i):
        a, b, dy, y = sets[i % len(sets)]
        glu.glu_fwd("silu", "separate", a, b, y)

    def bwd_only(i):
        a, b, dy, y = sets[i % len(sets)]
        glu.glu_bwd("silu", "separate", a, b, dy, inplace=True)

    fwd_avg = batched_ms(torch, stream, fwd_only, args.steps, nb, lambda: None) / args.steps
    bwd_avg = batched_ms(torch, stream, bwd_only, args.steps, nb, restore) / args.steps

    # Warm (context for the cold headline): every step on the same buffer
    # set, restored before each step; the restore's writes and the previous
    # step's are what the last-level cache holds when a step starts.
    warm_n = min(args.steps, 200)
    warm_ms = batched_ms(torch, stream, lambda i: step(0), warm_n, 1, restore) / warm_n

    # Same-run ceilings from the data-movement reference kernels.
    ref_f, ref_b, ref_c = attainable(torch, stream, sets, min(args.steps, 300), restore)

    def timed(fn, n):
        """Total milliseconds of n calls of fn(i) that leave the inputs intact."""
        return batched_ms(torch, stream, fn, n, nb, lambda: None)

    # Context: the same step in plain torch eager (silu then multiply, and
    # autograd for the gradients), timed the same way.
    eager = None
    if args.torch_eager:
        import torch.nn.functional as F
        reps = min(args.steps, 100)

        def eager_fwd(i):
            a, b, dy, y = sets[i % len(sets)]
            F.silu(a) * b

        def eager_step(i):
            a, b, dy, y = sets[i % len(sets)]
            a_ = a.detach().requires_grad_()
            b_ = b.detach().requires_grad_()
            (F.silu(a_) * b_).backward(dy)

        for i in range(5):
            eager_step(i)
        t_ef = timed(eager_fwd, reps) / reps
        t_es = timed(eager_step, reps) / reps
        eager = {"fwd_us": round(1e3 * t_ef, 2), "fwd_GBps": round(FWD_BYTES / (t_ef * 1e-3) / 1e9, 1),
                 "step_us": round(1e3 * t_es, 2), "step_GBps": round(STEP_BYTES / (t_es * 1e-3) / 1e9, 1),
                 "speedup_step": round(t_es / ms_per_step, 2),
                 "note": "F.silu(a) * b and autograd, bf16, same buffers; algorithmic bytes / time"}

    # Context: torch.compile of the same step, the other comparison provider
    # the pages name ("Write a Triton SiLU-Mul (SwiGLU) Kernel", Performance
    # requirements: a custom kernel should beat it clearly).  Opt-in: it
    # compiles on first use.
    compiled = None
    if args.torch_compile:
        import torch.nn.functional as F
        try:
            reps = min(args.steps, 100)
            cfwd = torch.compile(lambda a, b: F.silu(a) * b, dynamic=False)

            def comp_fwd(i):
                a, b, dy, y = sets[i % len(sets)]
                cfwd(a, b)

            def comp_step(i):
                a, b, dy, y = sets[i % len(sets)]
                a_ = a.detach().requires_grad_()
                b_ = b.detach().requires_grad_()
                cfwd(a_, b_).backward(dy)

            t0 = time.perf_counter()
            for i in range(5):
                comp_fwd(i)
                comp_step(i)
            torch.cuda.synchronize()
            t_compile = time.perf_counter() - t0
            t_cf = timed(comp_fwd, reps) / reps
            t_cs = timed(comp_step, reps) / reps
            compiled = {"fwd_us": round(1e3 * t_cf, 2), "fwd_GBps": round(FWD_BYTES / (t_cf * 1e-3) / 1e9, 1),
                        "step_us": round(1e3 * t_cs, 2), "step_GBps": round(STEP_BYTES / (t_cs * 1e-3) / 1e9, 1),
                        "speedup_step": round(t_cs / ms_per_step, 2), "first_calls_s": round(t_compile, 1),
                        "note": "torch.compile(F.silu(a) * b), forward and autograd backward, bf16, same buffers"}
        except Exception as e:   # context only: report, do not fail the benchmark
            compiled = {"error": f"{type(e).__name__}: {e}"[:300]}

    achieved = BWD_BYTES / (bwd_avg * 1e-3) / 1e9
    gbs = lambda nbytes, ms: round(nbytes / (ms * 1e-3) / 1e9, 1)
    attain_step = STEP_BYTES / ((ref_f + ref_b) * 1e-3) / 1e9
    traffic = committed_traffic()
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded a~N(0,4), b,dy~N(0,1) rounded to bf16; "
                f"{args.sets} rotating buffer sets, {args.sets * 4 * N * ES / 1e9:.2f} GB; a, b restored "
                "from a pristine device copy after every batch of one pass over the sets, untimed, so "
                "every timed step reads these values)",
        "config": {
            "workload": "SwiGLU bf16 separate a,b,dy (4096, 14336): fwd out-of-place + bwd in place",
            "rows": ROWS, "cols": COLS, "kind": "silu", "layout": "separate",
            "bytes_per_step": STEP_BYTES, "math": "fp32 in registers, one RNE rounding per output",
        },
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "pct_of_attainable": round(100 * value / attain_step, 2),
        "attainable": {
            "step_GBps": round(attain_step, 1),
            "fwd_mix": {"avg_us": round(1e3 * ref_f, 2), "GBps": gbs(FWD_BYTES, ref_f)},
            "bwd_mix": {"avg_us": round(1e3 * ref_b, 2), "GBps": gbs(BWD_BYTES, ref_b)},
            "copy_GBps": gbs(2 * N * ES, ref_c),
            "note": "data-movement reference kernels (libglu_ref.so) in this run on the same buffer sets: "
                    "the forward's 2:1 and the backward's 3:2 read:write mix with the streaming kernels' "
                    "access pattern and launch shape and no arithmetic; step = both mixes",
        },
        "kernels": {
            "fwd": {"avg_us": round(1e3 * fwd_avg, 2), "GBps": gbs(FWD_BYTES, fwd_avg), "bytes": FWD_BYTES,
                    "pct_of_mix": round(100 * ref_f / fwd_avg, 2)},
            "bwd": {"avg_us": round(1e3 * bwd_avg, 2), "GBps": round(achieved, 1), "bytes": BWD_BYTES,
                    "pct_of_mix": round(100 * ref_b / bwd_avg, 2)},
        },
        "warm": {"ms_per_step": round(warm_ms, 5), "GBps": round(STEP_BYTES / (warm_ms * 1e-3) / 1e9, 1),
                 "note": "the same buffer set every step, restored before each"},
        "torch_eager": eager,
        "torch_compile": compiled,
        "wall_s_timed": round(wall, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": "glu_kernel<bf16, silu, bwd, vec, flat>",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": None,
    }
    del sets
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(a_h, b_h, dy_h)
    print(json.dumps(result), flush=True)


def bench_providers(args, torch, glu, inputs, dev):
    """The SwiGLU op over the pages' benchmark sweep ("Kernel Profile: SwiGLU",
    Benchmarking: hidden size 1024 .. 16384, 4096 rows, bf16; providers this
    library, torch eager and torch.compile), forward and full (forward then
    backward), plus H = 1792, one rank's share of the 14336-wide activation
    under 8-way tensor parallelism.  Every provider is launched call by call
    from Python, as a training loop would; for this library a HIP graph of
    the same calls is timed as well.  Buffer sets rotate over at least 1 GiB, so every call
    streams from HBM.  Context only: the headline is the default op."""
    import torch.nn.functional as F
    stream = torch.cuda.current_stream(dev)
    reps = min(args.steps, 200)

    restore = lambda: None

    def timed(fn, n, batch=None):
        """Average ms per call; in-place inputs restored between batches."""
        return batched_ms(torch, stream, fn, n, batch or nsets, restore) / n

    rows_out = []
    compile_error = None
    sweep = [(h, f"swiglu_bf16_4096x{h}") for h in (1024, 2048, 4096, 8192, 16384)]
    sweep.insert(1, (1792, "swiglu_bf16_tp8_4096x1792"))     # one TP = 8 rank's share of 14336
    for h, wname in sweep:
        # a fresh compilation per size: the guard cache of one compiled
        # function would otherwise fill up and fall back to eager silently
        try:
            torch._dynamo.reset()
            cfwd = torch.compile(lambda a, b: F.silu(a) * b, dynamic=False)
        except Exception as e:   # context only
            cfwd, compile_error = None, f"{type(e).__name__}: {e}"[:300]
        w = inputs.WORKLOADS[wname]
        a_h, b_h, dy_h = w.make(seed=0)
        n = a_h.numel()
        nsets = max(2, -(-(1 << 30) // (4 * n * 2)))
        a_p, b_p = a_h.to(dev), b_h.to(dev)     # pristine copies for the in-place backward
        sets = [[a_p.clone(), b_p.clone(), dy_h.to(dev), torch.empty_like(a_h, device=dev)] for _ in range(nsets)]

        def restore():
            for s_ in sets:
                s_[0].copy_(a_p)
                s_[1].copy_(b_p)
        fwd_bytes, step_bytes = 3 * n * 2, 8 * n * 2

        def ours_fwd(i):
            a, b, dy, y = sets[i % nsets]
            glu.glu_fwd("silu", "separate", a, b, y)

        def ours_step(i):
            a, b, dy, y = sets[i % nsets]
            glu.glu_fwd("silu", "separate", a, b, y)
            glu.glu_bwd("silu", "separate", a, b, dy, inplace=True)

        def eager_fwd(i):
            a, b, dy, y = sets[i % nsets]
            F.silu(a) * b

        def eager_step(i):
            a, b, dy, y = sets[i % nsets]
            a_ = a.detach().requires_grad_()
            b_ = b.detach().requires_grad_()
            (F.silu(a_) * b_).backward(dy)

        def comp_fwd(i):
            a, b, dy, y = sets[i % nsets]
            cfwd(a, b)

        def comp_step(i):
            a, b, dy, y = sets[i % nsets]
            a_ = a.detach().requires_grad_()
            b_ = b.detach().requires_grad_()
            cfwd(a_, b_).backward(dy)

        def graph_of(fn):
            """A HIP graph of one call per buffer set; returns the time per call."""
            fn(0)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(nsets):
                    fn(i)
            g.replay()
            restore()
            torch.cuda.synchronize()
            r = max(1, reps // nsets)
            return timed(lambda i: g.replay(), r, batch=1) / nsets

        row = {"H": h, "workload": wname, "bytes_fwd": fwd_bytes, "bytes_full": step_bytes}
        legs = [("ours", ours_fwd, ours_step), ("torch", eager_fwd, eager_step)]
        if cfwd is not None:
            legs.append(("torch_compile", comp_fwd, comp_step))
        for name, f_fwd, f_step in legs:
            try:
                for i in range(5):
                    f_fwd(i)
                    f_step(i)
                restore()
                t_f, t_s = timed(f_fwd, reps), timed(f_step, reps)
                row[name] = {"fwd_us": round(1e3 * t_f, 2), "full_us": round(1e3 * t_s, 2),
                             "fwd_GBps": round(fwd_bytes / (t_f * 1e-3) / 1e9, 1),
                             "full_GBps": round(step_bytes / (t_s * 1e-3) / 1e9, 1)}
            except Exception as e:   # context only: report, do not fail the sweep
                row[name] = {"error": f"{type(e).__name__}: {e}"[:300]}
        t_f, t_s = graph_of(ours_fwd), graph_of(ours_step)
        row["ours_hip_graph"] = {"fwd_us": round(1e3 * t_f, 2), "full_us": round(1e3 * t_s, 2),
                                 "fwd_GBps": round(fwd_bytes / (t_f * 1e-3) / 1e9, 1),
                                 "full_GBps": round(step_bytes / (t_s * 1e-3) / 1e9, 1)}
        rows_out.append(row)
        print(f"providers: H={h} done", file=sys.stderr, flush=True)
        del sets
        torch.cuda.empty_cache()
    top = rows_out[-1]
    result = {
        "metric": "achieved HBM GB/s, SwiGLU fwd+bwd, bf16, 4096 x H (providers sweep)",
        "value": top["ours"].get("full_GBps"),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": reps,
        "warmup": 5,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded a~N(0,4), b,dy~N(0,1) rounded to bf16; >= 1 GiB of rotating buffer sets; "
                "a, b restored from a pristine device copy between timed batches, untimed)",
        "config": {"workload": "SwiGLU bf16 separate a,b,dy (4096, H), H = 1024 .. 16384 and 1792 (one "
                               "TP = 8 rank's share of 14336); value at H = 16384",
                   "providers": ["ours", "torch", "torch_compile", "ours_hip_graph"]},
        "sweep": rows_out,
        # context only: the headline op carries the oracle's CPU timing
        "cpu_baseline": None,
    }
    if compile_error is not None:
        result["torch_compile_error"] = compile_error
    print(json.dumps(result), flush=True)


def bench_configs(args, torch, glu, inputs, dev):
    """Every workload configuration, forward and backward per kernel through
    the binding: the metric shape with all four kinds, the 11008-wide and
    [gate | up] bf16 workloads, the hidden-size sweep and one TP = 8 rank's
    share, the fp16 [gate | up] workload with rare large gate values for all
    four kinds, and fp32 data (64 x 1024, and 4096 x 14336 with all four
    kinds).  Every kernel is warmed up for at least 40 launches, then timed
    over `--steps` (at most 60) launches rotating over at least 1.5 GB of
    sets; the in-place backward's inputs are restored from pristine copies
    between timed batches.  Calls go one by one through the binding, so the
    smallest shapes (a few microseconds per call) show host-bound figures;
    the providers op times them against HIP-graph replay.  Context: the
    headline is the default op."""
    stream = torch.cuda.current_stream(dev)
    reps = max(1, min(args.steps, 60))
    nothing = lambda: None
    out = []

    def time_kinds(name, layout, kinds, host):
        """host: (a, b, dy) for separate, (x, dy) for gate_up, on the CPU."""
        pristine = [t.to(dev) for t in host]
        es = pristine[0].element_size()
        R, C = pristine[-1].shape                      # dy is (rows, cols) in both layouts
        nsets = max(2, -(-int(1.5e9) // (4 * R * C * es)))
        sets = [[t.clone() for t in pristine] + [torch.empty(R, C, dtype=pristine[0].dtype, device=dev)]
                for _ in range(nsets)]
        nin = 2 if layout == "separate" else 1      # tensors the in-place backward overwrites

        def restore():
            for s_ in sets:
                for j in range(nin):
                    s_[j].copy_(pristine[j])
        for kind in kinds:
            if layout == "separate":
                fwd = lambda i: glu.glu_fwd(kind, "separate", sets[i % nsets][0], sets[i % nsets][1],
                                            sets[i % nsets][3])
                bwd = lambda i: glu.glu_bwd(kind, "separate", sets[i % nsets][0], sets[i % nsets][1],
                                            sets[i % nsets][2], inplace=True)
            else:
                fwd = lambda i: glu.glu_fwd(kind, "gate_up", sets[i % nsets][0], y=sets[i % nsets][2])
                bwd = lambda i: glu.glu_bwd(kind, "gate_up", sets[i % nsets][0], None, sets[i % nsets][1],
                                            inplace=True)
            # warm-up: the clock settles to each kernel's load within tens of launches
            warm = max(nsets, 40)
            batched_ms(torch, stream, fwd, warm, nsets, nothing)
            batched_ms(torch, stream, bwd, warm, nsets, restore)
            t_f = batched_ms(torch, stream, fwd, reps, nsets, nothing) / reps
            t_b = batched_ms(torch, stream, bwd, reps, nsets, restore) / reps
            fb, bb = 3 * R * C * es, 5 * R * C * es
            out.append({"workload": name, "kind": kind, "dtype": str(pristine[0].dtype).replace("torch.", ""),
                        "layout": layout, "rows": R, "cols": C,
                        "fwd_us": round(1e3 * t_f, 2), "fwd_GBps": round(fb / (t_f * 1e-3) / 1e9, 1),
                        "bwd_us": round(1e3 * t_b, 2), "bwd_GBps": round(bb / (t_b * 1e-3) / 1e9, 1),
                        "step_GBps": round((fb + bb) / ((t_f + t_b) * 1e-3) / 1e9, 1)})
        del sets, pristine
        torch.cuda.empty_cache()
        print(f"configs: {name} done", file=sys.stderr, flush=True)

    kinds4 = ["silu", "gelu_erf", "gelu_tanh", "relu"]
    W = inputs.WORKLOADS
    time_kinds("swiglu_bf16_4096x14336", "separate", kinds4, W["swiglu_bf16_4096x14336"].make(seed=0))
    time_kinds("swiglu_bf16_4096x11008", "separate", ["silu"], W["swiglu_bf16_4096x11008"].make(seed=0))
    time_kinds("swiglu_bf16_gateup_4096x14336", "gate_up", ["silu"], W["swiglu_bf16_gateup_4096x14336"].make(seed=0))
    for name in [f"swiglu_bf16_4096x{h}" for h in (1024, 2048, 4096, 8192, 16384)] + ["swiglu_bf16_tp8_4096x1792"]:
        time_kinds(name, "separate", ["silu"], W[name].make(seed=0))
    time_kinds("geglu_reglu_fp16_gateup_8191x18944", "gate_up", kinds4,
               W["geglu_reglu_fp16_gateup_8191x18944"].make(seed=0))
    time_kinds("swiglu_f32_64x1024", "separate", ["silu"], W["swiglu_f32_64x1024"].make(seed=0))
    time_kinds("fp32 4096x14336", "separate", kinds4, inputs.separate(4096, 14336, "fp32", 2.0, seed=0))
    head = [r for r in out if r["workload"] == "swiglu_bf16_4096x14336" and r["kind"] == "silu"][0]
    result = {
        "metric": "achieved HBM GB/s per configuration, forward and backward per kernel (context)",
        "value": head["step_GBps"], "unit": "GB/s", "n_gpus": 1, "steps": reps, "warmup": 1,
        "ms_per_step": round((head["fwd_us"] + head["bwd_us"]) * 1e-3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 (value); every dtype in rows",
        "data": "synthetic, the seeded workloads of mlp_gated_activation_amd.inputs; >= 1.5 GB of rotating "
                "buffer sets per configuration; in-place inputs restored between timed batches",
        "config": {"workload": "every configuration; value: SwiGLU bf16 (4096, 14336) fwd + bwd per kernel"},
        "rows": out,
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


def bench_mlp(args, torch, dev):
    """A whole SwiGLU MLP training step, down(silu(gate(x)) * up(x)) forward
    and backward, 4096 tokens, hidden 4096, intermediate 14336, bf16:
    GatedMLP (torch GEMMs around this library's activation kernels, in-place
    backward) against the same network in plain torch with the same weights,
    and optionally under torch.compile.  Time per step and the peak memory a
    step allocates beyond its inputs and weights ("Kernel Profile: SwiGLU",
    Key Patterns: the in-place backward saves an allocation).  Context for
    the op-level figures: the GEMMs dominate the step."""
    import torch.nn.functional as F
    from mlp_gated_activation_amd.functional import GatedMLP
    tokens, hidden, inter = 4096, 4096, 14336
    torch.manual_seed(0)
    ours = GatedMLP(hidden, inter, device=dev, dtype=torch.bfloat16)
    wg = ours.gate_up_proj.weight[:inter].detach()
    wu = ours.gate_up_proj.weight[inter:].detach()
    wd = ours.down_proj.weight.detach()

    class TorchMLP(torch.nn.Module):
        def __init__(self):
            super().__init__()
            self.gate_proj = torch.nn.Linear(hidden, inter, bias=False, device=dev, dtype=torch.bfloat16)
            self.up_proj = torch.nn.Linear(hidden, inter, bias=False, device=dev, dtype=torch.bfloat16)
            self.down_proj = torch.nn.Linear(inter, hidden, bias=False, device=dev, dtype=torch.bfloat16)

        def forward(self, x):
            return self.down_proj(F.silu(self.gate_proj(x)) * self.up_proj(x))

    ref = TorchMLP()
    with torch.no_grad():
        ref.gate_proj.weight.copy_(wg)
        ref.up_proj.weight.copy_(wu)
        ref.down_proj.weight.copy_(wd)
    x = torch.randn(tokens, hidden, device=dev, dtype=torch.bfloat16)
    dy = torch.randn(tokens, hidden, device=dev, dtype=torch.bfloat16)
    stream = torch.cuda.current_stream(dev)
    steps = min(args.steps, 50)

    def measure(module):
        params = list(module.parameters())

        def step(i):
            for q in params:
                q.grad = None
            xi = x.detach().requires_grad_()
            module(xi).backward(dy)

        for i in range(3):
            step(i)
        # peak of one step beyond inputs and weights: activations kept for the
        # backward, temporaries and the weight gradients it allocates
        for q in params:
            q.grad = None
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        xi = x.detach().requires_grad_()
        out = module(xi)
        torch.cuda.synchronize()
        # what the layer keeps between its forward and its backward (with
        # its output): the part that adds up over the layers of a model
        kept = torch.cuda.memory_allocated(dev) - base
        out.backward(dy)
        del out, xi
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated(dev) - base
        ms = event_ms(torch, stream, step, steps)
        return {"ms_per_step": round(ms, 4), "kept_for_backward_MB": round(kept / 2**20, 1),
                "peak_step_MB": round(peak / 2**20, 1)}

    result_ours = measure(ours)
    rec = GatedMLP(hidden, inter, recompute_activation=True, device=dev, dtype=torch.bfloat16)
    rec.load_state_dict(ours.state_dict())
    result_recompute = measure(rec)
    del rec
    result_torch = measure(ref)
    compiled = None
    if args.torch_compile:
        try:
            compiled = measure(torch.compile(ref))
        except Exception as e:   # context only
            compiled = {"error": f"{type(e).__name__}: {e}"[:300]}
    flops = 3 * 2 * tokens * hidden * inter * 3   # three GEMMs, forward and two per GEMM backward
    result = {
        "metric": "SwiGLU MLP training step time, bf16, 4096 tokens, 4096 -> 14336 -> 4096",
        "value": result_ours["ms_per_step"], "unit": "ms", "n_gpus": 1, "steps": steps, "warmup": 3,
        "ms_per_step": result_ours["ms_per_step"], "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded randn inputs and gradients; nn.Linear default initialisation)",
        "config": {"workload": "GatedMLP fwd+bwd vs the same network in torch", "tokens": tokens,
                   "hidden": hidden, "intermediate": inter, "matmul_TFLOP_per_step": round(flops / 1e12, 3)},
        "ours": result_ours, "ours_recompute_activation": result_recompute,
        "torch": result_torch, "torch_compile": compiled,
        "speedup_vs_torch": round(result_torch["ms_per_step"] / result_ours["ms_per_step"], 3),
        # the oracle covers the activation step, not a whole network's GEMMs
        "cpu_baseline": None,
        "peak_memory_saved_MB": round(result_torch["peak_step_MB"] - result_ours["peak_step_MB"], 1),
    }
    print(json.dumps(result), flush=True)


def bench_add_rmsnorm(args, torch, glu, inputs, dev):
    """The fused residual add + RMSNorm forward ("Write a Triton Fused
    Add+RMSNorm Kernel"): bf16 x, residual (4096, H), gamma (H,), eps 1e-6;
    h and y written out of place, rstd not saved (the inference step).
    Algorithmic bytes: read x, residual, write h, y = 4*R*H*2, plus gamma once."""
    R, H = 4096, args.hidden
    step_bytes = 4 * R * H * 2 + H * 2
    x_h, r_h, g_h = inputs.add_rmsnorm(R, H, "bf16", seed=0)
    nsets = max(4, -(-2_000_000_000 // (4 * R * H * 2)))
    sets = [[x_h.to(dev), r_h.to(dev), torch.empty(R, H, dtype=torch.bfloat16, device=dev),
             torch.empty(R, H, dtype=torch.bfloat16, device=dev)] for _ in range(nsets)]
    gamma = g_h.to(dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        x, r, h, y = sets[i % nsets]
        glu.glu_add_rmsnorm_fwd(x, r, gamma, 1e-6, h=h, y=y)

    ms = event_ms(torch, stream, step, args.steps, warmup=args.warmup)
    value = step_bytes / (ms * 1e-3) / 1e9

    # same-run ceiling: the data-movement reference kernel of this traffic
    from mlp_gated_activation_amd import stream_ref

    def ref_step(i):
        x, r, h, y = sets[i % nsets]
        stream_ref.rms_mix(x, r, h, y)

    ms_ref = event_ms(torch, stream, ref_step, min(args.steps, 300), warmup=5)
    attain = 4 * R * H * 2 / (ms_ref * 1e-3) / 1e9

    eager = None
    if args.torch_eager:
        import torch.nn.functional as F
        reps = min(args.steps, 100)
        def eager_step(i):
            x, r, h, y = sets[i % nsets]
            F.rms_norm(x + r, (H,), weight=gamma, eps=1e-6)

        te = event_ms(torch, stream, eager_step, reps, warmup=5)   # first calls pay one-time costs
        eager = {"us": round(1e3 * te, 2), "GBps": round(step_bytes / (te * 1e-3) / 1e9, 1),
                 "speedup": round(te / ms, 2), "note": "x + residual, then F.rms_norm, bf16; algorithmic bytes / time"}

    src = [p for p in RMS_SOURCES]
    traffic = committed_traffic(RMS_PMC_SUMMARY.format(h=H), "traffic_bytes", src)
    result = {
        "metric": f"achieved HBM GB/s (% of peak) for bf16 fused residual add + RMSNorm fwd at 4096x{H}",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": f"synthetic (seeded x, residual ~ N(0,1), gamma ~ 1 + 0.1 N(0,1), bf16; {nsets} rotating sets)",
        "config": {"workload": f"fused residual add + RMSNorm forward, bf16 (4096, {H}), eps 1e-6, h and y out of place",
                   "rows": R, "hidden": H, "bytes_per_step": step_bytes,
                   "math": "fp32 sum and statistics in registers, one RNE rounding per output"},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "pct_of_attainable": round(100 * value / attain, 2),
        "attainable": {"GBps": round(attain, 1), "avg_us": round(1e3 * ms_ref, 2),
                       "note": "data-movement reference kernel (libglu_ref.so) in this run on the same buffers: "
                               "read x and residual, write h and y, flat 16-byte non-temporal streams, no arithmetic"},
        "torch_eager": eager,
        "roofline": {"bound": "hbm", "kernel": "add_rmsnorm_kernel or add_rmsnorm_rows_kernel <bf16> (by width)",
                     "achieved": round(value, 1),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(value / PEAK_HBM_GBS, 4),
                     "traffic": traffic},
        "cpu_baseline": None,
    }
    del sets
    if not args.no_cpu_baseline:
        import oracle
        fx, fr, fg = (t.to(torch.float64).numpy() for t in (x_h, r_h, g_h))
        oracle.add_rmsnorm(fx[:8], fr[:8], fg, 1e-6)
        times = []
        t_all = time.perf_counter()
        while len(times) < 5 and time.perf_counter() - t_all < 10.0:
            t0 = time.perf_counter()
            oracle.add_rmsnorm(fx, fr, fg, 1e-6)
            times.append(time.perf_counter() - t0)
        best = min(times)
        result["cpu_baseline"] = {"value": round(step_bytes / best / 1e9, 3), "unit": "GB/s",
                                  "cores": oracle.num_threads(), "kind": "oracle",
                                  "sample": f"full workload (4096x{H}, fp64 scalar C, OpenMP), best of {len(times)}",
                                  "seconds_per_step": round(best, 4)}
    print(json.dumps(result), flush=True)


def bench_strided(args, torch, glu, inputs, dev):
    """SwiGLU bf16 (4096, 14336) on strided views, no .contiguous() copies:
      * bwd_dyT: backward in place with dy a transposed view (column-major)
        while a, b are row-major: the LDS-tiled kernel (the headline here);
      * fwd_yT: forward into a transposed output: the LDS-tiled kernel;
      * all_T: forward + backward with every operand transposed: the
        streaming kernels on the transposed problem;
      * copy_then_bwd: what a caller without strided support does,
        dy.contiguous() then the row-major backward.
    Algorithmic bytes as in the main step (fwd 3*N*2, bwd 5*N*2)."""
    w = inputs.WORKLOADS["swiglu_bf16_4096x14336"]
    a_h, b_h, dy_h = w.make(seed=0)
    dyT_h = dy_h.t().contiguous()
    a_p, b_p = a_h.to(dev), b_h.to(dev)     # pristine copies for the in-place calls
    sets = []
    for _ in range(args.sets):
        sets.append([a_p.clone(), b_p.clone(), dyT_h.to(dev).t(),
                     torch.empty(COLS, ROWS, dtype=torch.bfloat16, device=dev).t()])
    stream = torch.cuda.current_stream(dev)
    nb = len(sets)

    def restore():
        for s_ in sets:
            s_[0].copy_(a_p)
            s_[1].copy_(b_p)

    def timed(fn, n):
        """Average ms per call; in-place inputs restored between batches."""
        for i in range(min(n, args.warmup)):
            fn(i)
        restore()
        return batched_ms(torch, stream, fn, n, nb, restore) / n

    def bwd_dyT(i):
        a, b, dyT, yT = sets[i % len(sets)]
        glu.glu_bwd_strided("silu", a, b, dyT, da=a, db=b)

    def fwd_yT(i):
        a, b, dyT, yT = sets[i % len(sets)]
        glu.glu_fwd_strided("silu", a, b, yT)

    def copy_then_bwd(i):
        a, b, dyT, yT = sets[i % len(sets)]
        glu.glu_bwd("silu", "separate", a, b, dyT.contiguous(), inplace=True)

    t_bwd = timed(bwd_dyT, args.steps)
    t_fwd = timed(fwd_yT, args.steps)
    t_copy = timed(copy_then_bwd, min(args.steps, 200))
    # every operand transposed: reuse the buffers as (COLS, ROWS) matrices seen transposed
    tsets = [[s_[0].view(COLS, ROWS).t(), s_[1].view(COLS, ROWS).t(), s_[2], s_[3]] for s_ in sets]

    def all_T(i):
        aT, bT, dyT, yT = tsets[i % len(tsets)]
        glu.glu_fwd_strided("silu", aT, bT, yT)
        glu.glu_bwd_strided("silu", aT, bT, dyT, da=aT, db=bT)

    t_allT = timed(all_T, args.steps)
    # same-run ceilings: the tiled kernel's own access pattern without
    # arithmetic, and (context) the row-major streams on the same storage
    from mlp_gated_activation_amd import stream_ref

    def tile_bwd_ref(i):
        a, b, dyT, yT = sets[i % len(sets)]
        stream_ref.tile_bwd_mix(a, b, dyT.t(), a, b)

    def tile_fwd_ref(i):
        a, b, dyT, yT = sets[i % len(sets)]
        stream_ref.tile_fwd_mix(a, b, yT.t())

    n_ref = min(args.steps, 300)
    t_tile_b = timed(tile_bwd_ref, n_ref)
    t_tile_f = timed(tile_fwd_ref, n_ref)
    ref_f, ref_b, ref_c = attainable(torch, stream, [[s_[0], s_[1], s_[2].t(), s_[3].t()] for s_ in sets],
                                     n_ref, restore)
    del tsets, sets
    torch.cuda.empty_cache()
    gbs = lambda nbytes, ms: round(nbytes / (ms * 1e-3) / 1e9, 1)
    traffic = committed_traffic(TILE_PMC_SUMMARY, "bwd_traffic_bytes")
    value = gbs(BWD_BYTES, t_bwd)
    result = {
        "metric": "achieved HBM GB/s (% of peak) for bf16 silu backward, transposed dy view, 4096x14336",
        "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(t_bwd, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": f"synthetic (seeded as the main step; {args.sets} rotating buffer sets; a, b restored from a "
                "pristine device copy after every batch of one pass over the sets, untimed)",
        "config": {"workload": "SwiGLU bf16 backward in place, a, b row-major (4096, 14336), dy a transposed "
                               "view (column-major), no copies", "rows": ROWS, "cols": COLS,
                   "bytes_per_step": BWD_BYTES},
        "pct_of_peak": round(100 * value / PEAK_HBM_GBS, 2),
        "pct_of_attainable": round(100 * t_tile_b / t_bwd, 2),
        "attainable": {"tile_bwd_mix": {"avg_us": round(1e3 * t_tile_b, 2), "GBps": gbs(BWD_BYTES, t_tile_b)},
                       "tile_fwd_mix": {"avg_us": round(1e3 * t_tile_f, 2), "GBps": gbs(FWD_BYTES, t_tile_f)},
                       "rowmajor_fwd_mix": {"avg_us": round(1e3 * ref_f, 2), "GBps": gbs(FWD_BYTES, ref_f)},
                       "rowmajor_bwd_mix": {"avg_us": round(1e3 * ref_b, 2), "GBps": gbs(BWD_BYTES, ref_b)},
                       "copy_GBps": gbs(2 * N * ES, ref_c),
                       "note": "data-movement reference kernels (libglu_ref.so) in this run on the same storage: "
                               "the tiled kernel's own 64 x 64 tile pattern with the transposed operand turned "
                               "around through LDS and no arithmetic (pct_of_attainable: the backward against "
                               "it), and the row-major streams as context"},
        "kernels": {
            "bwd_dyT": {"avg_us": round(1e3 * t_bwd, 2), "GBps": value, "path": "tiles",
                        "pct_of_rowmajor_mix": round(100 * ref_b / t_bwd, 2)},
            "fwd_yT": {"avg_us": round(1e3 * t_fwd, 2), "GBps": gbs(FWD_BYTES, t_fwd), "path": "tiles",
                       "pct_of_tile_mix": round(100 * t_tile_f / t_fwd, 2),
                       "pct_of_rowmajor_mix": round(100 * ref_f / t_fwd, 2)},
            "all_T_fwd_bwd": {"avg_us": round(1e3 * t_allT, 2), "GBps": gbs(STEP_BYTES, t_allT),
                              "path": "streaming kernels on the transposed problem"},
            "copy_then_bwd": {"avg_us": round(1e3 * t_copy, 2), "GBps": gbs(BWD_BYTES, t_copy),
                              "path": "dy.contiguous() + row-major backward"},
        },
        "roofline": {"bound": "hbm", "kernel": "glu_tile_kernel<bf16, silu, bwd>", "achieved": value,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(value / PEAK_HBM_GBS, 4),
                     "traffic": traffic},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(a_h, b_h, dy_h, bwd_only=True)
    print(json.dumps(result), flush=True)


PEAK_BF16_TFLOPS = 2500.0


def gemm_shape_sweep(torch, glu, inputs, dev, timed):
    """Fused against unfused gate/up projection at few tokens over several MLP
    shapes, bf16 SwiGLU, with the path GatedMLP's default picks.  Weight
    copies rotate over at least 1 GiB, so every call streams them from HBM."""
    from mlp_gated_activation_amd.functional import fused_epilogue_wins
    out = []
    for K, N in ((4096, 11008), (5120, 13824), (8192, 28672), (3584, 18944), (2048, 8192)):
        nw = max(2, -(-(1 << 30) // (2 * N * K * 2)))
        x_h, w_h = inputs.gemm_glu(256, N, K, "bf16", seed=0)
        ws = [w_h.to(dev) for _ in range(nw)]
        x = x_h.to(dev)
        for M in (1, 16, 64, 128, 256):
            xs = x[:M]
            hs = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            gus = torch.empty(M, 2 * N, dtype=torch.bfloat16, device=dev)
            t_f = timed(lambda i: glu.glu_gemm_fwd("silu", xs, ws[i % nw], h=hs), 60)
            t_u = timed(lambda i: (torch.matmul(xs, ws[i % nw].t(), out=gus),
                                   glu.glu_fwd("silu", "gate_up", gus, y=hs)), 60)
            out.append({"hidden": K, "intermediate": N, "M": M, "fused_us": round(1e3 * t_f, 1),
                        "unfused_us": round(1e3 * t_u, 1), "speedup_vs_unfused": round(t_u / t_f, 3),
                        "auto_picks_fused": fused_epilogue_wins(M, N, dev)})
        del ws
        torch.cuda.empty_cache()
        print(f"gemm shapes: {K} x {N} done", file=sys.stderr, flush=True)
    return out


def bench_gemm(args, torch, glu, inputs, dev):
    """Gate/up projection with the activation fused into the GEMM epilogue
    ("Fused Kernels", section 4), bf16 SwiGLU: x (4096, 4096), fused
    [gate | up] weight (2*14336, 4096), h (4096, 14336).  Flops per step:
    2 * M * K * 2N.  Compared with hipBLASLt (F.linear) producing [g | u]
    followed by this library's elementwise forward."""
    M, K, N = 4096, 4096, 14336
    flops = 2 * M * K * 2 * N
    x_h, w_h = inputs.gemm_glu(M, N, K, "bf16", seed=0)
    nsets = 2
    sets = [(x_h.to(dev), w_h.to(dev), torch.empty(M, N, dtype=torch.bfloat16, device=dev)) for _ in range(nsets)]
    gu = torch.empty(M, 2 * N, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream(dev)
    import torch.nn.functional as F
    steps = min(args.steps, 200)

    def timed(fn, n):
        return event_ms(torch, stream, fn, n, warmup=min(n, 10))

    def fused(i):
        x, w, h = sets[i % nsets]
        glu.glu_gemm_fwd("silu", x, w, h=h)

    def fused_gu(i):
        x, w, h = sets[i % nsets]
        glu.glu_gemm_fwd("silu", x, w, h=h, gu=gu)

    def blas_only(i):
        x, w, h = sets[i % nsets]
        torch.matmul(x, w.t(), out=gu)

    def blas_then_glu(i):
        x, w, h = sets[i % nsets]
        torch.matmul(x, w.t(), out=gu)
        glu.glu_fwd("silu", "gate_up", gu, y=h)

    t_fused = timed(fused, steps)
    t_fused_gu = timed(fused_gu, steps)
    t_blas = timed(blas_only, steps)
    t_unfused = timed(blas_then_glu, steps)

    # Context: the same projection over token counts (four weight copies
    # rotate, so every call streams the weights from HBM).  At few tokens the
    # kernel takes its small-tile configuration.
    m_sweep = []
    ws = [sets[i % nsets][1] for i in range(2)] + [w_h.to(dev) for _ in range(2)]
    for Ms in (16, 64, 128, 256, 1024):
        xs = sets[0][0][:Ms]
        hs = torch.empty(Ms, N, dtype=torch.bfloat16, device=dev)
        gus = torch.empty(Ms, 2 * N, dtype=torch.bfloat16, device=dev)
        t_f = timed(lambda i: glu.glu_gemm_fwd("silu", xs, ws[i % 4], h=hs), 100)
        t_u = timed(lambda i: (torch.matmul(xs, ws[i % 4].t(), out=gus), glu.glu_fwd("silu", "gate_up", gus, y=hs)), 100)
        m_sweep.append({"M": Ms, "fused_us": round(1e3 * t_f, 1), "unfused_us": round(1e3 * t_u, 1),
                        "speedup_vs_unfused": round(t_u / t_f, 3),
                        "weights_GBps_fused": round(2 * N * K * 2 / (t_f * 1e-3) / 1e9, 1)})
    del sets, gu, ws
    torch.cuda.empty_cache()
    shape_sweep = gemm_shape_sweep(torch, glu, inputs, dev, timed) if args.gemm_shapes else None
    tf = lambda ms: round(flops / (ms * 1e-3) / 1e12, 1)
    value = tf(t_fused)
    result = {
        "metric": "achieved TFLOP/s (% of bf16 MFMA peak) for the gate/up projection with the SwiGLU "
                  "activation fused into its epilogue, 4096 tokens x hidden 4096 -> I 14336",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": 10,
        "ms_per_step": round(t_fused, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded x ~ N(0,1), w ~ N(0, 0.02^2), bf16; 2 rotating buffer sets)",
        "config": {"workload": "h = silu(x @ Wg^T) * (x @ Wu^T), bf16, M=4096, K=4096, N=14336, fp32 accumulation",
                   "M": M, "K": K, "N": N, "flops_per_step": flops},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "kernels": {
            "fused": {"avg_us": round(1e3 * t_fused, 1), "TFLOPs": value},
            "fused_with_gu": {"avg_us": round(1e3 * t_fused_gu, 1), "TFLOPs": tf(t_fused_gu),
                              "note": "also writes the pre-activations [g | u] for a backward"},
            "hipblaslt_gemm_only": {"avg_us": round(1e3 * t_blas, 1), "TFLOPs": tf(t_blas),
                                    "note": "torch.matmul x @ W^T -> [g | u], no activation"},
            "hipblaslt_then_glu_fwd": {"avg_us": round(1e3 * t_unfused, 1), "TFLOPs": tf(t_unfused),
                                       "note": "the unfused path: GEMM writes [g | u], glu_fwd reads it"},
        },
        "speedup_vs_unfused": round(t_unfused / t_fused, 3),
        "m_sweep": m_sweep,
        "shape_sweep": shape_sweep,
        "roofline": {"bound": "mfma", "kernel": "gemm_glu_kernel<bf16, silu>", "achieved": value,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(value / PEAK_BF16_TFLOPS, 4),
                     "traffic": committed_traffic(GEMM_PMC_SUMMARY, "traffic_bytes", GEMM_SOURCES)},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        rows = M
        fx = x_h[:rows].to(torch.float64).numpy()
        fw = w_h.to(torch.float64).numpy()
        t0 = time.perf_counter()
        oracle.gemm_glu("silu", fx, fw[:N], fw[N:])
        dt = time.perf_counter() - t0
        sample_flops = 2 * rows * K * 2 * N
        result["cpu_baseline"] = {"value": round(sample_flops / dt / 1e12, 6), "unit": "TFLOP/s",
                                  "cores": oracle.num_threads(), "kind": "oracle",
                                  "sample": "the full workload (fp64 scalar C, OpenMP over rows), one run",
                                  "seconds": round(dt, 2)}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
