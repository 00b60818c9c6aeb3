#!/usr/bin/env python3
"""Throughput of the MXFP8 GroupedMLP forward + backward on one MI355X.

Workload (the Mixtral-8x7B expert shape): T=16384 tokens routed top-2
(M=32768 token-sorted rows), E=8 experts, H=4096, F=14336 (gate-up W1
[8, 28672, 4096], down W2 [8, 4096, 14336]), Zipf(1.1) expert loads
[13047, 6087, 3897, 2839, 2221, 1818, 1534, 1325], dY ~ N(0, 1).  Seeded
synthetic inputs drawn on the GPU; everything stays resident in HBM.

One step = grouped_mlp_fwd + grouped_mlp_bwd in the default recompute mode:
quantization of X, W1, W2 and dY (rowwise and columnwise), the fused
gate-up/SwiGLU/routing-scale/requant GEMM (h stays on chip), the down GEMM,
the fused backward GEMM (h recomputed from the saved X codes, dz, SwiGLU
backward, dr, requant), the gate-up dgrad GEMM and both weight-gradient GEMMs.

Prints one JSON line: tokens/s (value) over exactly K steps bracketed by
device synchronizations, per-step GPU times (median, min, p90) from events on
the stream the library runs on, TFLOP/s counted as 18*H*F per routed row
(algorithmic; the recompute's 4*H*F per row is reported as the executed
figure beside it), the dominant kernel's roofline (launch durations from HIP
events the library records on its stream around each of its launches, in a
second pass of the same K steps so that the headline carries no event
overhead), and the FP64 CPU oracle timed on a bounded sample as a reported
baseline.  "save_h" times the same step in the mode that stores h as bf16
instead of recomputing it, with the activation bytes each mode keeps for the
backward; "forward_only" times the forward alone (with and without the weight
quantization); "weights_cached" the step with the forward reusing the MXFP8
weight copies of an earlier forward (as across the micro-batches of one
optimizer step); the headline always quantizes the weights.  "routing"
times the steps around the expert path at the same shape (router, sorted-row plan,
permute fused with quantization, combine and its backward), not in the step;
"fine_grained_64e" times the same fwd+bwd step at the 64-expert long-sequence
workload (T=32768 top-8, H=2048, F=1408, 8 empty experts), and
"ep8_one_rank_share" the share of the slowest rank if the 8 experts were spread
over 8 GPUs (E=1, the largest expert's 13047 rows), neither in the headline.
"grouped_linear" times GroupedLinear at its own workload (T=8192 top-2, E=8,
K=1024, N=2816) in MXFP8 and in per-tensor FP8, and the tiny BF16 workload
(T=256 top-2, E=4, K=128, N=256) as one grouped launch against a loop of one
launch per expert, not in the step either.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --headline-only [--workload fine_grained_64e]   (profiler runs)
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0     # MI355X dense FP8 / MXFP8 MFMA
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="time the headline step only (and its launch-record pass): no side "
                         "figures, for short profiler runs")
    ap.add_argument("--workload", default="mixtral_fwd_bwd",
                    choices=["mixtral_fwd_bwd", "fine_grained_64e"],
                    help="with --headline-only: the step's workload (the headline is the "
                         "Mixtral shape; the 64-expert workload is there for profiler runs)")
    ap.add_argument("--copy-calib-mib", type=int, default=0,
                    help="after the timed steps, run one plain device copy of this many "
                         "MiB (read + write), the reference dispatch that scales "
                         "FETCH_SIZE / WRITE_SIZE counter readings to bytes")
    return ap.parse_args()


def kernel_table(gm, lib):
    """Per-kernel aggregates of the launch records of the timed region."""
    n = lib.mx_profile_count()
    name = ctypes.c_char_p()
    ms = ctypes.c_float()
    work = ctypes.c_double()
    unit = ctypes.c_int32()
    agg = {}
    for i in range(n):
        st = lib.mx_profile_get(i, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(work),
                                ctypes.byref(unit))
        if st != 0:
            raise RuntimeError(gm.last_error())
        a = agg.setdefault(name.value.decode(), {"launches": 0, "ms": 0.0, "work": 0.0,
                                                 "unit": unit.value})
        a["launches"] += 1
        a["ms"] += ms.value
        a["work"] += work.value
    return agg


def step_stats(ms_list):
    """Median, min and p90 (nearest rank) of per-step GPU times in ms."""
    v = sorted(ms_list)
    n = len(v)
    med = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
    p90 = v[min(n - 1, max(0, -(-9 * n // 10) - 1))]
    return {"median": round(med, 4), "min": round(v[0], 4), "p90": round(p90, 4)}


def time_steps(step, steps, warmup, label):
    """Wall time of exactly `steps` calls of step(), bracketed by device
    synchronizations (after `warmup` untimed calls), and each call's GPU time
    from a pair of events on the current stream, the stream the library's
    kernels run on."""
    import torch
    for i in range(warmup):
        step()
        torch.cuda.synchronize()
        print(f"[bench] {label}: warmup {i + 1}/{warmup}", file=sys.stderr, flush=True)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    print(f"[bench] {label}: {steps} steps in {elapsed:.3f} s", file=sys.stderr, flush=True)
    return elapsed, step_stats([a.elapsed_time(b) for a, b in evs])


def profiled_pass(gm, lib, step, steps):
    """Per-kernel launch records of `steps` calls of step() (library launch
    timing on), after one untimed call."""
    import torch
    step()
    torch.cuda.synchronize()
    if lib.mx_profile_begin(64 * max(steps, 1)) != 0:
        raise RuntimeError(gm.last_error())
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    lib.mx_profile_end()
    return kernel_table(gm, lib)


TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "mixtral_fwd_bwd_hbm_traffic.json")


def kernel_sources_sha256():
    """Hash of the library's device and host sources, to tell whether the
    kernels have changed since the counter record was taken."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "grouped_gemm_mxfp8_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(f.encode())
            with open(os.path.join(d, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    record (FETCH_SIZE and WRITE_SIZE passes, scaled by a 1 GiB copy), or
    None when there is no record or the sources changed since it was taken."""
    try:
        with open(TRAFFIC_RECORD) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_sources_sha256():
        return None
    ent = rec.get("per_launch", {}).get(kernel)
    return None if ent is None else int(round(ent["bytes"]))


def roofline(agg, with_traffic=True):
    name, a = max(agg.items(), key=lambda kv: kv[1]["ms"])
    sec = a["ms"] / 1e3
    if a["unit"] == 0:
        achieved = a["work"] / sec / 1e12
        peak, unit, bound = FP8_PEAK_TFLOPS, "TFLOP/s", "mfma"
    else:
        achieved = a["work"] / sec / 1e9
        peak, unit, bound = HBM_PEAK_GBS, "GB/s", "hbm"
    return {"kernel": name, "bound": bound, "achieved": round(achieved, 2), "peak": peak,
            "unit": unit, "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(name) if with_traffic else None,
            "traffic_unit": "HBM bytes per launch",
            "launches": a["launches"], "avg_launch_ms": round(a["ms"] / a["launches"], 4)}


def cpu_baseline(seed, T, M, E, H, F):
    """The FP64 oracle (as it is) on a bounded sample of the same workload.

    Sample: one expert, full H=4096, a slice of Fs=2048 of the F=14336
    intermediate units (gate and up rows and the matching W2 columns), run on
    n=1024 and n=2048 rows (some 10-20 s of host time on 16 cores).  The
    oracle's time is linear in rows and in F, with a per-expert part (weight
    quantization) and a per-row part; the two runs give both, and the whole
    step is extrapolated as
        (F/Fs) * (E * per_expert + M * per_row).
    """
    import numpy as np
    import torch
    from oracle import mx_oracle as O
    # every host CPU this process may run on, all given to the BLAS the
    # oracle's matmuls call
    ncpu = len(os.sched_getaffinity(0))
    blas = "unknown"
    limiter = None
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=ncpu, user_api="blas")
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
            threads = max(i.get("num_threads", 1) for i in info)
        else:
            threads = 1
    except Exception:
        threads = 1
    Fs, n = 2048, 1024
    g = torch.Generator().manual_seed(seed)
    bf = lambda *s, std=1.0: (torch.randn(*s, generator=g) * std).to(torch.bfloat16).double().numpy()
    X, dY = bf(2 * n, H), bf(2 * n, H)
    W1, W2 = bf(1, 2 * Fs, H, std=0.02), bf(1, H, Fs, std=0.02)
    r = torch.rand(2 * n, generator=g, dtype=torch.float64).numpy()

    def run(rows):
        off = np.array([0, rows])
        t = time.perf_counter()
        Y, saved = O.grouped_mlp_fwd(X[:rows], W1, W2, r[:rows], off)
        O.grouped_mlp_bwd(dY[:rows], X[:rows], W1, W2, r[:rows], off, saved)
        return time.perf_counter() - t

    t1 = run(n)
    t2 = run(2 * n)
    if limiter is not None:
        limiter.unregister()
    per_row = max((t2 - t1) / n, 1e-12)
    per_expert = max(t1 - n * per_row, 0.0)
    est = (F / Fs) * (E * per_expert + M * per_row)
    return {"value": round(T / est, 3), "unit": "tokens/s", "cores": threads,
            "host_cpus": ncpu, "blas": blas, "kind": "oracle",
            "sample": (f"FP64 NumPy oracle fwd+bwd on 1 expert, H={H}, F slice {Fs}/{F}, "
                       f"{n} and {2 * n} rows ({t1:.1f} s + {t2:.1f} s); step time "
                       f"extrapolated linearly to E={E}, M={M} rows, F={F}: {est:.0f} s"),
            "est_step_s": round(est, 1)}


def time_call(gm, lib, f, reps, flush=None):
    """GPU ms per call of f(): the library's launch records (events on its
    stream around each of its launches) over reps calls, one call before,
    untimed.  Unlike a wall clock around the calls, this leaves out the
    host's time to issue them, which exceeds the kernels' for the small
    steps timed here.  flush: called before each timed call (not timed),
    to evict the caches."""
    import torch
    f()
    torch.cuda.synchronize()
    if lib.mx_profile_begin(64 * reps) != 0:
        raise RuntimeError(gm.last_error())
    for _ in range(reps):
        if flush is not None:
            flush()
        out = f()
    torch.cuda.synchronize()
    lib.mx_profile_end()
    agg = kernel_table(gm, lib)
    return sum(a["ms"] for a in agg.values()) / reps, out


def linear_figures(gm, lib, dev, reps):
    """GroupedLinear at its MXFP8 workload (T=8192 top-2, E=8, K=1024, N=2816,
    1% outliers x100): MXFP8 against per-tensor FP8 (not part of the step).
    Quantizers: algorithmic bytes (bf16 read once, codes and scales written;
    per-tensor FP8 reads its input twice, amax before cast)."""
    from workloads import make_linear_case
    case = make_linear_case("mxfp8_linear", seed=0)
    x, w, offs = case.X.to(dev), case.W.to(dev), case.offsets.to(dev)
    M, K = x.shape
    E, N, _ = w.shape
    flops = 2.0 * M * N * K
    gbs = lambda ms, nbytes: round(nbytes / ms / 1e6, 1)
    timed = lambda f: time_call(gm, lib, f, reps)
    ms_mqx, mx_x = timed(lambda: gm.mxfp8_quantize(x))
    ms_mqw, mx_w = timed(lambda: gm.mxfp8_quantize(w))
    ms_mg, _ = timed(lambda: gm.grouped_linear_fwd(mx_x["row"], offs, mx_w["row"]))
    # the same calls with the caches flushed before each one: the whole
    # working set fits the 256 MB Infinity Cache, so warm calls read it from
    # there; a 512 MB write in between evicts it
    flush = make_flush(dev)
    flushed = lambda f: time_call(gm, lib, f, reps, flush=flush)[0]
    fl_mqx = flushed(lambda: gm.mxfp8_quantize(x))
    fl_mg = flushed(lambda: gm.grouped_linear_fwd(mx_x["row"], offs, mx_w["row"]))
    T = case.T
    ms_pqx, pt_x = timed(lambda: gm.fp8_tensor_quantize(x, offs))
    ms_pqw, pt_w = timed(lambda: gm.fp8_tensor_quantize(w))
    ms_pg, _ = timed(lambda: gm.grouped_linear_fwd_fp8(pt_x, offs, pt_w))
    mx_bytes = lambda n: n * (2 + 1 + 1 / 32)
    pt_bytes = lambda n: n * (2 + 2 + 1)
    return {
        "shape": {"M": M, "K": K, "N": N, "E": E},
        "mxfp8": {"quant_x_ms": round(ms_mqx, 4), "quant_x_gbs": gbs(ms_mqx, mx_bytes(M * K)),
                  "quant_w_ms": round(ms_mqw, 4), "quant_w_gbs": gbs(ms_mqw, mx_bytes(E * N * K)),
                  "gemm_ms": round(ms_mg, 4), "gemm_tflops": round(flops / ms_mg / 1e9, 1),
                  "gemm_frac_fp8_peak": round(flops / ms_mg / 1e9 / FP8_PEAK_TFLOPS, 4),
                  "quant_x_plus_gemm_tokens_per_s": round(T / ((ms_mqx + ms_mg) / 1e3), 1),
                  "flushed": {"quant_x_ms": round(fl_mqx, 4),
                              "quant_x_gbs": gbs(fl_mqx, mx_bytes(M * K)),
                              "gemm_ms": round(fl_mg, 4),
                              "gemm_tflops": round(flops / fl_mg / 1e9, 1),
                              "quant_x_plus_gemm_tokens_per_s":
                                  round(T / ((fl_mqx + fl_mg) / 1e3), 1)}},
        "fp8_per_tensor": {"quant_x_ms": round(ms_pqx, 4),
                           "quant_x_gbs": gbs(ms_pqx, pt_bytes(M * K)),
                           "quant_w_ms": round(ms_pqw, 4),
                           "quant_w_gbs": gbs(ms_pqw, pt_bytes(E * N * K)),
                           "gemm_ms": round(ms_pg, 4),
                           "gemm_tflops": round(flops / ms_pg / 1e9, 1)},
    }


def make_flush(dev, mib=512):
    """A device write of `mib` MiB, twice the Infinity Cache, that evicts
    earlier data from the caches."""
    import torch
    buf = torch.empty(mib << 20, dtype=torch.uint8, device=dev)
    state = {"v": 0}

    def flush():
        state["v"] = (state["v"] + 1) & 0xFF
        buf.fill_(state["v"])
    return flush


def grouped_vs_loop_figures(gm, lib, dev, reps=200):
    """The tiny BF16 GroupedLinear workload (T=256 top-2, E=4, K=128, N=256):
    one grouped launch driven by the device offsets against one launch per
    expert (the loop the grouped call replaces; its per-expert row ranges are
    taken from the host, as such a loop needs them).  Both are bound by launch
    cost at this size, so the figure is wall-clock time per call with the
    host's issue included (reps calls back to back, one synchronization at
    the end), plus the GPU time of the grouped launch from the library's
    launch records."""
    import torch
    from workloads import make_linear_case
    case = make_linear_case("tiny_bf16_linear", seed=0)
    x, w, offs = case.X.to(dev), case.W.to(dev), case.offsets.to(dev)
    E = w.shape[0]
    off_h = case.offsets.tolist()
    parts = [(x[off_h[e]:off_h[e + 1]], torch.tensor([0, off_h[e + 1] - off_h[e]],
                                                    dtype=torch.int64, device=dev), w[e:e + 1])
             for e in range(E) if off_h[e + 1] > off_h[e]]

    def grouped():
        return gm.grouped_linear_fwd(x, offs, w)

    def loop():
        return [gm.grouped_linear_fwd(xe, oe, we) for xe, oe, we in parts]

    def wall_us(f):
        for _ in range(10):
            f()
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(reps):
            f()
        torch.cuda.synchronize()
        return (time.perf_counter() - t) / reps * 1e6

    g_us, l_us = wall_us(grouped), wall_us(loop)
    gpu_ms, _ = time_call(gm, lib, grouped, reps)
    gpu_fl_ms, _ = time_call(gm, lib, grouped, min(reps, 50), flush=make_flush(dev))
    return {"shape": {"M": int(x.shape[0]), "K": int(x.shape[1]), "N": int(w.shape[1]), "E": E},
            "grouped_us_per_call": round(g_us, 2), "per_expert_loop_us_per_call": round(l_us, 2),
            "loop_over_grouped": round(l_us / g_us, 2), "grouped_gpu_us": round(gpu_ms * 1e3, 2),
            "grouped_gpu_us_flushed": round(gpu_fl_ms * 1e3, 2)}


def one_rank_share_figures(gm, lib, dev, seed, steps):
    """Expert parallelism over 8 GPUs would give each rank one expert; under the
    Zipf loads the slowest rank holds the largest expert (13047 rows).  That
    rank's fwd+bwd at its real shape (E=1, M=13047, H=4096, F=14336), timed on
    this one GPU (not part of the headline)."""
    import torch
    from workloads import make_mlp_case
    n = 13047
    case = make_mlp_case(None, seed=seed, T=n, k=1, E=1, H=4096, F=14336, routing="counts",
                         counts=[n], device=dev)
    M, H, F, E = case.M, case.H, case.F, case.E
    fws = torch.empty(gm.fwd_ws_bytes(M, H, F, E), dtype=torch.uint8, device=dev)
    bws = torch.empty(gm.bwd_ws_bytes(M, H, F, E), dtype=torch.uint8, device=dev)

    def step():
        y, ctx = gm.grouped_mlp_fwd(case.X, case.offsets, case.W1, case.W2, case.r, ws=fws)
        return gm.grouped_mlp_bwd(case.dY, case.offsets, case.W1, case.W2, case.r, ctx, ws=bws)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t) / steps * 1e3
    tflops = 18.0 * H * F * M / (ms / 1e3) / 1e12
    return {"shape": {"M": M, "E": E, "H": H, "F": F}, "ms_per_step": round(ms, 4),
            "rows_per_s": round(M / (ms / 1e3), 1), "tflops": round(tflops, 2),
            "frac_fp8_peak": round(tflops / FP8_PEAK_TFLOPS, 4)}


def many_expert_figures(gm, lib, dev, seed, steps):
    """GroupedMLP fwd+bwd at the fine-grained long-sequence workload (T=32768
    tokens top-8, M=262144 rows, E=64, H=2048, F=1408; 8 experts get no rows,
    the largest gets ~12% of them): step time, throughput and the per-kernel
    split, from the library's launch records (not part of the headline)."""
    import torch
    from workloads import make_mlp_case
    case = make_mlp_case("fine_grained_64e", seed=seed, device=dev)
    M, H, F, E, T = case.M, case.H, case.F, case.E, case.T
    fws = torch.empty(gm.fwd_ws_bytes(M, H, F, E), dtype=torch.uint8, device=dev)
    bws = torch.empty(gm.bwd_ws_bytes(M, H, F, E), dtype=torch.uint8, device=dev)

    def step():
        y, ctx = gm.grouped_mlp_fwd(case.X, case.offsets, case.W1, case.W2, case.r, ws=fws)
        return gm.grouped_mlp_bwd(case.dY, case.offsets, case.W1, case.W2, case.r, ctx, ws=bws)

    for _ in range(2):
        step()
    torch.cuda.synchronize()
    if lib.mx_profile_begin(64 * steps) != 0:
        raise RuntimeError(gm.last_error())
    t = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t
    lib.mx_profile_end()
    agg = kernel_table(gm, lib)
    ms = elapsed / steps * 1e3
    tflops = 18.0 * H * F * M / (ms / 1e3) / 1e12
    counts = [int(c) for c in case.counts]
    return {"shape": {"T": T, "k": case.k, "M": M, "E": E, "H": H, "F": F,
                      "empty_experts": sum(c == 0 for c in counts),
                      "largest_expert_rows": max(counts)},
            "ms_per_step": round(ms, 4), "tokens_per_s": round(T / (ms / 1e3), 1),
            "tflops": round(tflops, 2), "frac_fp8_peak": round(tflops / FP8_PEAK_TFLOPS, 4),
            "kernels_ms_per_step": {k: round(v["ms"] / steps, 4)
                                    for k, v in sorted(agg.items(), key=lambda kv: -kv[1]["ms"])}}


def routing_figures(gm, lib, case, dev, reps):
    """The steps around the expert path at the same shape (not part of the
    step): the router (top-2 of fp32 logits and their softmax), the
    sorted-row plan of the top-2 routing, the permute of the token
    rows fused with both MXFP8 copies, the unweighted combine back to token
    order and its backward (the token -> sorted-row permute of a gradient).
    Algorithmic bytes per call: every row read and written once."""
    import numpy as np
    import torch
    T, k, E, H = case.T, case.k, case.E, case.H
    M = case.M
    expert_of_row = np.repeat(np.arange(E), case.counts)
    order = np.lexsort((expert_of_row, case.token))          # rows by (token, expert)
    ids = torch.from_numpy(expert_of_row[order].reshape(T, k).astype(np.int32)).to(dev)
    first = np.zeros(T, dtype=np.int64)
    first[case.token[::-1]] = np.arange(M)[::-1]             # a sorted row of every token
    x_tok = case.X[torch.from_numpy(first).to(dev)].contiguous()
    y = case.dY

    timed = lambda f: time_call(gm, lib, f, reps)

    logits = torch.randn((T, E), dtype=torch.float32, device=dev,
                         generator=torch.Generator(device=dev).manual_seed(3))
    ms_router, _ = timed(lambda: gm.router(logits, k))
    ms_plan, (offs, row_of, tok_of, _) = timed(lambda: gm.route_plan(ids, E))
    ms_pq, _ = timed(lambda: gm.permute_quantize(x_tok, tok_of, offs, M))
    ms_c, _ = timed(lambda: gm.combine(y, row_of))
    ms_cb, _ = timed(lambda: gm.combine_bwd(x_tok, row_of, M))
    fig = lambda ms, nbytes: {"ms": round(ms, 4), "gbs": round(nbytes / ms / 1e6, 1),
                              "frac_hbm": round(nbytes / ms / 1e6 / HBM_PEAK_GBS, 3)}
    return {
        "router": fig(ms_router, T * E * 4 + T * k * 8),
        "route_plan_ms": round(ms_plan, 4),
        "permute_quantize": fig(ms_pq, M * H * 2 + 2 * M * H * (1 + 1 / 32)),
        "combine": fig(ms_c, M * H * 2 + T * H * 2),
        "combine_bwd": fig(ms_cb, M * H * 2 * 2),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the expert path is "
                                   "built and measured on a single MI355X (no collectives); "
                                   "run with --gpus 1"}))
        return 2
    import torch
    import grouped_gemm_mxfp8_amd as gm
    from workloads import make_mlp_case

    lib = gm.lib()
    lib.mx_profile_begin.argtypes = [ctypes.c_int32]
    lib.mx_profile_get.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_char_p),
                                   ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double),
                                   ctypes.POINTER(ctypes.c_int32)]
    dev = torch.device("cuda:0")
    print(f"[bench] device {torch.cuda.get_device_name(dev)}; building inputs", file=sys.stderr,
          flush=True)
    if args.workload != "mixtral_fwd_bwd" and not args.headline_only:
        print(json.dumps({"error": "--workload other than the headline's needs --headline-only"}))
        return 2
    case = make_mlp_case(args.workload, seed=args.seed, device=dev)
    M, H, F, E, T = case.M, case.H, case.F, case.E, case.T
    x, w1, w2, r, off, dy = case.X, case.W1, case.W2, case.r, case.offsets, case.dY
    # workspaces large enough for both modes
    fws = torch.empty(max(gm.fwd_ws_bytes(M, H, F, E, sh) for sh in (False, True)),
                      dtype=torch.uint8, device=dev)
    bws = torch.empty(max(gm.bwd_ws_bytes(M, H, F, E, sh) for sh in (False, True)),
                      dtype=torch.uint8, device=dev)
    flops_step = 18.0 * H * F * M                 # algorithmic
    flops_recompute = 4.0 * H * F * M             # h = X W1^T again in the backward

    def make_step(save_h):
        def step():
            y, ctx = gm.grouped_mlp_fwd(x, off, w1, w2, r, ws=fws, save_h=save_h)
            return gm.grouped_mlp_bwd(dy, off, w1, w2, r, ctx, ws=bws)
        return step

    # ---- headline: recompute mode, library launch timing off ----
    step = make_step(False)
    elapsed, stats = time_steps(step, args.steps, args.warmup, "fwd+bwd")
    # the same steps with the library's launch records on, for the per-kernel
    # table and the roofline
    agg = profiled_pass(gm, lib, step, args.steps)

    if args.copy_calib_mib > 0:
        n = args.copy_calib_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy of {args.copy_calib_mib} MiB done", file=sys.stderr,
              flush=True)
        del src, dst

    def kernels_of(agg, steps):
        return {k: {"launches_per_step": v["launches"] / steps,
                    "ms_per_step": round(v["ms"] / steps, 4),
                    ("tflops" if v["unit"] == 0 else "gbs"):
                        round(v["work"] / (v["ms"] / 1e3) / (1e12 if v["unit"] == 0 else 1e9), 2)}
                for k, v in sorted(agg.items(), key=lambda kv: -kv[1]["ms"])}

    if args.headline_only:
        shape = ("Mixtral-8x7B expert shape" if args.workload == "mixtral_fwd_bwd" else
                 "64-expert long-sequence workload (T=32768 top-8, H=2048, F=1408)")
        out = {"metric": "GroupedMLP fwd+bwd tokens/s & TFLOP/s (MXFP8), " + shape,
               "value": round(T * args.steps / elapsed, 1), "unit": "tokens/s", "n_gpus": 1,
               "steps": args.steps, "warmup": args.warmup,
               "ms_per_step": round(elapsed / args.steps * 1e3, 4), "gpu_ms_per_step": stats,
               "tflops": round(flops_step * args.steps / elapsed / 1e12, 2),
               "roofline": roofline(agg, args.workload == "mixtral_fwd_bwd"),
               "kernels": kernels_of(agg, args.steps),
               "note": "headline only (--headline-only), workload " + args.workload}
        print(json.dumps(out), flush=True)
        return 0

    # ---- the save-h mode beside it ----
    nside = max(args.steps // 2, 3)
    el_s, stats_s = time_steps(make_step(True), nside, 1, "fwd+bwd save-h")
    agg_s = profiled_pass(gm, lib, make_step(True), 2)

    def saved_bytes(save_h):
        """Bytes the forward keeps for the backward that scale with the batch
        (everything in ctx past the weight copies)."""
        first = gm.MX_CTX_H if save_h else gm.MX_CTX_XROW
        off0 = int(lib.grouped_mlp_ctx_offset(first, M, H, F, E, gm.MX_MLP_SAVE_H if save_h else 0))
        return gm.ctx_bytes(M, H, F, E, save_h) - off0

    # ---- forward only, with and without the weight quantization ----
    fwd_flops = 6.0 * H * F * M
    cbuf = torch.empty(gm.ctx_bytes(M, H, F, E), dtype=torch.uint8, device=dev)
    el_f, stats_f = time_steps(lambda: gm.grouped_mlp_fwd(x, off, w1, w2, r, ws=fws,
                                                          ctx_buf=cbuf),
                               args.steps, 1, "fwd")
    el_fc, stats_fc = time_steps(lambda: gm.grouped_mlp_fwd(x, off, w1, w2, r, ws=fws,
                                                            ctx_buf=cbuf, reuse_weights=True),
                                 args.steps, 1, "fwd, weights cached")

    def fwd_fig(el, st, n):
        ms = el / n * 1e3
        tf = fwd_flops / (ms / 1e3) / 1e12
        return {"ms_per_step": round(ms, 4), "gpu_ms": st, "tokens_per_s": round(T / (ms / 1e3), 1),
                "tflops": round(tf, 2), "frac_fp8_peak": round(tf / FP8_PEAK_TFLOPS, 4)}

    # ---- fwd+bwd with the weight quantization cached ----
    gm.grouped_mlp_fwd(x, off, w1, w2, r, ws=fws, ctx_buf=cbuf)

    def step_cached():
        y, ctx = gm.grouped_mlp_fwd(x, off, w1, w2, r, ws=fws, ctx_buf=cbuf, reuse_weights=True)
        return gm.grouped_mlp_bwd(dy, off, w1, w2, r, ctx, ws=bws)

    el_c, stats_c = time_steps(step_cached, args.steps, 1, "fwd+bwd, weights cached")
    del cbuf

    routing = routing_figures(gm, lib, case, dev, reps=max(args.steps, 3))
    expert_rows = [int(c) for c in case.counts]
    del case, x, w1, w2, r, off, dy, fws, bws
    torch.cuda.empty_cache()
    many = many_expert_figures(gm, lib, dev, args.seed, steps=max(args.steps // 2, 3))
    torch.cuda.empty_cache()
    share = one_rank_share_figures(gm, lib, dev, args.seed, steps=max(args.steps // 2, 3))
    linear = linear_figures(gm, lib, dev, reps=max(args.steps, 3))
    linear["bf16_tiny_grouped_vs_loop"] = grouped_vs_loop_figures(gm, lib, dev)

    ms_step = elapsed / args.steps * 1e3
    tokens_s = T * args.steps / elapsed
    tflops = flops_step * args.steps / elapsed / 1e12
    ms_s = el_s / nside * 1e3
    tf_s = flops_step / (ms_s / 1e3) / 1e12

    out = {
        "metric": "GroupedMLP fwd+bwd tokens/s & TFLOP/s (MXFP8), Mixtral-8x7B expert shape",
        "value": round(tokens_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8_e4m3 (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": "mixtral_fwd_bwd: GroupedMLP fwd+bwd, T=16384 top-2 (M=32768 "
                               "rows), E=8, H=4096, F=14336, Zipf(1.1) loads; backward "
                               "recomputes h (nothing intermediate kept in HBM)",
                   "T": T, "M": M, "E": E, "H": H, "F": F,
                   "expert_rows": expert_rows},
        "gpu_ms_per_step": stats,
        "tflops": round(tflops, 2),
        "frac_fp8_peak": round(tflops / FP8_PEAK_TFLOPS, 4),
        "tflops_executed": round((flops_step + flops_recompute) * args.steps / elapsed / 1e12, 2),
        "frac_fp8_peak_executed": round((flops_step + flops_recompute) * args.steps / elapsed
                                        / 1e12 / FP8_PEAK_TFLOPS, 4),
        "roofline": roofline(agg),
        "kernels": kernels_of(agg, args.steps),
        "saved_for_backward": {
            "recompute": {"bytes": saved_bytes(False),
                          "bytes_per_token": round(saved_bytes(False) / T, 1),
                          "what": "rowwise and token-axis MXFP8 copies of X, token-axis copy "
                                  "of z, padded offsets"},
            "save_h": {"bytes": saved_bytes(True),
                       "bytes_per_token": round(saved_bytes(True) / T, 1),
                       "what": "bf16 pre-activation h, token-axis MXFP8 copies of X and z, "
                               "padded offsets"},
            "weights": {"bytes": int(lib.grouped_mlp_ctx_offset(gm.MX_CTX_XROW, M, H, F, E, 0)),
                        "what": "MXFP8 copies of W1 and W2 (rowwise and columnwise), made once "
                                "per step, independent of the batch"}},
        "save_h": {
            "ms_per_step": round(ms_s, 4), "gpu_ms_per_step": stats_s,
            "tokens_per_s": round(T / (ms_s / 1e3), 1), "tflops": round(tf_s, 2),
            "frac_fp8_peak": round(tf_s / FP8_PEAK_TFLOPS, 4),
            "kernels": kernels_of(agg_s, 2),
            "what": "same step, forward stores h as bf16 and the backward reads it instead of "
                    "recomputing it"},
        "forward_only": {
            "with_weight_quantization": fwd_fig(el_f, stats_f, args.steps),
            "weights_cached": fwd_fig(el_fc, stats_fc, args.steps),
            "what": "grouped_mlp_fwd alone (6*H*F flops per row): quantize X (and W1, W2), fused "
                    "gate-up + SwiGLU + routing scale + requantize, down GEMM"},
        "weights_cached": {
            "ms_per_step": round(el_c / args.steps * 1e3, 4), "gpu_ms_per_step": stats_c,
            "tokens_per_s": round(T * args.steps / el_c, 1),
            "what": "same step, forward reusing the MXFP8 weight copies of an earlier forward "
                    "(weights unchanged across micro-batches)"},
        "routing": routing,
        "fine_grained_64e": many,
        "ep8_one_rank_share": share,
        "grouped_linear": linear,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(args.seed, T, M, E, H, F)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
