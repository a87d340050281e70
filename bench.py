"""Benchmark of the fused attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--only {main,causal_mha,varlen_window,decode,bwd}]

A step is one fa_fwd call on the long-context causal GQA prefill workload
(B=1, Hq=32, Hkv=8, L=16384, d=128, bf16, seeded synthetic inputs resident in
HBM), the largest workload that the metric covers.  The timed region is
exactly K steps bracketed by torch.cuda.synchronize(); `value` is algorithmic
TFLOP/s (4*d FLOPs per visible (query, key) pair per query head) over that
wall time.  Each step is also bracketed by HIP events recorded on the launch
stream (torch's current stream, which the binding launches on), which give the
per-launch mean, median and minimum.

Before the W warmup steps each workload runs untimed for --prewarm-ms of wall
time: the GPU raises its engine clock only after some milliseconds of
sustained load.

"roofline" covers the dominant kernel of the step (the wide-tile prefill
kernel, which fa_fwd takes for head_dim 128 from 4096 query rows on): achieved = algorithmic FLOPs per launch / mean launch
duration from those events, against the bf16 dense MFMA peak.  "traffic" is
HBM bytes per launch from the committed rocprofv3 counter summary for that
kernel and workload, null if the kernel source changed since it was taken.
The causal MHA prefill (B=4, H=32, L=2048) and the paged decode call
(fa_decode_paged, no host plan) carry roofline blocks of their own; the other
workloads are reported under "workloads".  "hbm_context" gives the device
memory bandwidth measured on this GPU beside the 8 TB/s spec (a streaming
read by a probe kernel, and a device copy) and the decode rate as a fraction
of that read rate (context only; the decode roofline stays against the spec).  "cpu_baseline" times the CPU fp64
oracle on a bounded sample of the main workload on this host, and per
workload under "cpu_baseline.per_workload".  One JSON line is printed.
"""

import argparse
import ctypes
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0              # MI355X HBM3E (published)
MEMBW_LIB = os.path.join(ROOT, "exact_attention_17_amd", "libfa_membw.so")
METRIC = "prefill attn TFLOP/s (% MFMA peak); paged-decode KV GB/s (% HBM peak)"
PREFILL_SRC = os.path.join(ROOT, "exact_attention_17_amd", "csrc", "prefill_fwd.hip")
WIDE_SRC = os.path.join(ROOT, "exact_attention_17_amd", "csrc", "prefill_wide.hip")
DECODE_SRC = os.path.join(ROOT, "exact_attention_17_amd", "csrc", "decode_paged.hip")
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 512 << 20             # plain device copy used to calibrate the byte counters
PREFILL_KERNEL = "prefill_fwd_kernel<128, 0, false>"   # head_dim 128, fewer than 4096 query rows
WIDE_KERNEL = "prefill_fwd_wide_kernel"                 # head_dim 128, from 4096 query rows on


def visible_pairs(Lq, Lk, causal, wl, wr):
    """Number of visible (query, key) pairs of one head (closed form per row)."""
    i = np.arange(Lq, dtype=np.int64)
    pos = i + (Lk - Lq)
    lo = np.zeros(Lq, np.int64) if wl < 0 else np.maximum(0, pos - wl)
    hi = np.full(Lq, Lk, np.int64)
    if causal:
        hi = np.minimum(hi, pos + 1)
    if wr >= 0:
        hi = np.minimum(hi, pos + wr + 1)
    return int(np.maximum(0, hi - lo).sum())


def dense_flops(w):
    B, Lq, Hq, d = w.q.shape
    return 4.0 * d * Hq * B * visible_pairs(Lq, w.k.shape[1], w.causal, *w.window)


def varlen_flops(w):
    d, H = w.q.shape[2], w.q.shape[1]
    return 4.0 * d * H * sum(visible_pairs(int(L), int(L), w.causal, *w.window) for L in w.lens)


def decode_bytes(w):
    """Compulsory HBM bytes of one decode step: the used K/V rows once, q, o, lse,
    and the used block-table entries."""
    B, _, Hq, d = w.q.shape
    Hkv = w.k_cache.shape[2]
    tokens = int(w.seqlens.astype(np.int64).sum())
    pages = int((-(-w.seqlens.astype(np.int64) // w.page_size)).sum())
    return 2 * tokens * Hkv * d * 2 + 2 * B * Hq * d * 2 + B * Hq * 4 + pages * 4


def file_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def prewarm(fn, ms):
    """Call fn back to back for about `ms` of wall time (untimed), syncing every
    few calls so the launch queue stays short."""
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def timed_steps(fn, steps, warmup, prewarm_ms):
    """Pre-warm, W warmup calls, then exactly `steps` calls between two
    synchronisations, each call bracketed by HIP events on the launch stream.
    Returns wall ms per call and the per-call event durations (ms)."""
    prewarm(fn, prewarm_ms)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for s, e in ev:
        s.record()
        fn()
        e.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return wall, [s.elapsed_time(e) for s, e in ev]


def stats(durations):
    return {"mean": statistics.fmean(durations), "median": statistics.median(durations),
            "min": min(durations)}


def rate_entry(work, durations, unit, peak, scale):
    """Per-workload entry: ms (mean / median / min) and the rate at the mean."""
    st = stats(durations)
    rate = work / st["mean"] / scale
    out = {"ms": round(st["mean"], 4), "median_ms": round(st["median"], 4),
           "min_ms": round(st["min"], 4), "calls": len(durations), unit: round(rate, 2)}
    out["frac_mfma" if unit == "TFLOP/s" else "frac_hbm"] = round(rate / peak, 4)
    return out


def roofline_block(bound, work, durations, unit, peak, scale, traffic, kernel):
    st = stats(durations)
    ach = work / st["mean"] / scale
    return {"bound": bound, "achieved": round(ach, 2), "peak": peak, "unit": unit,
            "frac": round(ach / peak, 4), "traffic": traffic, "kernel": kernel,
            "avg_launch_ms": round(st["mean"], 4), "median_launch_ms": round(st["median"], 4),
            "min_launch_ms": round(st["min"], 4),
            "frac_at_median": round(work / st["median"] / scale / peak, 4),
            "launches": len(durations)}


def load_traffic(summary_name, src):
    """HBM bytes per launch from a committed counter summary (profiles/<name>.md),
    or None if missing or if the kernel source changed since it was taken."""
    vals = {}
    try:
        for line in open(os.path.join(PROFILES, summary_name + ".md")):
            if ":" in line and line.strip().startswith(("bytes_per_launch", "source_sha256_16")):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip().strip("`")
    except OSError:
        return None
    if vals.get("source_sha256_16") != file_hash(src) or "bytes_per_launch" not in vals:
        return None
    return float(vals["bytes_per_launch"])


def copy_calibration(reps=5):
    """A plain device-to-device copy of COPY_BYTES, so a counter run sees the
    FETCH_SIZE / WRITE_SIZE that a kernel of known traffic produces."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def _event_median(fn, reps):
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return statistics.median([a.elapsed_time(b) for a, b in ev])


def hbm_context(reps=20, nbytes=1 << 32):
    """Device memory bandwidth measured on this GPU, as context for the 8 TB/s
    spec: a streaming read of `nbytes` by the probe library (16-byte
    non-temporal loads, best of four grid sizes) and torch's device-to-device
    copy (bytes read + written).  Medians of `reps` event-timed calls."""
    if not os.path.exists(MEMBW_LIB):
        return {"error": "libfa_membw.so is not built"}
    lib = ctypes.CDLL(MEMBW_LIB)
    fn = lib.fa_membw_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    sink = torch.empty(16384 * 256, dtype=torch.int32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    per_grid = {}
    for blocks in (2048, 4096, 8192, 16384):
        def call(blocks=blocks):
            if fn(src.data_ptr(), nbytes, sink.data_ptr(), blocks, stream) != 0:
                raise RuntimeError("fa_membw_read failed")
        per_grid[blocks] = round(nbytes / _event_median(call, reps) / 1e6, 1)
    del sink
    half = src[: src.numel() // 2]
    dst = torch.empty_like(half)
    copy = 2 * half.numel() * 4 / _event_median(lambda: dst.copy_(half), reps) / 1e6
    del src, dst, half
    return {"read_GB/s": max(per_grid.values()), "read_GB/s_by_grid": per_grid,
            "copy_GB/s": round(copy, 1), "read_bytes": nbytes, "spec_GB/s": PEAK_HBM_GBS,
            "kinds": "read: fa_membw_read (16-byte non-temporal loads); copy: torch copy_ "
                     "(read + write)"}


# ------------------------------------------------------------------ CPU oracle
def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        return int(os.environ.get("OMP_NUM_THREADS", "1"))


def u16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def time_oracle_dense(w, heads, flops_total):
    """The oracle on every row of the given (batch, head) pairs of a dense workload."""
    import oracle
    B, L, Hq, _ = w.q.shape
    qb, kb, vb = u16(w.q), u16(w.k), u16(w.v)
    t0 = time.perf_counter()
    for b, h in heads:
        for r0 in range(0, L, 1024):
            oracle.attention_rows_ref(qb, kb, vb, b, h, np.arange(r0, min(L, r0 + 1024)),
                                      w.scale, w.causal, w.window)
    dt = time.perf_counter() - t0
    return dt, flops_total * len(heads) / (B * Hq)


def cpu_baseline(main_w, main_flops, per_workload):
    """The oracle (plain numpy fp64, as it is) on a bounded sample of the main
    workload, plus bounded samples of the others: seconds and the algorithmic rate
    of each sample."""
    heads = [(0, h) for h in (0, 6, 13, 19, 25, 31)]   # 6 of 32 query heads, every row
    dt, fl = time_oracle_dense(main_w, heads, main_flops)
    out = {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": oracle_threads(),
           "kind": "oracle", "seconds": round(dt, 2), "cpu_model": cpu_model(),
           "sample": f"query heads 0, 6, 13, 19, 25 and 31 (6 of 32) of {main_w.name}, all 16384 "
                     "rows each (3/16 of one step), full S and P rows in float64 (numpy)"}
    if per_workload:
        out["per_workload"] = per_workload_oracle()
    return out


def per_workload_oracle():
    import oracle
    res = {}
    w1 = workloads.small_dense(Hkv=1)
    t0 = time.perf_counter()
    oracle.attention_ref(u16(w1.q), u16(w1.k), u16(w1.v), w1.scale, w1.causal, w1.window)
    dt = time.perf_counter() - t0
    res[w1.name] = {"seconds": round(dt, 4), "sample": "whole step",
                    "GFLOP/s": round(dense_flops(w1) / dt / 1e9, 3)}
    w2 = workloads.causal_mha()
    dt, fl = time_oracle_dense(w2, [(0, h) for h in range(32)], dense_flops(w2))
    res[w2.name] = {"seconds": round(dt, 2), "sample": "batch 0, all 32 heads (1/4 of a step)",
                    "GFLOP/s": round(fl / dt / 1e9, 2)}
    del w2
    w4 = workloads.paged_decode()
    n = 16
    t0 = time.perf_counter()
    oracle.decode_paged_ref(u16(w4.q[:n]), u16(w4.k_cache), u16(w4.v_cache), w4.block_table[:n],
                            w4.seqlens[:n], w4.page_size, w4.scale)
    dt = time.perf_counter() - t0
    sub = workloads.Paged(w4.name, w4.q[:n], w4.k_cache, w4.v_cache, w4.block_table[:n],
                          w4.seqlens[:n], w4.page_size, w4.split_tokens, w4.scale)
    res[w4.name] = {"seconds": round(dt, 2), "sample": f"requests 0..{n - 1} (of 64)",
                    "GB/s": round(decode_bytes(sub) / dt / 1e9, 3)}
    del w4, sub
    w5 = workloads.varlen_window()
    heads = [0, 15]
    q5, k5, v5 = (u16(t[:, heads]) for t in (w5.q, w5.k, w5.v))
    cu = w5.cu_seqlens
    t0 = time.perf_counter()
    oracle.attention_varlen_ref(q5, k5, v5, cu, cu, w5.scale, w5.causal, w5.window)
    dt = time.perf_counter() - t0
    res[w5.name] = {"seconds": round(dt, 2), "sample": "heads 0 and 15 (2 of 16), every sequence",
                    "GFLOP/s": round(varlen_flops(w5) * len(heads) / 16 / dt / 1e9, 2)}
    return res


# ------------------------------------------------------------------ GPU parts
def bench_main(fa, w3, flops3, args):
    """The contract step: K timed fa_fwd calls on the long-context GQA workload."""
    q, k, v = w3.q.cuda(), w3.k.cuda(), w3.v.cuda()
    B, L, Hq, d = w3.q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")
    step = lambda: fa.fa_fwd(q, k, v, w3.scale, True, (-1, -1), out=o, lse=lse)
    wall, dur = timed_steps(step, args.steps, args.warmup, args.prewarm_ms)
    st = stats(dur)
    return {
        "value": round(flops3 / (wall * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
        "ms_per_step": round(wall, 4), "median_ms": round(st["median"], 4),
        "min_ms": round(st["min"], 4),
        "config": {"workload": w3.name, "B": B, "Hq": Hq, "Hkv": w3.k.shape[2], "L": L, "d": d,
                   "causal": True, "flops_per_step": flops3},
        "roofline": roofline_block("mfma", flops3, dur, "TFLOP/s", PEAK_BF16_TFLOPS, 1e9,
                                   load_traffic("prefill_fwd_wide_causal_gqa_long_traffic", WIDE_SRC),
                                   WIDE_KERNEL),
    }


def bench_causal_mha(fa, args):
    w2 = workloads.causal_mha()
    q, k, v = w2.q.cuda(), w2.k.cuda(), w2.v.cuda()
    o = torch.empty_like(q)
    lse = torch.empty((4, 32, 2048), dtype=torch.float32, device="cuda")
    f2 = dense_flops(w2)
    _, dur = timed_steps(lambda: fa.fa_fwd(q, k, v, w2.scale, True, (-1, -1), out=o, lse=lse),
                         args.steps, args.warmup, args.prewarm_ms)
    roof = roofline_block("mfma", f2, dur, "TFLOP/s", PEAK_BF16_TFLOPS, 1e9,
                          load_traffic("prefill_fwd_causal_mha_traffic", PREFILL_SRC),
                          PREFILL_KERNEL)
    roof["workload"] = w2.name
    entry = rate_entry(f2, dur, "TFLOP/s", PEAK_BF16_TFLOPS, 1e9)
    entry["flops"] = f2
    return entry, roof


def bench_varlen(fa, args):
    wl = {}
    w5 = workloads.varlen_window()
    a = [t.cuda() for t in (w5.q, w5.k, w5.v)]
    cu = torch.from_numpy(w5.cu_seqlens).cuda()
    f5 = varlen_flops(w5)
    o = torch.empty_like(a[0])
    lse = torch.empty((16, a[0].shape[0]), dtype=torch.float32, device="cuda")
    _, dur = timed_steps(lambda: fa.fa_fwd_varlen(*a, cu, cu, w5.max_seqlen, w5.max_seqlen,
                                                  w5.scale, True, w5.window, out=o, lse=lse),
                         args.steps, args.warmup, args.prewarm_ms)
    wl["varlen_window"] = rate_entry(f5, dur, "TFLOP/s", PEAK_BF16_TFLOPS, 1e9)
    wl["varlen_window"]["flops"] = f5
    # plan / run split: the host plan (heaviest tiles first) is made once for the
    # batch's lengths and reused; its host time is reported beside the run
    t0 = time.perf_counter()
    plan = fa.fa_varlen_plan(w5.cu_seqlens, w5.cu_seqlens, True, w5.window)
    plan_ms = (time.perf_counter() - t0) * 1e3
    plan_d = torch.from_numpy(plan).cuda()
    _, dur = timed_steps(lambda: fa.fa_fwd_varlen_run(*a, cu, cu, plan_d, w5.max_seqlen,
                                                      w5.max_seqlen, w5.scale, True, w5.window,
                                                      out=o, lse=lse),
                         args.steps, args.warmup, args.prewarm_ms)
    e = rate_entry(f5, dur, "TFLOP/s", PEAK_BF16_TFLOPS, 1e9)
    e.update({"flops": f5, "plan_host_ms": round(plan_ms, 4), "plan_items": int(plan.shape[0])})
    wl["varlen_window_planned"] = e
    return wl


def bench_bwd(fa, args, all_workloads):
    """Backward: prep + dK/dV + dQ kernels; algorithmic work = the five products of
    the chain rule (S, dP, dV, dK, dQ), 2.5x the forward."""
    wl = {}
    w2 = workloads.causal_mha()
    a = [t.cuda() for t in (w2.q, w2.k, w2.v)]
    do2 = workloads.upstream_grad(1002, tuple(w2.q.shape)).cuda()
    o2, l2 = fa.fa_fwd(*a, w2.scale, True)
    gq, gk, gv = torch.empty_like(a[0]), torch.empty_like(a[1]), torch.empty_like(a[2])
    ws2 = torch.empty(fa.fa_bwd_workspace_size(4, 32, 2048), dtype=torch.uint8, device="cuda")
    fb = 2.5 * dense_flops(w2)
    _, dur = timed_steps(lambda: fa.fa_bwd(*a, o2, l2, do2, w2.scale, True, dq=gq, dk=gk, dv=gv,
                                           workspace=ws2), max(20, args.steps // 4), args.warmup,
                         args.prewarm_ms)
    wl["bwd_causal_mha"] = rate_entry(fb, dur, "TFLOP/s", PEAK_BF16_TFLOPS, 1e9)
    wl["bwd_causal_mha"].update({"flops": fb, "kernels": "bwd_prep + bwd_dkdv + bwd_dq"})
    del a, do2, o2, l2, gq, gk, gv, ws2, w2
    torch.cuda.empty_cache()
    if not all_workloads:
        return wl
    w3 = workloads.causal_gqa_long()
    a = [t.cuda() for t in (w3.q, w3.k, w3.v)]
    do3 = workloads.upstream_grad(1003, tuple(w3.q.shape)).cuda()
    o3, l3 = fa.fa_fwd(*a, w3.scale, True)
    ws3 = torch.empty(fa.fa_bwd_workspace_size(1, 32, 16384), dtype=torch.uint8, device="cuda")
    g3 = [torch.empty_like(t) for t in a]
    fb3 = 2.5 * dense_flops(w3)
    _, dur = timed_steps(lambda: fa.fa_bwd(*a, o3, l3, do3, w3.scale, True, dq=g3[0], dk=g3[1],
                                           dv=g3[2], workspace=ws3), 10, 2, args.prewarm_ms)
    wl["bwd_causal_gqa_long"] = rate_entry(fb3, dur, "TFLOP/s", PEAK_BF16_TFLOPS, 1e9)
    wl["bwd_causal_gqa_long"]["flops"] = fb3
    del a, do3, o3, l3, ws3, g3, w3
    torch.cuda.empty_cache()
    w5 = workloads.varlen_window()
    a = [t.cuda() for t in (w5.q, w5.k, w5.v)]
    cu5 = torch.from_numpy(w5.cu_seqlens).cuda()
    do5 = workloads.upstream_grad(1005, tuple(w5.q.shape)).cuda()
    o5, l5 = fa.fa_fwd_varlen(*a, cu5, cu5, w5.max_seqlen, w5.max_seqlen, w5.scale, True,
                              w5.window)
    ws5 = torch.empty(fa.fa_bwd_varlen_workspace_size(len(w5.lens), 16, int(w5.cu_seqlens[-1])),
                      dtype=torch.uint8, device="cuda")
    g5 = [torch.empty_like(t) for t in a]
    fb5 = 2.5 * varlen_flops(w5)
    _, dur = timed_steps(lambda: fa.fa_bwd_varlen(*a, o5, l5, do5, cu5, cu5, w5.max_seqlen,
                                                  w5.max_seqlen, w5.scale, True, w5.window,
                                                  dq=g5[0], dk=g5[1], dv=g5[2], workspace=ws5),
                         max(20, args.steps // 4), args.warmup, args.prewarm_ms)
    wl["bwd_varlen_window"] = rate_entry(fb5, dur, "TFLOP/s", PEAK_BF16_TFLOPS, 1e9)
    wl["bwd_varlen_window"]["flops"] = fb5
    del a, cu5, do5, o5, l5, ws5, g5, w5
    torch.cuda.empty_cache()
    return wl


def bench_small_and_chunked(fa, args):
    wl = {}
    w1 = workloads.small_dense(Hkv=1)
    a = [t.cuda() for t in (w1.q, w1.k, w1.v)]
    _, dur = timed_steps(lambda: fa.fa_fwd(*a, w1.scale, False), args.steps, args.warmup,
                         args.prewarm_ms)
    st = stats(dur)
    wl["small_dense"] = {"ms": round(st["mean"], 4), "median_ms": round(st["median"], 4),
                         "TFLOP/s": round(dense_flops(w1) / st["mean"] / 1e9, 3)}
    del a
    w6 = workloads.chunked_prefill()
    q6, kc6, vc6 = w6.q.cuda(), w6.k_cache.cuda(), w6.v_cache.cuda()
    kn6, vn6 = w6.k_new.cuda(), w6.v_new.cuda()
    bt6 = torch.from_numpy(w6.block_table).cuda()
    sl6 = torch.from_numpy(w6.cache_seqlens).cuda()
    Lq6, Hq6, d6 = w6.q.shape[1], w6.q.shape[2], w6.q.shape[3]
    f6 = 4.0 * d6 * Hq6 * sum(visible_pairs(Lq6, int(n) + Lq6, True, -1, -1) for n in w6.cache_seqlens)
    # a step appends the chunk's K/V rows (same values each call) and attends over the cache
    _, dur = timed_steps(lambda: fa.fa_fwd_kvcache(q6, kc6, vc6, bt6, sl6, kn6, vn6, w6.scale, True),
                         args.steps, args.warmup, args.prewarm_ms)
    wl["chunked_prefill"] = rate_entry(f6, dur, "TFLOP/s", PEAK_BF16_TFLOPS, 1e9)
    wl["chunked_prefill"].update({"flops": f6, "kernels": "kvcache_append + prefill_fwd<paged>"})
    del q6, kc6, vc6, kn6, vn6, w6
    return wl


def bench_decode(fa, args, extras):
    """fa_decode_paged (the boundary call: no host plan) is the decode roofline;
    the planned run and the 64-query-head variant are reported beside it."""
    wl = {}
    w4 = workloads.paged_decode()
    qd, kc, vc = w4.q.cuda(), w4.k_cache.cuda(), w4.v_cache.cuda()
    bt = torch.from_numpy(w4.block_table).cuda()
    sl = torch.from_numpy(w4.seqlens).cuda()
    ws = torch.empty(fa.fa_decode_paged_workspace_size(64, 32, 128, bt.shape[1], 16, 512),
                     dtype=torch.uint8, device="cuda")
    od = torch.empty_like(qd)
    ld = torch.empty((64, 32), dtype=torch.float32, device="cuda")
    nb = decode_bytes(w4)
    kernels = "decode_split_heads<128,4,nt> (self-ordered) + decode_merge"
    _, dur = timed_steps(lambda: fa.fa_decode_paged(qd, kc, vc, bt, sl, w4.scale, -1, 512, out=od,
                                                    lse=ld, workspace=ws),
                         args.steps, args.warmup, args.prewarm_ms)
    wl["paged_decode"] = rate_entry(nb, dur, "GB/s", PEAK_HBM_GBS, 1e6)
    wl["paged_decode"].update({"bytes": nb, "kernels": kernels})
    roof = roofline_block("hbm", nb, dur, "GB/s", PEAK_HBM_GBS, 1e6,
                          load_traffic("decode_paged_traffic", DECODE_SRC), kernels)
    roof["workload"] = w4.name
    if extras:
        # plan / run split: the host plan lists only the (request, split) pairs that hold
        # keys, heaviest first; made once per batch composition, its host time is
        # reported beside the run (a decode loop remakes it whenever lengths change)
        t0 = time.perf_counter()
        plan = fa.fa_decode_plan(w4.seqlens, 16, bt.shape[1], -1, 512)
        plan_ms = (time.perf_counter() - t0) * 1e3
        plan_d = torch.from_numpy(plan).cuda()
        _, dur = timed_steps(lambda: fa.fa_decode_paged_run(qd, kc, vc, bt, sl, plan_d, w4.scale,
                                                            -1, 512, out=od, lse=ld, workspace=ws),
                             args.steps, args.warmup, args.prewarm_ms)
        e = rate_entry(nb, dur, "GB/s", PEAK_HBM_GBS, 1e6)
        e.update({"bytes": nb, "plan_host_ms": round(plan_ms, 4), "plan_items": int(plan.shape[0]),
                  "kernels": "decode_split_heads<128,4,nt> (planned) + decode_merge"})
        e["GB/s_with_host_plan"] = round(nb / (e["ms"] + plan_ms) / 1e6, 1)
        wl["paged_decode_planned"] = e
        # the same cache and plan with 64 query heads (8 per KV head: two-KV-head sets)
        q8 = workloads.device_normal(40, (64, 1, 64, 128))
        o8, l8 = torch.empty_like(q8), torch.empty((64, 64), dtype=torch.float32, device="cuda")
        ws8 = torch.empty(fa.fa_decode_paged_workspace_size(64, 64, 128, bt.shape[1], 16, 512),
                          dtype=torch.uint8, device="cuda")
        _, dur = timed_steps(lambda: fa.fa_decode_paged_run(q8, kc, vc, bt, sl, plan_d, w4.scale,
                                                            -1, 512, out=o8, lse=l8, workspace=ws8),
                             args.steps, args.warmup, args.prewarm_ms)
        nb8 = nb + 2 * 64 * 32 * 128 * 2 + 64 * 32 * 4     # q, o and lse of the 32 more heads
        e = rate_entry(nb8, dur, "GB/s", PEAK_HBM_GBS, 1e6)
        e.update({"bytes": nb8, "kernels": "decode_split_heads<128,2> (planned) + decode_merge"})
        wl["paged_decode_gqa8_planned"] = e
        del q8, o8, l8, ws8, plan_d
    del qd, kc, vc, w4
    torch.cuda.empty_cache()
    return wl, roof


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prewarm-ms", type=float, default=300.0,
                    help="untimed back-to-back calls before the warmup steps of each workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["main", "causal_mha", "varlen_window", "decode", "bwd"],
                    help="time one workload only (for profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain copy of known size (for byte-counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU sharding is a design note, not a measured path.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        print("bench.py: --steps must be at least 1", file=sys.stderr)
        sys.exit(2)

    import exact_attention_17_amd as fa
    fa.load_library()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    props = torch.cuda.get_device_properties(0)
    if args.copy_calibration:
        copy_calibration()

    result = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
              "data": "synthetic", "device": props.name, "prewarm_ms": args.prewarm_ms}
    only = args.only
    w3 = workloads.causal_gqa_long()
    flops3 = dense_flops(w3)
    wl = {}
    if only in (None, "main"):
        result.update(bench_main(fa, w3, flops3, args))
    if only in (None, "causal_mha"):
        wl["causal_mha"], result["roofline_causal_mha"] = bench_causal_mha(fa, args)
    if only in (None, "varlen_window"):
        wl.update(bench_varlen(fa, args))
    if only in (None, "decode"):
        dwl, result["roofline_decode"] = bench_decode(fa, args, extras=only is None)
        wl.update(dwl)
        if only is None:
            ctx = hbm_context()
            if "read_GB/s" in ctx:
                ctx["decode_vs_read"] = round(result["roofline_decode"]["achieved"] / ctx["read_GB/s"], 4)
            result["hbm_context"] = ctx
    if only in (None, "bwd"):
        wl.update(bench_bwd(fa, args, all_workloads=only is None))
    if only is None:
        wl.update(bench_small_and_chunked(fa, args))
    result["workloads"] = wl
    if not args.no_cpu_baseline and only in (None, "main"):
        result["cpu_baseline"] = cpu_baseline(w3, flops3, per_workload=only is None)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
