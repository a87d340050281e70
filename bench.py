"""Benchmark of the fused attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one fa_fwd call on the causal MHA prefill workload (B=4, H=32,
L=2048, d=128, bf16, seeded synthetic inputs resident in HBM).  The timed
region is exactly K steps bracketed by torch.cuda.synchronize(); `value` is
algorithmic TFLOP/s (4*d FLOPs per visible (query, key) pair per head).

Before the W warmup steps each workload runs untimed for --prewarm-ms of wall
time: the GPU raises its engine clock only after some milliseconds of
sustained load, and without this the first tens of milliseconds (the whole
timed region at small K) run at a lower clock.
The other workloads (long-context GQA prefill, paged decode, varlen window
prefill, the small dense case, and a chunk of 512 new tokens appended to and
attending over a paged cache) are timed in the same run and reported under
"workloads".  One JSON line is printed.

"roofline" covers the dominant kernel (the prefill kernel on the main
workload): achieved = algorithmic FLOPs per launch / the launch's average
duration from HIP events on the launch stream, against the bf16 dense MFMA
peak.  "traffic" comes from the committed rocprofv3 counter summary for that
kernel and is null if the kernel source changed since it was taken.
"cpu_baseline" times the CPU fp64 oracle on a bounded sample of the same
workload on this host.
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

import numpy as np  # noqa: E402
import torch  # noqa: E402

import workloads  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0              # MI355X HBM3E (published)
METRIC = "prefill attn TFLOP/s (% MFMA peak); paged-decode KV GB/s (% HBM peak)"
PREFILL_SRC = os.path.join(ROOT, "exact_attention_17_amd", "csrc", "prefill_fwd.hip")
DECODE_SRC = os.path.join(ROOT, "exact_attention_17_amd", "csrc", "decode_paged.hip")
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 512 << 20             # plain device copy used to calibrate the byte counters


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


def time_calls(fn, steps, warmup, prewarm_ms=0.0):
    """Average ms per call from HIP events recorded on the launch stream
    (torch's current stream, which the binding launches on)."""
    prewarm(fn, prewarm_ms)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


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


def cpu_baseline(w, flops_total):
    """Time the CPU fp64 oracle on a bounded sample of the workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = int(os.environ.get("OMP_NUM_THREADS", "1"))
    B, L, Hq, d = w.q.shape
    pairs = [(b, h) for b in range(B) for h in range(Hq)]     # the whole step (a few seconds)
    qb = w.q.contiguous().view(torch.int16).numpy().view(np.uint16)
    kb = w.k.contiguous().view(torch.int16).numpy().view(np.uint16)
    vb = w.v.contiguous().view(torch.int16).numpy().view(np.uint16)
    t0 = time.perf_counter()
    for b, h in pairs:
        oracle.attention_rows_ref(qb, kb, vb, b, h, np.arange(L), w.scale, w.causal, w.window)
    dt = time.perf_counter() - t0
    sample_flops = flops_total * len(pairs) / (B * Hq)
    return {"value": round(sample_flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores),
            "kind": "oracle", "seconds": round(dt, 2),
            "sample": f"all {len(pairs)} (batch, head) pairs of {w.name} (one whole step), all {L} "
                      "rows each, full S and P in float64 (numpy)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--prewarm-ms", type=float, default=300.0,
                    help="untimed back-to-back calls before the warmup steps of each workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-main", action="store_true", help="time only the main workload")
    ap.add_argument("--only-decode", action="store_true", help="time only the paged decode workload")
    ap.add_argument("--only-bwd", action="store_true", help="time only the backward workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain copy of known size (for byte-counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU sharding is a design note, not a measured path.", file=sys.stderr)
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
    w2 = workloads.causal_mha()
    flops2 = dense_flops(w2)
    if not args.only_decode and not args.only_bwd:
        result.update(bench_main(fa, w2, flops2, args))
    wl = {}
    if args.only_bwd:
        wl = bench_bwd(fa, args)
    elif not args.only_main:
        wl, roof_dec = bench_others(fa, args)
        result["roofline_decode"] = roof_dec
    result["workloads"] = wl
    if not args.no_cpu_baseline and not args.only_decode and not args.only_bwd:
        result["cpu_baseline"] = cpu_baseline(w2, flops2)
    print(json.dumps(result), flush=True)


def bench_main(fa, w2, flops2, args):
    """The contract step: K timed fa_fwd calls on the causal MHA workload."""
    q, k, v = w2.q.cuda(), w2.k.cuda(), w2.v.cuda()
    o = torch.empty_like(q)
    lse = torch.empty((4, 32, 2048), dtype=torch.float32, device="cuda")
    step = lambda: fa.fa_fwd(q, k, v, w2.scale, True, (-1, -1), out=o, lse=lse)
    prewarm(step, args.prewarm_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ev_ms = time_calls(step, args.steps, 2)
    value = flops2 / (wall_ms * 1e-3) / 1e12
    achieved = flops2 / (ev_ms * 1e-3) / 1e12
    traffic = load_traffic("prefill_fwd_causal_mha_traffic", PREFILL_SRC)
    return {
        "value": round(value, 2), "unit": "TFLOP/s", "ms_per_step": round(wall_ms, 4),
        "config": {"workload": w2.name, "B": 4, "Hq": 32, "Hkv": 32, "L": 2048, "d": 128,
                   "causal": True, "flops_per_step": flops2},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel": "prefill_fwd_kernel<128,false>",
                     "avg_launch_ms": round(ev_ms, 4)},
    }


def bench_bwd(fa, args):
    """Backward of the causal MHA workload: prep + dK/dV + dQ kernels; algorithmic
    work = the five products of the chain rule (S, dP, dV, dK, dQ), 2.5x the forward."""
    wl = {}
    w2 = workloads.causal_mha()
    a = [t.cuda() for t in (w2.q, w2.k, w2.v)]
    do2 = workloads.upstream_grad(1002, tuple(w2.q.shape)).cuda()
    o2, l2 = fa.fa_fwd(*a, w2.scale, True)
    gq, gk, gv = torch.empty_like(a[0]), torch.empty_like(a[1]), torch.empty_like(a[2])
    ws2 = torch.empty(fa.fa_bwd_workspace_size(4, 32, 2048), dtype=torch.uint8, device="cuda")
    fb = 2.5 * dense_flops(w2)
    ms = time_calls(lambda: fa.fa_bwd(*a, o2, l2, do2, w2.scale, True, dq=gq, dk=gk, dv=gv,
                                      workspace=ws2), max(20, args.steps // 4), args.warmup,
                    args.prewarm_ms)
    wl["bwd_causal_mha"] = {"ms": round(ms, 4), "TFLOP/s": round(fb / ms / 1e9, 2),
                            "frac_mfma": round(fb / ms / 1e9 / PEAK_BF16_TFLOPS, 4), "flops": fb,
                            "kernels": "bwd_prep + bwd_dkdv + bwd_dq"}
    del a, do2, o2, l2, gq, gk, gv, ws2, w2
    torch.cuda.empty_cache()
    if not args.only_bwd:
        # long-context GQA backward (B=1, Hq=32, Hkv=8, L=16384): dK, dV of a KV
        # head sum its 4 query heads inside one workgroup
        w3 = workloads.causal_gqa_long()
        a = [t.cuda() for t in (w3.q, w3.k, w3.v)]
        do3 = workloads.upstream_grad(1003, tuple(w3.q.shape)).cuda()
        o3, l3 = fa.fa_fwd(*a, w3.scale, True)
        ws3 = torch.empty(fa.fa_bwd_workspace_size(1, 32, 16384), dtype=torch.uint8, device="cuda")
        g3 = [torch.empty_like(t) for t in a]
        fb3 = 2.5 * dense_flops(w3)
        ms = time_calls(lambda: fa.fa_bwd(*a, o3, l3, do3, w3.scale, True, dq=g3[0], dk=g3[1],
                                          dv=g3[2], workspace=ws3), 5, 2, args.prewarm_ms)
        wl["bwd_causal_gqa_long"] = {"ms": round(ms, 4), "TFLOP/s": round(fb3 / ms / 1e9, 2),
                                     "frac_mfma": round(fb3 / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                                     "flops": fb3}
        del a, do3, o3, l3, ws3, g3, w3
        torch.cuda.empty_cache()
        # varlen + sliding-window backward (the varlen window workload, d = 64)
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
        ms = time_calls(lambda: fa.fa_bwd_varlen(*a, o5, l5, do5, cu5, cu5, w5.max_seqlen,
                                                 w5.max_seqlen, w5.scale, True, w5.window,
                                                 dq=g5[0], dk=g5[1], dv=g5[2], workspace=ws5),
                        max(20, args.steps // 4), args.warmup, args.prewarm_ms)
        wl["bwd_varlen_window"] = {"ms": round(ms, 4), "TFLOP/s": round(fb5 / ms / 1e9, 2),
                                   "frac_mfma": round(fb5 / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                                   "flops": fb5}
        del a, cu5, do5, o5, l5, ws5, g5, w5
        torch.cuda.empty_cache()
    return wl


def bench_others(fa, args):
    """Time the remaining workloads; returns (per-workload dict, decode roofline)."""
    wl = {}
    if not args.only_decode:
        w1 = workloads.small_dense(Hkv=1)
        a = [t.cuda() for t in (w1.q, w1.k, w1.v)]
        ms = time_calls(lambda: fa.fa_fwd(*a, w1.scale, False), args.steps, args.warmup, args.prewarm_ms)
        wl["small_dense"] = {"ms": round(ms, 4), "TFLOP/s": round(dense_flops(w1) / ms / 1e9, 3)}
        del a

        wl.update(bench_bwd(fa, args))

        w3 = workloads.causal_gqa_long()
        a = [t.cuda() for t in (w3.q, w3.k, w3.v)]
        f3 = dense_flops(w3)
        ms = time_calls(lambda: fa.fa_fwd(*a, w3.scale, True), max(5, args.steps // 10), 3, args.prewarm_ms)
        wl["causal_gqa_long"] = {"ms": round(ms, 4), "TFLOP/s": round(f3 / ms / 1e9, 2),
                                 "frac_mfma": round(f3 / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                                 "flops": f3}
        del a, w3

        w5 = workloads.varlen_window()
        a = [t.cuda() for t in (w5.q, w5.k, w5.v)]
        cu = torch.from_numpy(w5.cu_seqlens).cuda()
        f5 = varlen_flops(w5)
        ms = time_calls(lambda: fa.fa_fwd_varlen(*a, cu, cu, w5.max_seqlen, w5.max_seqlen, w5.scale,
                                                 True, w5.window), args.steps, args.warmup,
                        args.prewarm_ms)
        wl["varlen_window"] = {"ms": round(ms, 4), "TFLOP/s": round(f5 / ms / 1e9, 2),
                               "frac_mfma": round(f5 / ms / 1e9 / PEAK_BF16_TFLOPS, 4), "flops": f5}
        # plan / run split: the host plan (heaviest tiles first) is made once for the
        # batch's lengths and reused; its host time is reported beside the run
        t0 = time.perf_counter()
        plan = fa.fa_varlen_plan(w5.cu_seqlens, w5.cu_seqlens, True, w5.window)
        plan_ms = (time.perf_counter() - t0) * 1e3
        plan_d = torch.from_numpy(plan).cuda()
        ms = time_calls(lambda: fa.fa_fwd_varlen_run(*a, cu, cu, plan_d, w5.max_seqlen,
                                                     w5.max_seqlen, w5.scale, True, w5.window),
                        args.steps, args.warmup, args.prewarm_ms)
        wl["varlen_window_planned"] = {"ms": round(ms, 4), "TFLOP/s": round(f5 / ms / 1e9, 2),
                                       "frac_mfma": round(f5 / ms / 1e9 / PEAK_BF16_TFLOPS, 4),
                                       "flops": f5, "plan_host_ms": round(plan_ms, 4),
                                       "plan_items": int(plan.shape[0])}
        del a, w5, plan_d

        w6 = workloads.chunked_prefill()
        q6, kc6, vc6 = w6.q.cuda(), w6.k_cache.cuda(), w6.v_cache.cuda()
        kn6, vn6 = w6.k_new.cuda(), w6.v_new.cuda()
        bt6 = torch.from_numpy(w6.block_table).cuda()
        sl6 = torch.from_numpy(w6.cache_seqlens).cuda()
        Lq6, Hq6, d6 = w6.q.shape[1], w6.q.shape[2], w6.q.shape[3]
        f6 = 4.0 * d6 * Hq6 * sum(visible_pairs(Lq6, int(n) + Lq6, True, -1, -1) for n in w6.cache_seqlens)
        # a step appends the chunk's K/V rows (same values each call) and attends over the cache
        ms = time_calls(lambda: fa.fa_fwd_kvcache(q6, kc6, vc6, bt6, sl6, kn6, vn6, w6.scale, True),
                        args.steps, args.warmup, args.prewarm_ms)
        wl["chunked_prefill"] = {"ms": round(ms, 4), "TFLOP/s": round(f6 / ms / 1e9, 2),
                                 "frac_mfma": round(f6 / ms / 1e9 / PEAK_BF16_TFLOPS, 4), "flops": f6,
                                 "kernels": "kvcache_append + prefill_fwd<paged>"}
        del q6, kc6, vc6, kn6, vn6, w6

    w4 = workloads.paged_decode()
    qd, kc, vc = w4.q.cuda(), w4.k_cache.cuda(), w4.v_cache.cuda()
    bt = torch.from_numpy(w4.block_table).cuda()
    sl = torch.from_numpy(w4.seqlens).cuda()
    ws = torch.empty(fa.fa_decode_paged_workspace_size(64, 32, 128, bt.shape[1], 16, 512),
                     dtype=torch.uint8, device="cuda")
    od = torch.empty_like(qd)
    ld = torch.empty((64, 32), dtype=torch.float32, device="cuda")
    nb = decode_bytes(w4)
    if not args.only_decode:
        # every (split slot, request) launched; slots past a request's length exit at once
        ms = time_calls(lambda: fa.fa_decode_paged(qd, kc, vc, bt, sl, w4.scale, -1, 512, out=od,
                                                   lse=ld, workspace=ws), args.steps,
                        args.warmup, args.prewarm_ms)
        gbs = nb / ms / 1e6
        wl["paged_decode"] = {"ms": round(ms, 4), "GB/s": round(gbs, 1),
                              "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "bytes": nb,
                              "kernels": "decode_order + decode_split_heads<128,4,nt> (device-made order) + decode_merge"}
    # plan / run split: the host plan lists only the (request, split) pairs that hold
    # keys, heaviest first; it is made once for the batch's lengths and its host time
    # is reported beside the run.  The decode roofline is this run's.
    t0 = time.perf_counter()
    plan = fa.fa_decode_plan(w4.seqlens, 16, bt.shape[1], -1, 512)
    plan_ms = (time.perf_counter() - t0) * 1e3
    plan_d = torch.from_numpy(plan).cuda()
    ms = time_calls(lambda: fa.fa_decode_paged_run(qd, kc, vc, bt, sl, plan_d, w4.scale, -1, 512,
                                                   out=od, lse=ld, workspace=ws),
                    args.steps, args.warmup, args.prewarm_ms)
    gbs = nb / ms / 1e6
    wl["paged_decode_planned"] = {"ms": round(ms, 4), "GB/s": round(gbs, 1),
                                  "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "bytes": nb,
                                  "plan_host_ms": round(plan_ms, 4),
                                  "plan_items": int(plan.shape[0]),
                                  "kernels": "decode_split_heads<128,4,nt> (planned) + decode_merge"}
    roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": load_traffic("decode_paged_traffic", DECODE_SRC),
            "kernel": "decode_split_heads<128,4,nt> (planned) + decode_merge", "avg_launch_ms": round(ms, 4)}
    if not args.only_decode:
        # the same cache and plan with 64 query heads (8 per KV head: two-KV-head sets);
        # not a bench line of its own, reported beside it
        q8 = workloads.device_normal(40, (64, 1, 64, 128))
        o8, l8 = torch.empty_like(q8), torch.empty((64, 64), dtype=torch.float32, device="cuda")
        ws8 = torch.empty(fa.fa_decode_paged_workspace_size(64, 64, 128, bt.shape[1], 16, 512),
                          dtype=torch.uint8, device="cuda")
        ms8 = time_calls(lambda: fa.fa_decode_paged_run(q8, kc, vc, bt, sl, plan_d, w4.scale, -1, 512,
                                                        out=o8, lse=l8, workspace=ws8),
                         args.steps, args.warmup, args.prewarm_ms)
        nb8 = nb + 2 * 64 * 32 * 128 * 2 + 64 * 32 * 4     # q, o and lse of the 32 more heads
        gbs8 = nb8 / ms8 / 1e6
        wl["paged_decode_gqa8_planned"] = {"ms": round(ms8, 4), "GB/s": round(gbs8, 1),
                                           "frac_hbm": round(gbs8 / PEAK_HBM_GBS, 4), "bytes": nb8,
                                           "kernels": "decode_split_heads<128,2> (planned) + decode_merge"}
        del q8, o8, l8, ws8
    del qd, kc, vc, w4, plan_d
    torch.cuda.empty_cache()
    return wl, roof


if __name__ == "__main__":
    main()
