#!/usr/bin/env python3
"""Benchmark of the WildCat forward (coreset selection + weights + attention) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long128k] [--bins B]
                    [--pivot-block b]

A step is one whole forward (randomly pivoted Cholesky, Nystroem weights, attention over the
coreset) over every head of one batch of seeded synthetic inputs that are already resident
in HBM.  The default workload is the long-context one (8 heads, n = m = 131072, d = dv = 128,
r = 2048, bf16), run as the method is stated: one bin, one pivot per step.  The other
workloads of coreset_head_rpcholesky_amd.synth can be selected with --workload.  Prints one
JSON line.

Beside the GPU number it reports:
  * roofline: the dominant kernel, its algorithmic bytes (or flops) over its measured time,
    timed with HIP events on the stream the kernels are launched on (the streaming pivot
    loop for every workload but the small-head one, whose whole forward is one kernel);
  * roofline_attend: the attention pass (wc_attend) against the bf16 matrix-core peak;
  * variants: the divide-and-conquer and block-pivot forwards of the same inputs, timed in
    the same run;
  * cpu_baseline: the fp64 CPU oracle timed on a bounded sample of the same workload, and a
    one-thread run of it on the image-shaped workload;
  * exact softmax attention (PyTorch SDPA) on the same tensors, for context;
  * attainable: what this GPU sustains on the operations that bound the hot path (an HBM read
    stream, a copy, bf16 and fp32 matrix-core chains, and the clock under the bf16 load), from
    the library's calibration kernels, with each roofline's fraction of it beside the fraction
    of the datasheet peak.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "WildCat forward tokens/sec (coreset+weights+attend); % HBM/MFMA roofline"
FP32_PEAK_TFLOPS = 157.3  # MI355X fp32, vector and matrix, published
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0

# Kernel sources a stored counter summary belongs to.
KERNEL_SOURCES = {
    "resident": ["wc_resident.hip", "wc_device.h", "wc_kernels.h"],
    "stream": ["wc_stream.hip", "wc_device.h", "wc_kernels.h"],
    "attend": ["wc_attend.hip", "wc_device.h", "wc_kernels.h"],
}
# (workload, kernel kind) -> committed rocprofv3 counter summary
COUNTER_FILES = {
    ("vit197", "resident"): "profiles/resident_kernel_vit197_counters.txt",
    ("long128k", "stream"): "profiles/rpc_step_kernel_long128k_counters.txt",
    ("kv32k", "stream"): "profiles/rpc_step_kernel_kv32k_counters.txt",
    ("img4096", "stream"): "profiles/rpc_step_kernel_img4096_counters.txt",
    ("long128k", "attend"): "profiles/attend_bf16_kernel_long128k_counters.txt",
}
# Binned and block-pivot forwards timed beside the default one: (bins, pivot_block)
DEFAULT_VARIANTS = {
    "long128k": [(16, 1), (64, 1), (64, 32), (1, 64)],
    "kv32k": [(16, 1), (64, 1), (16, 64)],
    "img4096": [(4, 1), (16, 1), (4, 64)],
}


_T0 = time.perf_counter()


def log(msg: str) -> None:
    """Progress line on stderr (the JSON result alone goes to stdout)."""
    print(f"[bench {time.perf_counter() - _T0:7.1f}s] {msg}", file=sys.stderr, flush=True)


def source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "coreset_head_rpcholesky_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_counters(workload: str, kind: str):
    """key = value pairs of the committed rocprofv3 counter summary for this workload and
    kernel, or None when there is none or the kernel source changed since it was taken."""
    path = COUNTER_FILES.get((workload, kind))
    if not path or not os.path.exists(os.path.join(ROOT, path)):
        return None
    vals = {}
    for line in open(os.path.join(ROOT, path)):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha") != source_hash(kind):
        return None
    return vals


def stored_float(vals, key):
    try:
        return float(vals[key]) if vals else None
    except (KeyError, ValueError):
        return None


def workload_accounting(w, bins: int = 1):
    """Algorithmic bytes and flops of one forward over all heads (per-head figures x heads).
    With bins, the pivot loop and the weights run on heads x bins sub-heads of n/bins keys
    and r/bins pivots; the attention still covers all r coreset rows per head."""
    b = 2 if w.dtype == "bf16" else 4
    H, n, m, d, dv, r = w.heads, w.n, w.m, w.d, w.dv, w.r
    compulsory = H * ((m * d + n * d + n * dv) * b + m * dv * b)
    Hs, ns, rs = H * bins, n // bins, r // bins
    # per step t: K re-read (n d b), F columns 0..t-1 (4 n t), residual read and written and
    # the new column written (12 n); summed over the r steps
    pivot_bytes = Hs * (ns * rs * d * b + 2 * ns * rs * (rs - 1) + 12 * ns * rs)
    # a sub-head small enough for the resident kernel keeps its factor on chip: only K in
    # and F, pivots out reach HBM
    pivot_resident_bytes = Hs * (ns * d * b + 4 * ns * rs + 4 * rs)
    pivot_flops = Hs * (2 * ns * rs * d + ns * rs * (rs - 1))
    weight_flops = Hs * (2 * rs * ns * (dv + 1) + rs * rs * (dv + 1))
    attend_flops = H * 2 * m * r * (d + dv + 1)
    return dict(compulsory_bytes=compulsory, pivot_bytes=pivot_bytes,
                pivot_resident_bytes=pivot_resident_bytes, pivot_flops=pivot_flops,
                weight_flops=weight_flops, attend_flops=attend_flops)


def graph_of(fn, copies: int = 1):
    """fn() (which launches on the current stream) captured `copies` times in one HIP graph."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for _ in range(copies):
                fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return g


def time_replays(g, reps: int, stream) -> float:
    """Mean ms per replay of graph g: one untimed warm replay, then `reps` timed ones, HIP
    events on the stream the replays run on."""
    import torch

    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def exact_attention_timing(w, Q, K, V, stream):
    """Exact softmax attention on the same tensors with PyTorch SDPA ([1, heads, len, d] so
    the fused backends are eligible); the first backend that runs is recorded."""
    import torch
    import torch.nn.functional as Fn
    from torch.nn.attention import SDPBackend, sdpa_kernel

    q, k, v = Q.unsqueeze(0), K.unsqueeze(0), V.unsqueeze(0)
    err = ""
    for name, backend in [("flash", SDPBackend.FLASH_ATTENTION),
                          ("efficient", SDPBackend.EFFICIENT_ATTENTION),
                          ("math", SDPBackend.MATH)]:
        try:
            with sdpa_kernel([backend]):
                for _ in range(2):
                    Fn.scaled_dot_product_attention(q, k, v)
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                reps = 5
                e0.record(stream)
                for _ in range(reps):
                    Fn.scaled_dot_product_attention(q, k, v)
                e1.record(stream)
                torch.cuda.synchronize()
            ems = e0.elapsed_time(e1) / reps
            return {"ms_per_step": round(ems, 4), "tokens_per_s": round(w.tokens / (ems / 1e3), 1),
                    "op": f"torch.nn.functional.scaled_dot_product_attention ({name} backend)"}
        except Exception as e:  # noqa: BLE001 - try the next backend
            err = str(e)[:160]
            torch.cuda.synchronize()
    return {"error": err}


def error_vs_exact(w, Q, K, V, O, rows: int = 256):
    """Relative Frobenius error of the WildCat output against exact softmax attention (fp32,
    on the GPU) over up to `rows` evenly spaced queries per head, the mean over heads."""
    import torch

    idx = torch.linspace(0, w.m - 1, min(rows, w.m), device=Q.device).round().long().unique()
    q = Q[:, idx].float().unsqueeze(0)
    ex = torch.nn.functional.scaled_dot_product_attention(q, K.float().unsqueeze(0), V.float().unsqueeze(0))[0]
    got = O[:, idx].float()
    err = torch.linalg.vector_norm(got - ex, dim=(1, 2)) / torch.linalg.vector_norm(ex, dim=(1, 2))
    return round(float(err.mean()), 6)


def _blas_threads():
    """Threads the BLAS pools actually use (the largest pool), from threadpoolctl."""
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return 1


def _oracle_head(ow, philox, w, Q, K, V, h, bins, pivot_block):
    """One head of the oracle forward with the bench's Philox uniforms (seed 42); returns the
    rank it reached."""
    import numpy as np

    if bins > 1 or pivot_block > 1:
        rb = w.r // bins
        per = ow.BLOCK_DRAWS * rb if pivot_block > 1 else rb
        # each bin (sub-head h B + b) draws its own Philox stream, as the device does
        u = np.concatenate([philox.pivot_uniforms(42, h * bins + b, per) for b in range(bins)])
        out = ow.forward_binned(Q[h], K[h], V[h], w.r, bins, u, pivot_block=pivot_block)
    else:
        out = ow.forward(Q[h], K[h], V[h], w.r, np.array(philox.pivot_uniforms(42, h, w.r)))
    return int(out["rank"])


def cpu_baseline(w, Q, K, V, budget_s: float, bins: int = 1, pivot_block: int = 1, threads=None):
    """The fp64 oracle on as many heads as fit in the time budget (at least one), going round
    the workload's heads again when one pass takes less; tokens/s scaled to the whole workload
    (tokens per head = tokens / heads).  threads: BLAS threads (None: the pools' default,
    which follows OMP_NUM_THREADS)."""
    from oracle import philox
    from oracle import wildcat as ow

    limiter = None
    if threads is not None:
        try:
            from threadpoolctl import threadpool_limits
            limiter = threadpool_limits(threads)
        except Exception:  # pragma: no cover
            limiter = None
    cores = _blas_threads()
    t0 = time.perf_counter()
    done, ranks = 0, []
    while True:
        h = done % min(w.heads, Q.shape[0])
        ranks.append(_oracle_head(ow, philox, w, Q, K, V, h, bins, pivot_block))
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.unregister()
    tokens = w.tokens * done / w.heads
    what = (f"{done} of {w.heads} heads of one {w.name} forward" if done <= w.heads else
            f"{done} heads ({done / w.heads:.1f} passes over the {w.heads} heads of a {w.name} forward)")
    extrap = (f"; tokens/s = {w.tokens // w.heads} tokens per head x {done} heads / {dt:.1f} s, i.e. the "
              f"whole {w.heads}-head forward extrapolated as {w.heads / done:.2f} x the measured time"
              if done < w.heads else "")
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{what}{f' with {bins} bins' if bins > 1 else ''}"
                      f"{f', {pivot_block} candidates per round' if pivot_block > 1 else ''}, fp64 numpy/scipy, "
                      f"{dt:.1f} s{extrap}",
            "oracle_rank_min": int(min(ranks)),
            "host_cpu_count": os.cpu_count(),
            "host_cpus_in_affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def run_decode(args, w, Q, K, V, dt_t, dev):
    """COMPRESSKV measurement: compress the workload's keys and values into a cache once, then
    time decode steps over it (queries_per_head queries per head per step, the first ones of
    the workload), beside exact decode attention over the full key/value cache (SDPA)."""
    import torch

    from coreset_head_rpcholesky_amd import binding

    bins = max(1, args.bins)
    m = max(1, min(args.decode_queries, w.m))
    rows = w.r
    Qd = Q[:, :m].contiguous()
    stream = torch.cuda.current_stream()
    pb = max(1, args.pivot_block)
    p = binding.problem(w.heads, w.n, m, w.d, w.dv, w.r, dt_t, bins, 0, pb)
    ws = binding.workspace(p, dev)
    cache = torch.empty(binding.wc_cache_bytes(p, rows), dtype=torch.uint8, device=dev)
    dws = torch.empty(max(binding.wc_decode_workspace_bytes(p, rows), 256), dtype=torch.uint8, device=dev)
    O = torch.empty((w.heads, m, w.dv), dtype=dt_t, device=dev)
    flags = torch.zeros((w.heads,), dtype=torch.int32, device=dev)

    def compress():
        return binding.wc_compress(K, V, w.r, rows, seed=args.seed, bins=bins, pivot_block=pb, cache=cache, ws=ws)

    def decode():
        binding.wc_decode(Qd, cache, rows, rows, w.dv, flags=flags, ws=dws, out=O)

    def timed(fn, reps, per_graph):
        fn()
        torch.cuda.synchronize()
        return time_replays(graph_of(fn, per_graph), reps, stream) / per_graph

    compress_ms = timed(compress, 3, 1)
    c = compress()
    torch.cuda.synchronize()
    per = 10
    ms = timed(decode, max(1, args.steps // per), per)
    decode()
    torch.cuda.synchronize()
    # exact decode attention over the full cache
    q, k, v = Qd.unsqueeze(0), K.unsqueeze(0), V.unsqueeze(0)
    ex = torch.nn.functional.scaled_dot_product_attention(q.float(), k.float(), v.float())[0]
    err = torch.linalg.vector_norm(O.float() - ex, dim=(1, 2)) / torch.linalg.vector_norm(ex, dim=(1, 2))

    def sdpa():
        torch.nn.functional.scaled_dot_product_attention(q, k, v)

    exact_ms = timed(sdpa, max(1, args.steps // per), per)
    esz = 2 if w.dtype == "bf16" else 4
    # bytes one decode step must move: the cache rows (keys, weights and the bf16 normaliser
    # column; hi and lo parts for fp32), the queries and the outputs
    row_bytes = (w.d + w.dv) * 2 * (1 if w.dtype == "bf16" else 2) + 2
    step_bytes = w.heads * (rows * row_bytes + m * (w.d + w.dv) * esz)
    achieved = step_bytes / (ms / 1e3) / 1e9
    exact_bytes = w.heads * (w.n * (w.d + w.dv) * esz + m * (w.d + w.dv) * esz)
    line = {
        "metric": "WildCat COMPRESSKV decode queries/sec over the compressed cache",
        "value": round(w.heads * m / (ms / 1e3), 1), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "heads": w.heads, "prefix_keys": w.n, "cache_rows": rows,
                   "d": w.d, "dv": w.dv, "bins": bins, "pivot_block": pb, "queries_per_head": m,
                   "pivot_uniforms": f"Philox4x64-10 seed {args.seed}"},
        "roofline": {"kernel": "attend kernels over the cache (decode step)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_step": step_bytes},
        "compress_ms": round(compress_ms, 4),
        "cache_bytes": int(cache.numel()),
        "full_kv_bytes": int(w.heads * w.n * (w.d + w.dv) * esz),
        "exact_decode": {"ms_per_step": round(exact_ms, 5), "bytes_per_step": exact_bytes,
                         "op": "torch.nn.functional.scaled_dot_product_attention over the full cache"},
        "rel_err_vs_exact": round(float(err.mean()), 6),
        "checks": {"rank_min": int(c["rank"].min()), "flags_max": int(c["flags"].max())},
    }
    print(json.dumps(line), flush=True)


def pivot_loop_roofline(w, K, dt_t, dev, seed, bins, pb, stream, acc, reps):
    """The selection loop alone (wc_rpcholesky on the per-bin view, graph-replayed, warm),
    against HBM (one pivot per step: the streaming step kernel, or the resident kernel's loop)
    or against the bf16 / fp32 matrix-core mix (block pivots)."""
    from coreset_head_rpcholesky_amd import binding

    Ksel = K.view(w.heads * bins, w.n // bins, w.d)
    pws = binding.workspace(binding.problem(w.heads * bins, w.n // bins, 0, w.d, w.dv, w.r // bins, dt_t,
                                            1, 0, pb), dev)
    res = {}

    def rpc():
        res["out"] = binding.wc_rpcholesky(Ksel, w.r // bins, seed=seed, ws=pws, with_diag=False,
                                           with_trace=False, pivot_block=pb)

    rpc()
    loop_ms = time_replays(graph_of(rpc), reps, stream)
    Hs, ns, rs = w.heads * bins, w.n // bins, w.r // bins
    sub_resident = w.dtype == "bf16" and ns <= 256 and rs <= 32 and pb == 1
    if pb > 1:
        name = (f"block pivot selection, {rs // pb} rounds of {pb} candidates"
                f"{f', {Hs} bins' if bins > 1 else ''} (candidate columns: kernel part on "
                f"bf16 MFMA, factor part on fp32 MFMA; factor update fp32 vector)")
        # kernel part K K_S^T on the bf16 matrix cores; factor part F F_S^T and the update
        # F_new = G M^T in fp32 (matrix cores and vector units share the 157.3 TFLOP/s peak).
        # The roofline of the mix: the time both parts would take at their own peaks.
        kflops = Hs * 2 * ns * rs * w.d
        fflops = Hs * (ns * rs * (rs - pb) + 2 * ns * pb * rs)
        flops = kflops + fflops
        ideal_s = kflops / (MFMA_BF16_PEAK_TFLOPS * 1e12) + fflops / (FP32_PEAK_TFLOPS * 1e12)
        peak = flops / ideal_s / 1e12
        achieved = flops / (loop_ms / 1e3) / 1e12
        roof = {"kernel": name, "bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1),
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                "peak_of_mix": f"bf16 {MFMA_BF16_PEAK_TFLOPS} for {kflops} flops, fp32 {FP32_PEAK_TFLOPS} for {fflops}",
                "algorithmic_flops_per_loop": flops, "rounds": rs // pb, "loop_ms": round(loop_ms, 3)}
        return roof, res["out"]
    if sub_resident:
        name = f"resident_kernel (pivot loop only, {Hs} sub-heads, factor on chip)"
        loop_bytes, traffic = acc["pivot_resident_bytes"], None
    else:
        name = (f"rpc_step_kernel x {rs} launches (streaming pivot loop, one launch per pivot step over "
                f"all {Hs} {'bins' if bins > 1 else 'heads'})")
        loop_bytes = acc["pivot_bytes"]
        traffic = stored_float(stored_counters(w.name, "stream"), "traffic_bytes_per_loop") if bins == 1 else None
    achieved = loop_bytes / (loop_ms / 1e3) / 1e9
    roof = {"kernel": name, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "unit_of_work": f"one pivot loop: {rs} step launches (plus the initial-residual and bookkeeping "
                            f"kernels, timed with it)",
            "algorithmic_bytes_per_loop": loop_bytes, "loop_ms": round(loop_ms, 3),
            "launches": rs, "avg_launch_ms": round(loop_ms / rs, 5)}
    return roof, res["out"]


def attend_roofline(w, Q, K, V, rpc, stream, acc, reps):
    """The attention pass alone (wc_attend: coreset staging plus the matrix-core kernel) on the
    pivots of the selection loop and their weights, graph-replayed, against the bf16 peak."""
    from coreset_head_rpcholesky_amd import binding

    import torch

    W = binding.wc_weights(V, rpc["pivots"], rpc["rank"], rpc["F"])
    p = binding.problem(w.heads, w.n, w.m, w.d, w.dv, w.r, Q.dtype)
    ws = binding.workspace(p, Q.device)
    flags = torch.zeros((w.heads,), dtype=torch.int32, device=Q.device)
    O = torch.empty((w.heads, w.m, w.dv), dtype=Q.dtype, device=Q.device)

    def att():
        binding.wc_attend(Q, K, rpc["pivots"], rpc["rank"], W, flags=flags, ws=ws, out=O)

    att()
    # ten calls to a graph, so the replay's own start-up is spread over them
    ms = time_replays(graph_of(att, 10), max(1, reps // 5), stream) / 10
    flops = acc["attend_flops"]
    achieved = flops / (ms / 1e3) / 1e12
    cnt = stored_counters(w.name, "attend")
    roof = {"kernel": "wc_attend: attend_prep_kernel (coreset staging) + attend_bf16_kernel (bf16 MFMA)",
            "bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
            "algorithmic_flops_per_launch": flops, "avg_launch_ms": round(ms, 5),
            "flops_formula": "2 m r (d + dv + 1) per head"}
    if cnt:
        roof["counters"] = {k: cnt[k] for k in ("mfma_busy_frac", "mfma_flops_per_launch", "sclk_ghz")
                            if k in cnt}
    return roof, W


def attainable(dev, stream) -> dict:
    """Rates this GPU sustains on the operations that bound the hot path's kernels
    (wc_calibrate), each the mean of several launches timed with HIP events on `stream`:
    a 4 GiB read stream, a 2 GiB copy (read + write bytes), bf16 and fp32 MFMA chains on
    register operands (two waves per SIMD), and the shader clock under the bf16 chains."""
    import torch

    from coreset_head_rpcholesky_amd import binding as b

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    res = torch.empty(b.WC_CAL_RESULT_BYTES, dtype=torch.uint8, device=dev)
    nb = 4 << 30
    buf = torch.full((nb,), 0x5A, dtype=torch.uint8, device=dev)
    read_ms = timed(lambda: b.wc_calibrate(b.WC_CAL_READ, res, src=buf, nbytes=nb, stream=stream), 10)
    half = nb // 2
    src, dst = buf[:half], buf[half:]
    copy_ms = timed(lambda: b.wc_calibrate(b.WC_CAL_COPY, dst, src=src, nbytes=half, stream=stream), 10)
    del buf, src, dst
    clocks = torch.zeros(4, dtype=torch.int64, device=dev)
    waves = 512 * 4
    it16, it32 = 80000, 40000
    bf16_ms = timed(lambda: b.wc_calibrate(b.WC_CAL_MFMA_BF16, res, iters=it16, clocks=clocks, stream=stream), 3)
    c = clocks.cpu().tolist()
    sclk = (c[2] - c[0]) / (c[3] - c[1]) * 0.1 if c[3] > c[1] else None  # reference clock 100 MHz
    f32_ms = timed(lambda: b.wc_calibrate(b.WC_CAL_MFMA_F32, res, iters=it32, stream=stream), 3)
    torch.cuda.empty_cache()
    return {"kernels": "wc_calibrate (READ, COPY, MFMA_BF16, MFMA_F32)",
            "hbm_read_GBps": round(nb / (read_ms / 1e3) / 1e9, 1),
            "hbm_copy_GBps": round(2 * half / (copy_ms / 1e3) / 1e9, 1),
            "mfma_bf16_TFLOPs": round(waves * it16 * 8 * 32768 / (bf16_ms / 1e3) / 1e12, 1),
            "mfma_f32_TFLOPs": round(waves * it32 * 8 * 4096 / (f32_ms / 1e3) / 1e12, 2),
            "sclk_GHz_under_bf16_mfma": round(sclk, 3) if sclk else None,
            "datasheet": {"hbm_GBps": HBM_PEAK_GBS, "mfma_bf16_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                          "mfma_f32_TFLOPs": 157.3, "sclk_GHz": 2.4}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long128k")
    ap.add_argument("--seed", type=int, default=42)
    ap.add_argument("--bins", type=int, default=1,
                    help="divide-and-conquer selection with this many bins (must divide n and r)")
    ap.add_argument("--pivot-block", type=int, default=1,
                    help="block pivot selection: 16, 32 or 64 candidates per round (1: one pivot per step)")
    ap.add_argument("--variants", default=None,
                    help="extra forwards timed in the same run, 'B:b,B:b' (bins:pivot_block); 'none' for none")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work (at least one head)")
    ap.add_argument("--cpu-1core-workload", default="img4096",
                    help="workload of the one-thread oracle run ('none' to skip)")
    ap.add_argument("--cpu-1core-budget", type=float, default=8.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-exact", action="store_true")
    ap.add_argument("--no-roofline", action="store_true", help="skip the separate loop and attention timings")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--decode", action="store_true",
                    help="COMPRESSKV: compress the workload once, then time decode steps over the cache")
    ap.add_argument("--decode-queries", type=int, default=1, help="queries per head per decode step")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="run a plain copy kernel of this size first (for counter scaling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py measures one GPU: every head is independent, so "
                          "more GPUs would shard heads with no communication; only --gpus 1 "
                          "is measured"}))
        sys.exit(2)

    import numpy as np
    import torch

    from coreset_head_rpcholesky_amd import binding, synth

    w = synth.WORKLOADS[args.workload]
    dt_t = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    Qn, Kn, Vn = synth.make_inputs(w.name)

    def up(x):
        return torch.from_numpy(x).to(dev, dt_t).contiguous()

    Q, K, V = up(Qn), up(Kn), up(Vn)
    log(f"inputs of {w.name} resident on the GPU")
    if args.decode:
        run_decode(args, w, Q, K, V, dt_t, dev)
        return
    bins = max(1, args.bins)
    pb = max(1, args.pivot_block)
    p = binding.problem(w.heads, w.n, w.m, w.d, w.dv, w.r, dt_t, bins, 0, pb)
    ws = binding.workspace(p, dev)
    out = dict(O=torch.empty((w.heads, w.m, w.dv), dtype=dt_t, device=dev),
               pivots=torch.empty((w.heads, w.r), dtype=torch.int32, device=dev),
               rank=torch.empty((w.heads,), dtype=torch.int32, device=dev),
               flags=torch.empty((w.heads,), dtype=torch.int32, device=dev))

    if args.copy_calibration_mb > 0:
        nel = args.copy_calibration_mb * (1 << 20) // 4
        src = torch.ones(nel, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    stream = torch.cuda.current_stream()

    def fwd():
        binding.wc_forward(Q, K, V, w.r, seed=args.seed, bins=bins, pivot_block=pb, ws=ws, out=out)

    # One forward is captured in a HIP graph and replayed, so the host-side launch path
    # (Python, ctypes, one launch per pivot step on the streaming path) is not what is timed.
    # Short forwards are captured several to a graph, so the replays' own launch gaps are
    # amortised and back-to-back forwards run as they would inside a model.
    fwd()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    fwd()
    torch.cuda.synchronize()
    once_ms = (time.perf_counter() - t0) * 1e3
    log(f"two forwards done ({once_ms:.1f} ms the second)")
    graph = None
    per_replay = 1
    if not args.no_graph:
        want = max(1, min(10, int(10.0 / max(once_ms, 1e-3))))
        per_replay = max(d for d in range(1, want + 1) if args.steps % d == 0)
        graph = graph_of(fwd, per_replay)

    def launch():
        if graph is not None:
            graph.replay()
        else:
            fwd()

    nlaunch = args.steps // per_replay
    for _ in range(max(1, args.warmup // per_replay)):
        launch()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nlaunch + 1)]
    wall0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(nlaunch):
        launch()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    log(f"{args.steps} timed forwards done")
    per = [evs[i].elapsed_time(evs[i + 1]) / per_replay for i in range(nlaunch)]
    ms = evs[0].elapsed_time(evs[nlaunch]) / args.steps
    value = w.tokens / (ms / 1e3)
    rank = out["rank"].cpu().numpy()
    flags = out["flags"].cpu().numpy()

    acc = workload_accounting(w, bins)
    resident = w.dtype == "bf16" and w.n <= 256 and w.r <= 32 and bins == 1 and pb == 1
    roof_att = None
    reps = 2 if once_ms > 200 else 10
    if resident:
        # one launch per step: the resident kernel; only compulsory bytes reach HBM
        kernel_ms = float(np.mean(per))
        achieved = acc["compulsory_bytes"] / (kernel_ms / 1e3) / 1e9
        traffic = stored_float(stored_counters(w.name, "resident"), "traffic_bytes_per_launch")
        roof = {"kernel": "resident_kernel (pivot loop + weights + attention, one workgroup per head)",
                "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": acc["compulsory_bytes"],
                "avg_launch_ms": round(kernel_ms, 5)}
    elif args.no_roofline:
        roof = None
    else:
        roof, rpc = pivot_loop_roofline(w, K, dt_t, dev, args.seed, bins, pb, stream, acc, reps)
        if bins == 1 and w.m > 0:
            roof_att, _ = attend_roofline(w, Q, K, V, rpc, stream, acc, max(reps, 10))
        del rpc
        torch.cuda.empty_cache()

    log("rooflines done")
    exact = None
    if not args.no_exact:
        exact = exact_attention_timing(w, Q, K, V, stream)
        exact["rel_err_of_wildcat"] = error_vs_exact(w, Q, K, V, out["O"])

    # the divide-and-conquer and block-pivot forwards of the same inputs
    variants = []
    vspec = args.variants if args.variants is not None else ",".join(
        f"{b}:{c}" for b, c in DEFAULT_VARIANTS.get(w.name, []))
    if vspec and vspec != "none":
        for item in vspec.split(","):
            vb, vp = (int(x) for x in item.split(":"))
            if (vb, vp) == (bins, pb):
                continue
            vws = binding.workspace(binding.problem(w.heads, w.n, w.m, w.d, w.dv, w.r, dt_t, vb, 0, vp), dev)
            vout = dict(O=torch.empty_like(out["O"]), pivots=torch.empty_like(out["pivots"]),
                        rank=torch.empty_like(out["rank"]), flags=torch.empty_like(out["flags"]))

            def vfwd(vb=vb, vp=vp, vws=vws, vout=vout):
                binding.wc_forward(Q, K, V, w.r, seed=args.seed, bins=vb, pivot_block=vp, ws=vws, out=vout)

            vfwd()
            torch.cuda.synchronize()
            vms = time_replays(graph_of(vfwd), 5, stream)
            entry = {"bins": vb, "pivot_block": vp, "ms_per_step": round(vms, 4),
                     "tokens_per_s": round(w.tokens / (vms / 1e3), 1),
                     "rank_min": int(vout["rank"].min()), "flags_or": int(np.bitwise_or.reduce(vout["flags"].cpu().numpy()))}
            if not args.no_exact:
                entry["rel_err_vs_exact"] = error_vs_exact(w, Q, K, V, vout["O"])
            variants.append(entry)
            del vws, vout
            torch.cuda.empty_cache()

    log("exact attention and variants done")
    att = None
    if not args.no_roofline:
        att = attainable(dev, stream)
        if roof and roof.get("unit") == "GB/s":
            roof["frac_of_attainable"] = round(roof["achieved"] / att["hbm_read_GBps"], 4)
        if roof_att:
            roof_att["frac_of_attainable"] = round(roof_att["achieved"] / att["mfma_bf16_TFLOPs"], 4)
        log("attainable rates measured")
    cpu = None
    cpu1 = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, Qn, Kn, Vn, args.cpu_budget, bins, pb)
        if args.cpu_1core_workload != "none":
            # the first few heads of the workload, generated alone (each head has its own stream)
            w1 = synth.WORKLOADS[args.cpu_1core_workload]
            Q1, K1, V1 = synth.make_inputs(w1.name, heads=range(min(w1.heads, 4)))
            cpu1 = cpu_baseline(w1, Q1, K1, V1, args.cpu_1core_budget, threads=1)
            cpu1["workload"] = w1.name

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "description": w.description, "heads": w.heads, "n": w.n,
                   "m": w.m, "d": w.d, "dv": w.dv, "r": w.r, "bins": bins, "pivot_block": pb,
                   "tokens_per_step": w.tokens,
                   "pivot_uniforms": f"Philox4x64-10 seed {args.seed}"},
        "roofline": roof,
        "roofline_attend": roof_att,
        "cpu_baseline": cpu,
        "cpu_baseline_1thread": cpu1,
        "exact_attention": exact,
        "variants": variants,
        "attainable": att,
        "checks": {"rank_min": int(rank.min()), "flags_or": int(np.bitwise_or.reduce(flags)),
                   "wall_s_timed": round(wall, 4),
                   "launch": (f"hip graph replay, {per_replay} forwards per graph" if graph is not None
                              else "eager")},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
