#!/usr/bin/env python3
"""Benchmark of the WildCat forward (coreset selection + weights + attention) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload vit197]

A step is one whole forward (randomly pivoted Cholesky, Nystroem weights, attention over the
coreset) over every head of one batch of seeded synthetic inputs that are already resident
in HBM.  The default workload is the ViT-classification-shaped one (64 x 12 heads, n = 197,
d = 64, r = 32, bf16); the other workloads of coreset_head_rpcholesky_amd.synth can be
selected with --workload.  Prints one JSON line.

Beside the GPU number it reports:
  * roofline of the dominant kernel: algorithmic bytes (or flops) of one launch over its
    average duration, timed with HIP events on the stream the kernel is launched on;
  * cpu_baseline: the fp64 CPU oracle timed on a bounded sample of the same workload;
  * exact softmax attention (PyTorch SDPA) on the same tensors, for context.
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

# Kernel sources whose counters a stored traffic figure belongs to.
KERNEL_SOURCES = {
    "resident": ["wc_resident.hip", "wc_device.h", "wc_kernels.h"],
    "stream": ["wc_stream.hip", "wc_device.h", "wc_kernels.h"],
}
COUNTER_FILES = {
    "vit197": "profiles/resident_kernel_vit197_counters.txt",
}


def source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, "coreset_head_rpcholesky_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_traffic(workload: str, kind: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when the
    kernel source changed since the counters were taken."""
    path = COUNTER_FILES.get(workload)
    if not path or not os.path.exists(os.path.join(ROOT, path)):
        return None
    vals = {}
    for line in open(os.path.join(ROOT, path)):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha") != source_hash(kind):
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
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


def exact_attention_timing(w, Q, K, V, stream):
    """Exact softmax attention on the same tensors with PyTorch SDPA ([1, heads, len, d] so
    the fused backends are eligible); the first backend that runs is recorded."""
    import torch
    import torch.nn.functional as Fn
    from torch.nn.attention import SDPBackend, sdpa_kernel

    q, k, v = Q.unsqueeze(0), K.unsqueeze(0), V.unsqueeze(0)
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


def cpu_baseline(w, Q, K, V, budget_s: float, bins: int = 1, pivot_block: int = 1):
    """The fp64 oracle on as many heads as fit in the time budget, going round the workload's
    heads again when one pass takes less; tokens/s scaled to the whole workload (tokens per
    head = tokens / heads)."""
    import numpy as np

    from oracle import philox
    from oracle import wildcat as ow

    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        cores = min(16, os.cpu_count() or 1)
        limiter = threadpool_limits(cores)
        info = threadpool_info()
        cores = max([p.get("num_threads", 1) for p in info] + [1])
    except Exception:  # pragma: no cover
        limiter, cores = None, 1
    t0 = time.perf_counter()
    done = 0
    while True:
        h = done % w.heads
        if bins > 1 or pivot_block > 1:
            u = np.concatenate([philox.pivot_uniforms(42, h * bins + b, w.r // bins) for b in range(bins)])
            ow.forward_binned(Q[h], K[h], V[h], w.r, bins, u, pivot_block=pivot_block)
        else:
            u = np.array(philox.pivot_uniforms(42, h, w.r))
            ow.forward(Q[h], K[h], V[h], w.r, u)
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.unregister()
    tokens = w.tokens * done / w.heads
    what = (f"{done} of {w.heads} heads of one {w.name} forward" if done <= w.heads else
            f"{done} heads ({done / w.heads:.1f} passes over the {w.heads} heads of a {w.name} forward)")
    return {"value": tokens / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{what}{f' with {bins} bins' if bins > 1 else ''}, fp64 numpy/scipy, {dt:.1f} s"}


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
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                for _ in range(per_graph):
                    fn()
        torch.cuda.current_stream().wait_stream(side)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * per_graph)

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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="vit197")
    ap.add_argument("--seed", type=int, default=42)
    ap.add_argument("--bins", type=int, default=1,
                    help="divide-and-conquer selection with this many bins (must divide n and r)")
    ap.add_argument("--pivot-block", type=int, default=1,
                    help="block pivot selection: 16, 32 or 64 candidates per round (1: one pivot per step)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-exact", action="store_true")
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

    def fwd():
        binding.wc_forward(Q, K, V, w.r, seed=args.seed, bins=bins, pivot_block=pb, ws=ws, out=out)

    # One forward is captured in a HIP graph and replayed: the host-side launch path (Python,
    # ctypes, one launch per pivot step on the streaming path) would otherwise be what is timed.
    # A graph holds `per_replay` consecutive forwards, so the replays' own launch gaps are
    # amortised and back-to-back forwards run as they would inside a model.
    graph = None
    per_replay = 1
    if not args.no_graph:
        per_replay = max(d for d in range(1, 11) if args.steps % d == 0)
        fwd()
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                for _ in range(per_replay):
                    fwd()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()

    def launch():
        if graph is not None:
            graph.replay()
        else:
            fwd()

    nlaunch = args.steps // per_replay
    for _ in range(max(1, args.warmup // per_replay)):
        launch()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nlaunch + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(nlaunch):
        launch()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = [evs[i].elapsed_time(evs[i + 1]) / per_replay for i in range(nlaunch)]
    ms = evs[0].elapsed_time(evs[nlaunch]) / args.steps
    value = w.tokens / (ms / 1e3)
    rank = out["rank"].cpu().numpy()
    flags = out["flags"].cpu().numpy()

    acc = workload_accounting(w, bins)
    resident = w.dtype == "bf16" and w.n <= 256 and w.r <= 32 and bins == 1 and pb == 1
    if resident:
        # one launch per step: the resident kernel; only compulsory bytes reach HBM
        kernel_ms = float(np.mean(per))
        achieved = acc["compulsory_bytes"] / (kernel_ms / 1e3) / 1e9
        traffic = stored_traffic(w.name, "resident")
        roof = {"kernel": "resident_kernel (pivot loop + weights + attention, one workgroup per head)",
                "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes_per_launch": acc["compulsory_bytes"],
                "avg_launch_ms": round(kernel_ms, 5)}
    else:
        # the pivot loop dominates: time wc_rpcholesky alone (graph replay) on the same stream;
        # with bins, on the per-bin view (heads x bins sub-heads), which is what the forward runs
        Ksel = K.view(w.heads * bins, w.n // bins, w.d)
        pws = binding.workspace(binding.problem(w.heads * bins, w.n // bins, 0, w.d, w.dv, w.r // bins, dt_t,
                                                1, 0, pb), dev)

        def rpc():
            binding.wc_rpcholesky(Ksel, w.r // bins, seed=args.seed, ws=pws, with_diag=False, with_trace=False,
                                  pivot_block=pb)

        rgraph = None
        if not args.no_graph:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            rgraph = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side):
                with torch.cuda.graph(rgraph, stream=side):
                    rpc()
            torch.cuda.current_stream().wait_stream(side)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        rgraph.replay() if rgraph is not None else rpc()
        e1.record(stream)
        torch.cuda.synchronize()
        loop_ms = e0.elapsed_time(e1)
        sub_resident = w.dtype == "bf16" and w.n // bins <= 256 and w.r // bins <= 32 and pb == 1
        if pb > 1:
            name = (f"block pivot selection, {w.r // bins // pb} rounds of {pb} candidates"
                    f"{f', {w.heads * bins} bins' if bins > 1 else ''} (candidate columns: kernel part on "
                    f"bf16 MFMA, factor part on fp32 MFMA; factor update fp32 vector)")
            loop_bytes = None
        elif sub_resident:
            name = f"resident_kernel (pivot loop only, {w.heads * bins} sub-heads, factor on chip)"
            loop_bytes = acc["pivot_resident_bytes"]
        else:
            name = (f"rpc_step_kernel x {w.r // bins} launches (streaming pivot loop"
                    f"{f', {w.heads * bins} bins' if bins > 1 else ''})")
            loop_bytes = acc["pivot_bytes"]
        if pb > 1:
            # candidate columns G = exp(beta K K_S^T) - F F_S^T and F_new = G M^T, per sub-head
            Hs, ns, rs = w.heads * bins, w.n // bins, w.r // bins
            rounds = rs // pb
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
                    "algorithmic_flops_per_loop": flops, "rounds": rounds, "loop_ms": round(loop_ms, 3)}
        else:
            achieved = loop_bytes / (loop_ms / 1e3) / 1e9
            roof = {"kernel": name, "bound": "hbm",
                    "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                    "algorithmic_bytes_per_loop": loop_bytes, "loop_ms": round(loop_ms, 3)}

    exact = None
    if not args.no_exact:
        exact = exact_attention_timing(w, Q, K, V, stream)
        exact["rel_err_of_wildcat"] = error_vs_exact(w, Q, K, V, out["O"])

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, Qn, Kn, Vn, args.cpu_budget, bins, pb)

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
        "cpu_baseline": cpu,
        "exact_attention": exact,
        "checks": {"rank_min": int(rank.min()), "flags_or": int(np.bitwise_or.reduce(flags)),
                   "wall_s_timed": round(wall, 4), "launch": (f"hip graph replay, {per_replay} forwards per graph" if graph is not None
                              else "eager")},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
