"""Throughput of the compressed-KV compressor on one MI355X.

Workloads (--workload):
  stack32_long (default) the 32-layer Flash stack (30 compressed layers, hidden
              4096, head_dim 512, indexer head_dim 128, bf16) over a 65536-token
              prompt in 16 chunks of 4096, then 256 single-token decode steps:
              a step is one ds4c_compress_stack_prefill call and one
              ds4c_compress_stack_decode call (256 steps looped in the library).
  r4_flash    one Flash ratio-4 layer, one 4096-token chunk, hidden 4096,
              head_dim 512, indexer head_dim 128, bf16.  A step is one
              ds4c_compress_prefill call: projection GEMM + fused pool kernel.
  r128_flash  the same for a ratio-128 layer (head_dim 512).
  stack32     the 32-layer Flash stack (30 compressed layers), one 4096-token
              chunk: a step is one ds4c_compress_stack_prefill call.
  stack32_pro the 32-layer Pro-schedule stack (layers 0-1 ratio 128, then
              ratio 4 / 128 alternating; 32 compressed layers), one chunk.
  indexer_c5  indexer scoring + top-512 of one query over the 16,448 indexer
              rows a ratio-4 layer holds after the long prompt; a step is one
              ds4c_indexer_topk call (value in queries/s).

Every step starts from position 0 (the frontier counters are reset on the
host; a call at position 0 reads nothing from the frontier).  Inputs are
resident in HBM before timing.  Kernel times come from events the dispatch
itself records around each kernel (the library's timing mode), over the
timed region; `roofline` describes the kernel class that takes the most time
there (the decode GEMV for stack32_long), the other of the two is given
beside it.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--eager]
  python bench.py --copy-mib N     plain device copy of N MiB (counter calibration)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "compressor tokens/sec + compressed rows/sec; % HBM and MFMA peak (1 GPU)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
GEMM_SOURCE = os.path.join(ROOT, "compressed_kv_attention_compressor_amd", "csrc", "proj_gemm.hip")
POOL_SOURCE = os.path.join(ROOT, "compressed_kv_attention_compressor_amd", "csrc", "pool.hip")
DECODE_SOURCE = os.path.join(ROOT, "compressed_kv_attention_compressor_amd", "csrc", "decode.hip")
INDEXER_SOURCE = os.path.join(ROOT, "compressed_kv_attention_compressor_amd", "csrc", "indexer.hip")
ATTENTION_SOURCE = os.path.join(ROOT, "compressed_kv_attention_compressor_amd", "csrc", "attention.hip")


def fused_call(shape, n0, T):
    """Whether the library pools this call inside the projection epilogue.

    Mirrors the library's rule: the call starts on a window boundary and the
    fused grid is not too small (ratio 4: 80 workgroups of 256 x 160; ratio
    128: 32 of 128 x 128), or the hidden size is small enough that every
    path is short.
    """
    if n0 % shape.ratio:
        return False
    d_tot = shape.d_attn + (shape.d_index or 0)
    if shape.ratio == 4:
        grid, tile, need = -(-T // 256) * -(-d_tot // 40), 256 * 160, 80
    else:
        grid, tile, need = -(-T // 128) * (d_tot // 64), 128 * 128, 32
    if -(-grid // 256) * tile * shape.hidden < 256 * 160 * 1024:
        return True
    return grid >= need


def layer_algorithmic(shape, n0, T):
    """GEMM flops and pool-launch bytes of one prefill call (tokens n0 .. n0+T-1).

    Plain path, pool bytes: every projected kv/score element read once, the
    APE table, the rows written, and (ratio 128, whose finishing launch also
    carries the frontier) the live frontier rows written after the call; a
    ratio-4 call carries its frontier in a separate launch, counted by
    carry_bytes.  Fused path (window pooling in the projection epilogue), the
    finishing launch's bytes: the pooled rows read once, the rows written and
    the frontier rows the call writes from the staged tokens (read once).
    """
    lanes = [shape.d_attn] + ([shape.d_index] if shape.d_index else [])
    W = [shape.coff * d for d in lanes]
    N = 2 * sum(W)
    flops = 2.0 * T * N * shape.hidden
    n = n0 + T
    n_emit = n // shape.ratio - n0 // shape.ratio
    c = n % shape.ratio
    m = n - c
    live = ((4 if m >= 4 else 0) + c) if shape.ratio == 4 else c
    if fused_call(shape, n0, T):
        kept = min(live, T)
        pool_bytes = n_emit * sum(lanes) * 4 * 2 + kept * sum(W) * 2 * 4 * 2
    else:
        pool_bytes = T * N * 4 + shape.ratio * sum(W) * 4 + n_emit * sum(lanes) * 4
        if shape.ratio == 128:
            pool_bytes += live * sum(W) * 2 * 4
    return flops, pool_bytes, n_emit * len(lanes), N


def decode_gemv_bytes(shapes) -> float:
    """Weight bytes one decode token streams through every compressed layer
    of a stack (each layer's projection weights read once; x, the frontier
    row and the APE row are under 0.1 % and not counted)."""
    tot = 0.0
    for _, s in shapes:
        if s is None:
            continue
        lanes = [s.d_attn] + ([s.d_index] if s.d_index else [])
        N = 2 * sum(s.coff * d for d in lanes)
        tot += N * s.hidden * (2 if s.dtype == "bf16" else 4)
    return tot


def carry_bytes(shape, n0, T):
    """Bytes of the separate ratio-4 frontier carry: kept kv/score rows read and written."""
    W = [shape.coff * d for d in [shape.d_attn] + ([shape.d_index] if shape.d_index else [])]
    n = n0 + T
    c = n % shape.ratio
    live = (4 if n - c >= 4 else 0) + c
    return 2 * live * sum(W) * 2 * 4


def proj_plan(M: int, N: int, K: int):
    """(tile rows, K splits) of the library's plain projection for an [M, N] output.

    Mirrors the library: per tile shape, the K split that keeps the splits
    resident in one round, then the least estimated time from measured
    per-round times (75, 42 and 25 us for 256 x 160, 128 x 128 and 64 x 64
    at K = 4096; extra 64 x 64 tiles per CU cost 0.7 of a round each).
    """
    best = None
    for bm, bn, rnd in ((256, 160, 75.0), (128, 128, 42.0), (64, 64, 25.0)):
        tiles = -(-M // bm) * -(-N // bn)
        s = 1
        while bm != 256 and s < 16:
            s2 = 2 * s
            if tiles * s2 > (512 if bm == 64 else 256) or M * s2 > 1024 or K % (64 * s2) or K // s2 < 128:
                break
            s = s2
        per_cu = -(-(tiles * s) // 256)
        rounds = 1.0 + 0.7 * (per_cu - 1) if bm == 64 else float(per_cu)
        us = rounds * rnd * K / s / 4096.0
        if best is None or us < best[0]:
            best = (us, bm, s)
    return best[1], best[2]


def proj_kernel_name(M: int, N: int, K: int) -> str:
    """Projection kernel the library launches for a plain [M, N] output."""
    bm, s = proj_plan(M, N, K)
    name = "proj_splitk_kernel" if bm == 256 else "proj_mfma_kernel"
    return name + (f" (K split {s})" if s > 1 else "")


# What a kernel source compiles with besides itself: the shared device
# helpers and argument structs, and the build script that holds the flags.
SHARED_SOURCES = [os.path.join(ROOT, "compressed_kv_attention_compressor_amd", "csrc", f)
                  for f in ("device_common.h", "kernel_args.h", "launch.h")] + \
                 [os.path.join(ROOT, "compressed_kv_attention_compressor_amd", "build.py")]


def source_digest(source: str) -> str:
    """sha256 over a kernel source followed by SHARED_SOURCES, in that order."""
    h = hashlib.sha256()
    for path in [source] + SHARED_SOURCES:
        h.update(open(path, "rb").read())
    return h.hexdigest()


def read_traffic(workload: str, key: str = "gemm_hbm_bytes_per_launch"):
    """HBM bytes per launch (GEMM, or another key of the summary) from the
    committed counter summary, or None.

    The summary names the digest (source_digest) of the kernel sources it
    was taken on (the projection's for GEMM figures, the pool's for pool
    figures, the decode, indexer or attention source's for theirs); a
    different digest means the counters are stale and none is used.
    """
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    kind = next((k for k in ("decode", "indexer", "attention") if key.startswith(k)),
                "pool" if "pool" in key else "gemm")
    source = {"decode": DECODE_SOURCE, "pool": POOL_SOURCE, "gemm": GEMM_SOURCE, "indexer": INDEXER_SOURCE,
              "attention": ATTENTION_SOURCE}[kind]
    if kv.get(f"{kind}_sources_sha256") != source_digest(source):
        return None
    try:
        return float(kv[key])
    except (KeyError, ValueError):
        return None


def cpu_baseline(shape, x, params, budget_s=12.0, one_thread=False):
    """The oracle as it is, timed on this host over whole prefill steps of the layer."""
    from threadpoolctl import threadpool_info

    import oracle
    from tests._helpers import oracle_spec

    spec = oracle_spec(shape, params)
    steps, t0 = 0, time.perf_counter()
    while True:
        st = oracle.new_layer_state(spec)
        oracle.prefill(spec, st, x)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 50:
            break
    info = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] + [1])
    blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in info
                             if i.get("user_api") == "blas"})) or "unknown"
    out = {"value": steps * len(x) / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{steps} full {len(x)}-token prefill steps of one ratio-{shape.ratio} layer "
                     f"({el:.1f} s); float64 NumPy, BLAS threads {threads}, recurrence single-threaded",
           "cpu_model": cpu_model(), "blas": blas,
           "cpus_visible": len(os.sched_getaffinity(0))}
    if one_thread:
        # The same oracle with BLAS held to one thread, over a shorter sample.
        from threadpoolctl import threadpool_limits

        with threadpool_limits(limits=1):
            n1, t1 = 0, time.perf_counter()
            while True:
                st = oracle.new_layer_state(spec)
                oracle.prefill(spec, st, x)
                n1 += 1
                el1 = time.perf_counter() - t1
                if el1 >= budget_s / 2 or n1 >= 50:
                    break
        out["one_thread"] = {"value": n1 * len(x) / el1, "unit": "tokens/s", "cores": 1,
                             "sample": f"{n1} full {len(x)}-token prefill steps ({el1:.1f} s)"}
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_calibration(mib: int, reps: int = 20) -> None:
    import torch

    n = mib * 1024 * 1024 // 4
    a = torch.randn(n, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    print(json.dumps({"copy_mib": mib, "bytes_read_per_launch": mib * 2 ** 20,
                      "bytes_written_per_launch": mib * 2 ** 20, "reps": reps, "us_per_copy": el / reps * 1e6}),
          flush=True)


def calls_graph_timing(step, outputs, steps, per_graph=20):
    """Seconds per call of `step` with the host's enqueue cost taken off the
    GPU's timeline: `per_graph` calls captured as one HIP graph, replayed
    between two events.  None when capture is not available or one replay
    does not reproduce the eager call's `outputs` bit for bit (the outputs
    are poisoned first)."""
    import torch
    try:
        ref = [t.clone() for t in outputs]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                step()
        for t in outputs:
            t.fill_(-1 if not t.is_floating_point() else float("nan"))
        g.replay()
        torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(outputs, ref)):
            print("graph replay differs from the eager call; wall timing kept", file=sys.stderr)
            return None
    except Exception as e:  # capture not supported here: keep the wall timing
        torch.cuda.synchronize()
        print(f"graph capture unavailable ({e}); wall timing kept", file=sys.stderr)
        return None
    reps = max(1, steps // per_graph)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(reps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    ok = all(torch.equal(a, b) for a, b in zip(outputs, ref))
    if not ok:
        print("timed graph replays differ from the eager call; wall timing kept", file=sys.stderr)
        return None
    return ev0.elapsed_time(ev1) * 1e-3 / (reps * per_graph)


def bench_indexer(w, args):
    """One query's indexer scoring and top-512 over 16,448 rows (64 heads x 128
    dims): the score launch reads every row once; one select launch follows."""
    import torch

    from compressed_kv_attention_compressor_amd import binding as B
    from compressed_kv_attention_compressor_amd import synth

    n, H, Dh, k = w.tokens, 64, 128, 512
    steps = args.steps or 200
    warmup = args.warmup if args.warmup >= 0 else 10
    q_np, w_np, rows_np = synth.indexer_inputs(w.wid, n, H, Dh)
    q, hw, rows = (torch.from_numpy(a).cuda() for a in (q_np, w_np, rows_np))
    idx = torch.empty(k, dtype=torch.int32, device="cuda")
    sc = torch.empty(k, dtype=torch.float32, device="cuda")
    ws = torch.empty(B.ds4c_indexer_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
    def step():
        B.ds4c_indexer_topk(q.data_ptr(), hw.data_ptr(), H, Dh, rows.data_ptr(), n, k, idx.data_ptr(),
                            sc.data_ptr(), 0, 0, ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    B.ds4c_profile_enable([B.KCLASS_INDEXER])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms, cnt = B.ds4c_profile_read()
    B.ds4c_profile_enable(False)
    call_ms = ms[B.KCLASS_INDEXER] / max(cnt[B.KCLASS_INDEXER], 1)
    per_call = calls_graph_timing(step, [idx, sc], steps)
    t_call = per_call if per_call is not None else el / steps
    # Algorithmic bytes: rows read once, query and head weights, scores written
    # and read back by the sort, the selected rows and scores written.
    alg = n * Dh * 4 + H * Dh * 4 + H * 4 + 2 * n * 4 + k * 8
    gbs = alg / (call_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC, "value": 1.0 / t_call, "unit": "queries/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": t_call * 1e3,
        "timing": ("replays of a captured HIP graph of 20 calls between two events (one replay checked to write the "
                   "eager call's results)" if per_call is not None else "wall clock over back-to-back calls"),
        "wall_ms_per_step": el / steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (seeded N(0,1) query heads and rows, N(0,1/64) head weights)",
        "config": {"workload": w.name, "rows": n, "heads": H, "head_dim": Dh, "top_k": k},
        "rows_per_s": n / t_call,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                     "traffic": read_traffic("indexer_c5", "indexer_hbm_bytes_per_call"),
                     "kernel": "indexer_score_kernel + indexer_select_kernel (one call)",
                     "avg_ms": call_ms, "algorithmic_bytes": alg},
    }
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_info
        calls, t0 = 0, time.perf_counter()
        while True:
            oracle.indexer.select(q_np, w_np, rows_np, k)
            calls += 1
            el_c = time.perf_counter() - t0
            if el_c >= 10.0 or calls >= 200:
                break
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        out["cpu_baseline"] = {"value": calls / el_c, "unit": "queries/s", "cores": threads, "kind": "oracle",
                               "sample": f"{calls} whole calls ({el_c:.1f} s); float64 NumPy, BLAS threads {threads}",
                               "cpu_model": cpu_model(), "cpus_visible": len(os.sched_getaffinity(0))}
    print(json.dumps(out), flush=True)


def bench_mixed_attention(w, args):
    """One decode query's ratio-4 mixed attention: 64 heads x 512 dims over
    the 128 raw window rows and the top 512 of 16,448 compressed rows."""
    import torch

    from compressed_kv_attention_compressor_amd import binding as B
    from compressed_kv_attention_compressor_amd import synth

    n, H, D, ring_cap, k = w.tokens, 64, 512, 128, 512
    qpos = 4 * n - 1                       # the last token of the prompt whose rows are all emitted
    first = qpos + 1 - ring_cap
    steps = args.steps or 200
    warmup = args.warmup if args.warmup >= 0 else 10
    q_np, ring_np, comp_np, topk_np = synth.mixed_attention_inputs(w.wid, n, H, D, ring_cap, k)
    q, ring, comp = (torch.from_numpy(a).cuda() for a in (q_np, ring_np, comp_np))
    topk = torch.from_numpy(topk_np).cuda()
    out = torch.empty(H, D, dtype=torch.float32, device="cuda")
    ws = torch.empty(B.ds4c_mixed_attention_workspace_bytes(H, D, ring_cap, k), dtype=torch.uint8, device="cuda")
    def step():
        B.ds4c_mixed_attention(q, ring, first, qpos, ring_cap, comp, topk, qpos, 4, out, ws,
                               torch.cuda.current_stream().cuda_stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    B.ds4c_profile_enable([B.KCLASS_ATTENTION])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms, cnt = B.ds4c_profile_read()
    B.ds4c_profile_enable(False)
    call_ms = ms[B.KCLASS_ATTENTION] / max(cnt[B.KCLASS_ATTENTION], 1)
    per_call = calls_graph_timing(step, [out], steps)
    t_call = per_call if per_call is not None else el / steps
    # Algorithmic bytes: each attended row read once, the query read, the
    # output written, the list read.
    rows = ring_cap + k
    alg = rows * D * 4 + 2 * H * D * 4 + k * 4
    flops = 2 * 2 * H * rows * D           # logits and weighted rows
    gbs = alg / (call_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": 1.0 / t_call, "unit": "queries/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": t_call * 1e3,
        "timing": ("replays of a captured HIP graph of 20 calls between two events (one replay checked to write the "
                   "eager call's results)" if per_call is not None else "wall clock over back-to-back calls"),
        "wall_ms_per_step": el / steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic (seeded N(0,1) query heads, raw and compressed rows; a random top-512)",
        "config": {"workload": w.name, "compressed_rows": n, "heads": H, "head_dim": D, "raw_rows": ring_cap,
                   "top_k": k, "qpos": qpos},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                     "traffic": read_traffic("mixed_attn_c5", "attention_hbm_bytes_per_call"),
                     "kernel": "mixed_attn_part_kernel + mixed_attn_merge_kernel (one call)",
                     "avg_ms": call_ms, "algorithmic_bytes": alg, "algorithmic_flops": flops},
    }
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_info
        calls, t0 = 0, time.perf_counter()
        while True:
            oracle.mixed_attention.mixed_attention(q_np, ring_np, first, qpos, ring_cap, comp_np, topk_np, qpos, 4)
            calls += 1
            el_c = time.perf_counter() - t0
            if el_c >= 10.0 or calls >= 2000:
                break
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        res["cpu_baseline"] = {"value": calls / el_c, "unit": "queries/s", "cores": threads, "kind": "oracle",
                               "sample": f"{calls} whole calls ({el_c:.1f} s); float64 NumPy, BLAS threads {threads}",
                               "cpu_model": cpu_model(), "cpus_visible": len(os.sched_getaffinity(0))}
    print(json.dumps(res), flush=True)


GRAPH_FIGURES = {}  # per-step replay times behind the graph timing, reported with the result


def graph_timing(w, L, reinit, work, step, steps):
    """Seconds for `steps` steps of a single-layer workload, timed as replays
    of captured HIP graphs: the host cost of enqueueing a step (a few tens
    of microseconds, comparable to a ratio-128 step) is then off the GPU's
    timeline.  One graph holds SPG steps (re-initialisation + the call, SPG
    times), another SPG re-initialisations alone; both keep the GPU busy for
    longer than the host needs to replay them, so the difference of their
    replay times is the steps' own GPU time.  None when capture is not
    available or a replay does not write exactly the rows an eager step
    writes (checked on the first and the last replay)."""
    import torch

    spg = 10
    try:
        step()
        torch.cuda.synchronize()
        ref = {k: L.live_rows(k).clone() for k in L.kinds}
        g_init, g_full = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_init):
            for _ in range(spg):
                reinit()
        with torch.cuda.graph(g_full):
            for _ in range(spg):
                reinit()
                work()
        for k in L.kinds:
            L.rows[k].fill_(float("nan"))
        g_full.replay()
        torch.cuda.synchronize()
        if not all(torch.equal(L.rows[k][:ref[k].shape[0]], ref[k]) for k in L.kinds):
            print("graph replay differs from the eager step; eager timing kept", file=sys.stderr)
            return None
    except Exception as e:  # capture not supported here: keep the eager timing
        torch.cuda.synchronize()
        print(f"graph capture unavailable ({e}); eager timing kept", file=sys.stderr)
        return None

    n_rep = max(1, steps // spg)

    def run(g):
        g.replay()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        for _ in range(n_rep):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / (n_rep * spg)

    for k in L.kinds:
        L.rows[k].fill_(float("nan"))
    t_full, t_init = run(g_full), run(g_init)
    # The last timed replay wrote the rows too (the re-initialisation graph
    # leaves them alone): they must still be the eager step's.
    same = all(torch.equal(L.rows[k][:ref[k].shape[0]], ref[k]) for k in L.kinds)
    L.reset()
    torch.cuda.synchronize()
    if not same:
        print("timed graph replays differ from the eager step; eager timing kept", file=sys.stderr)
        return None
    GRAPH_FIGURES.update({"graph_steps_per_replay": spg, "graph_full_ms_per_step": t_full * 1e3,
                          "graph_reinit_ms_per_step": t_init * 1e3})
    return (t_full - t_init) * steps


def decode_graph_timing(stack, layers, x, T, Td, chunk, reinit, steps):
    """Seconds for `steps` steps of a stack workload with decode steps, the
    decode part replayed from a captured HIP graph.

    The Td decode steps are thousands of small launches whose host-side
    enqueueing (tens of microseconds per launch with Python and the library's
    validation) outruns their GPU time; captured once (after a prefill, at
    the positions every step decodes) and replayed, they run back to back on
    the GPU.  Each timed step is: re-initialisation (not timed), the prefill
    calls (eager) and one replay, between two events.  None when capture is
    not available or a replay does not reproduce the eager run's rows and
    frontiers bit for bit (checked after the first and the last timed step).
    """
    import torch

    def snapshot_state():
        # rows a step emits (the host counters do not follow graph replays)
        # and the frontier tensors
        out = []
        for L in layers:
            if L is None:
                continue
            out += [v[:(T + Td) // L.ratio].clone() for v in L.rows.values()]
            out += [t.clone() for pair in L.frontier_views().values() for t in pair]
        return out

    def same(ref):
        cur = snapshot_state()
        return len(cur) == len(ref) and all(torch.equal(a, b) for a, b in zip(cur, ref))

    try:
        reinit()
        stack.prefill(x[:T], chunk_cap=chunk)
        stack.decode(x[T:T + Td])
        torch.cuda.synchronize()
        ref = snapshot_state()
        reinit()
        stack.prefill(x[:T], chunk_cap=chunk)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            stack.decode(x[T:T + Td])        # enqueued into the graph, not run
        for L in layers:
            if L is not None:
                for v in L.rows.values():
                    v.fill_(float("nan"))
        reinit()
        stack.prefill(x[:T], chunk_cap=chunk)
        g.replay()
        torch.cuda.synchronize()
        if not same(ref):
            print("decode graph replay differs from the eager steps; eager timing kept", file=sys.stderr)
            return None
    except Exception as e:  # capture not supported here: keep the eager timing
        torch.cuda.synchronize()
        print(f"graph capture unavailable ({e}); eager timing kept", file=sys.stderr)
        return None
    evs = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    for ev_a, ev_m, ev_b in evs:
        reinit()
        ev_a.record()
        stack.prefill(x[:T], chunk_cap=chunk)
        ev_m.record()
        g.replay()
        ev_b.record()
    torch.cuda.synchronize()
    ok = same(ref)
    step_ms = sorted(a.elapsed_time(b) for a, _, b in evs)
    el = sum(step_ms) * 1e-3
    el_pre = sum(a.elapsed_time(m) for a, m, _ in evs) * 1e-3
    reinit()
    torch.cuda.synchronize()
    if not ok:
        print("timed decode graph replays differ from the eager steps; eager timing kept", file=sys.stderr)
        return None
    GRAPH_FIGURES.update({"graph_decode_steps": Td, "graph_ms_per_step": el / steps * 1e3,
                          "ms_per_step_median": step_ms[len(step_ms) // 2], "ms_per_step_min": step_ms[0],
                          "prefill_ms_per_step": el_pre / steps * 1e3,
                          "decode_us_per_token": (el - el_pre) / steps / Td * 1e6})
    return el


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0, help="timed steps (default depends on the workload)")
    ap.add_argument("--warmup", type=int, default=-1)
    ap.add_argument("--workload", default="stack32_long",
                    choices=["r4_flash", "r128_flash", "stack32", "stack32_long", "stack32_pro", "indexer_c5",
                             "mixed_attn_c5"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time every step eagerly, without HIP graph capture (for profiler counter passes)")
    ap.add_argument("--copy-mib", type=int, default=0)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus must be 1)", file=sys.stderr)
        sys.exit(2)
    if args.copy_mib:
        copy_calibration(args.copy_mib)
        return

    import torch

    from compressed_kv_attention_compressor_amd import binding as B
    from compressed_kv_attention_compressor_amd import synth
    from compressed_kv_attention_compressor_amd.layer import CompressorLayer, CompressorStack

    w = synth.WORKLOADS[args.workload]
    if args.workload == "indexer_c5":
        bench_indexer(w, args)
        return
    if args.workload == "mixed_attn_c5":
        bench_mixed_attention(w, args)
        return
    long_run = args.workload == "stack32_long"
    steps = args.steps or (3 if long_run else 20 if w.layer is None else 50)
    warmup = args.warmup if args.warmup >= 0 else (1 if long_run else 5)
    T, Td = w.tokens, w.decode_tokens

    if w.layer is not None:
        shapes = [(0, w.layer)]
        params = {0: synth.layer_params(w.wid, 0, w.layer)}
    else:
        shapes = [(l, synth.stack_layer_shape(B.ds4c_layer_ratio(w.variant, l))) for l in range(w.n_layers)]
        params = {l: synth.layer_params(w.wid, l, s) for l, s in shapes if s is not None}
    hidden = 4096 if w.layer is None else w.layer.hidden
    dtype = "bf16" if w.layer is None else w.layer.dtype
    x_np = synth.hidden_states(w.wid, hidden, 0, T + Td, dtype)
    x = torch.from_numpy(x_np).to("cuda", torch.bfloat16 if dtype == "bf16" else torch.float32)
    layers = [None if s is None else
              CompressorLayer(s.ratio, s.hidden, params[l], dtype=s.dtype, n_rot=s.n_rot, rope_base=s.rope_base,
                              rms_eps=s.rms_eps, max_tokens=T + Td) for l, s in shapes]

    # Algorithmic work of one step.
    flops = pool_bytes = 0.0
    rows = 0
    gemm_launches = 0
    chunk = min(T, 4096)
    for (l, s), L in zip(shapes, layers):
        if s is None:
            continue
        for t0 in range(0, T, chunk):
            f, pb, r_, _ = layer_algorithmic(s, t0, min(chunk, T - t0))
            flops, pool_bytes, rows = flops + f, pool_bytes + pb, rows + r_
            gemm_launches += 1
        rows += ((T + Td) // s.ratio - T // s.ratio) * (2 if s.ratio == 4 else 1)
    # Rows a step emits per lane (every step starts from empty frontiers).
    rows_lanes = {"attention": sum((T + Td) // s.ratio for _, s in shapes if s is not None),
                  "indexer": sum((T + Td) // 4 for _, s in shapes if s is not None and s.ratio == 4)}
    assert rows == rows_lanes["attention"] + rows_lanes["indexer"], (rows, rows_lanes)

    # One step: every layer's frontier back to its initial state (kv 0,
    # score -inf, counters 0; a fill launch per layer, not timed), then the
    # step's calls, which are timed.
    if w.layer is not None:
        L = layers[0]
        L.reserve(T)

        def reinit():
            L.reset()

        def work():
            L.prefill(x[:T])
    else:
        stack = CompressorStack(layers)
        stack.reserve(chunk)

        def reinit():
            for L in layers:
                if L is not None:
                    L.reset()

        def work():
            stack.prefill(x[:T], chunk_cap=chunk)
            if Td:
                stack.decode(x[T:T + Td])   # Td single-token steps, looped in the library

    def step():
        reinit()
        work()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # Timed region: each step's calls between two events on the library's
    # stream (the re-initialisation stays outside them); the projection GEMMs
    # and, with decode steps, the decode GEMVs (the two largest kernel
    # classes) are also bracketed by dispatch-recorded events.
    timed_classes = [B.KCLASS_PROJ] + ([B.KCLASS_DECODE] if Td else [])
    B.ds4c_profile_enable(timed_classes)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for ev_a, ev_b in evs:
        reinit()
        ev_a.record()
        work()
        ev_b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    eager_steps_ms = sorted(a.elapsed_time(b) for a, b in evs)
    el_eager = sum(eager_steps_ms) * 1e-3
    ms, cnt = B.ds4c_profile_read()
    B.ds4c_profile_enable(False)
    if args.eager:
        el_graph = None
    elif w.layer is not None:
        el_graph = graph_timing(w, L, reinit, work, step, steps)
    elif Td:
        el_graph = decode_graph_timing(stack, layers, x, T, Td, chunk, reinit, steps)
    else:
        el_graph = None
    el = el_graph if el_graph is not None else el_eager
    # A separate pass times the pool kernels (and the decode boundary launches).
    side_steps = max(1, min(steps, 10))
    side = [B.KCLASS_POOL, B.KCLASS_DECODE_POOL] + ([] if Td else [B.KCLASS_DECODE])
    B.ds4c_profile_enable(side)
    for _ in range(side_steps):
        step()
    torch.cuda.synchronize()
    ms2, cnt2 = B.ds4c_profile_read()
    B.ds4c_profile_enable(False)
    for c in side:
        ms[c], cnt[c] = ms2[c], cnt2[c]

    gemm_ms = ms[B.KCLASS_PROJ] / max(cnt[B.KCLASS_PROJ], 1)
    all_fused = all(fused_call(s, 0, min(T, chunk)) for _, s in shapes if s is not None)
    gemm_kernel = " + ".join(sorted({("proj_splitk_kernel (fused ratio-4 pool epilogue)" if s.ratio == 4 else
                                      "proj_r128_splitk4_kernel (fused ratio-128 pool epilogue)") if fused_call(s, 0, min(T, chunk)) else
                                     proj_kernel_name(min(T, chunk), 2 * sum(s.coff * d for d in (s.d_attn, s.d_index) if d), s.hidden)
                                     for _, s in shapes if s is not None}))
    pool_ms = ms[B.KCLASS_POOL] / max(cnt[B.KCLASS_POOL], 1)
    flops_per_launch = flops / max(gemm_launches, 1)
    pool_bytes_per_launch = pool_bytes / max(gemm_launches, 1)
    gemm_tflops = flops_per_launch / (gemm_ms * 1e-3) / 1e12
    pool_gbs = pool_bytes_per_launch / (pool_ms * 1e-3) / 1e9
    peak = PEAK_BF16_TFLOPS if dtype == "bf16" else PEAK_FP32_TFLOPS
    traffic = read_traffic(args.workload)
    # MFMA pipes busy over the GEMM's run, from the committed counter summary
    # (SQ_VALU_MFMA_BUSY_CYCLES summed over the 1024 SIMDs against
    # GRBM_GUI_ACTIVE summed over the 8 XCDs); None when stale or absent.
    busy, active = (read_traffic(args.workload, k) for k in ("gemm_mfma_busy_cycles", "gemm_grbm_gui_active"))
    mfma_busy = busy / 1024 / (active / 8) if busy and active else None
    gemm_roofline = {"bound": "mfma", "achieved": gemm_tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": gemm_tflops / peak, "traffic": traffic, "mfma_busy": mfma_busy, "kernel": gemm_kernel,
                     "avg_ms": gemm_ms, "launches": cnt[B.KCLASS_PROJ], "total_ms": ms[B.KCLASS_PROJ],
                     "algorithmic_flops": flops_per_launch}
    decode_roofline = None
    if Td:
        # Decode GEMV: every layer's projection weights stream once per token
        # (the per-token figure of the measurement plan); the launches of the
        # ratio-4 and ratio-128 layers are averaged together, as one kernel.
        gemv_ms = ms[B.KCLASS_DECODE] / max(cnt[B.KCLASS_DECODE], 1)
        gemv_bytes = decode_gemv_bytes(shapes) / max(sum(1 for _, s in shapes if s is not None), 1)
        gemv_gbs = gemv_bytes / (gemv_ms * 1e-3) / 1e9
        decode_roofline = {"bound": "hbm", "achieved": gemv_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": gemv_gbs / PEAK_HBM_GBS,
                           "traffic": read_traffic(args.workload, "decode_gemv_hbm_bytes_per_launch"),
                           "kernel": "decode_gemv_kernel (ratio-4 and ratio-128 layers)", "avg_ms": gemv_ms,
                           "launches": cnt[B.KCLASS_DECODE], "total_ms": ms[B.KCLASS_DECODE],
                           "algorithmic_bytes": gemv_bytes}
    # The roofline reported is the one of the kernel class that takes the most
    # time in the timed region; the other is given beside it.
    if decode_roofline is not None and ms[B.KCLASS_DECODE] > ms[B.KCLASS_PROJ]:
        roofline, other = decode_roofline, ("mfma_roofline", gemm_roofline)
    else:
        roofline, other = gemm_roofline, ("decode_roofline", decode_roofline)

    cfg = {"workload": w.name, "tokens": T, "decode_tokens": Td, "hidden": hidden, "chunk": chunk,
           "layers": sum(1 for s in shapes if s[1] is not None), "dtype": dtype}
    if w.layer is not None:
        cfg.update({"ratio": w.layer.ratio, "head_dim": w.layer.d_attn, "index_head_dim": w.layer.d_index})
    out = {
        "metric": METRIC,
        "value": steps * (T + Td) / el,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": el / steps * 1e3,
        "timing": ("replays of a captured HIP graph of 10 steps (frontier re-initialisation + the step's calls, "
                   "ten times) minus replays of a graph of the 10 re-initialisations alone; the first and the last "
                   "replay were checked to write the eager run's rows" if el_graph is not None and w.layer is not None
                   else "sum of per-step event intervals on the library's stream, each step the prefill calls "
                   "(eager) and one replay of a HIP graph holding the step's decode launches (captured once; "
                   "rows and frontiers of the first and last timed step checked bitwise against the eager run); "
                   "the frontier re-initialisation between steps is outside the intervals" if el_graph is not None
                   else "sum of per-step event intervals on the library's stream; the frontier re-initialisation "
                   "between steps is outside them"),
        **GRAPH_FIGURES,
        "eager_ms_per_step": el_eager / steps * 1e3,
        "eager_ms_per_step_median": eager_steps_ms[len(eager_steps_ms) // 2],
        "eager_ms_per_step_min": eager_steps_ms[0],
        "wall_ms_per_step": wall / steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,1) hidden states, N(0,0.02) weights, N(0,0.1) APE)",
        "config": cfg,
        "rows_per_s": steps * rows / el,
        "rows_per_step": rows_lanes,
        "roofline": roofline,
        **({other[0]: other[1]} if other[1] is not None else {}),
        "pool_roofline": {"bound": "hbm", "achieved": pool_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": pool_gbs / PEAK_HBM_GBS,
                          "kernel": "pool (all launches of one call)" if not all_fused else
                                    "row finisher (window pooling runs in the projection epilogue)",
                          "measured": f"separate pass of {side_steps} steps",
                          "avg_ms": pool_ms, "algorithmic_bytes": pool_bytes_per_launch},
        "kernel_launches": {"proj (timed region)": cnt[B.KCLASS_PROJ],
                            f"pool (pass of {side_steps} steps)": cnt[B.KCLASS_POOL],
                            ("decode GEMV (timed region)" if Td else f"decode GEMV (pass of {side_steps} steps)"):
                                cnt[B.KCLASS_DECODE],
                            f"decode boundary (pass of {side_steps} steps)": cnt[B.KCLASS_DECODE_POOL]},
    }
    if cnt[B.KCLASS_DECODE]:
        out["decode_avg_ms"] = ms[B.KCLASS_DECODE] / cnt[B.KCLASS_DECODE]
    if cnt[B.KCLASS_DECODE_POOL]:
        out["decode_boundary_avg_ms"] = ms[B.KCLASS_DECODE_POOL] / cnt[B.KCLASS_DECODE_POOL]
    if long_run:
        # Session snapshot of the whole stack at the end of a step (rows and
        # frontiers of every layer through pageable host memory), then a
        # restore into the same buffers; outside the timed region.
        t_s = time.perf_counter()
        blob = stack.snapshot()
        t_m = time.perf_counter()
        stack.restore(blob)
        t_e = time.perf_counter()
        out["snapshot"] = {"bytes": len(blob), "save_ms": (t_m - t_s) * 1e3, "load_ms": (t_e - t_m) * 1e3,
                           "save_GBs": len(blob) / (t_m - t_s) / 1e9, "load_GBs": len(blob) / (t_e - t_m) / 1e9,
                           "host_memory": "pageable"}
        del blob
    if w.layer is not None and T > w.layer.ratio:
        # Calls that start inside a window keep the separate pool launch(es):
        # one token, then the rest of the chunk from n0 = 1; the second call's
        # pool is timed.  Warm: it reads the projection output the call's own
        # GEMM has just written.
        # One pool interval per call: the median of 21 calls is reported (a
        # single late dispatch would dominate a mean of a few samples).
        L = layers[0]
        pl, cr = [], []
        for _ in range(21):
            L.reset()
            L.prefill(x[:1])
            B.ds4c_profile_enable([B.KCLASS_POOL, B.KCLASS_CARRY])
            L.prefill(x[1:T])
            m_, c_ = B.ds4c_profile_read()
            B.ds4c_profile_enable(False)
            if c_[B.KCLASS_POOL]:
                pl.append(m_[B.KCLASS_POOL] / c_[B.KCLASS_POOL])
            if c_[B.KCLASS_CARRY]:
                cr.append(m_[B.KCLASS_CARRY] / c_[B.KCLASS_CARRY])
        # Cold: the library passes over a 1 GiB scratch buffer between each
        # call's projection and pool launches (outside the timed interval),
        # which evicts the projection output from the L2s and the Infinity
        # Cache.  Read eviction leaves clean lines; write eviction leaves
        # dirty ones, whose write-back then falls on the pool.
        scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        cold = {}
        for write in (False, True):
            B.ds4c_profile_evict(scratch.data_ptr(), scratch.numel(), write=write)
            ts = []
            for _ in range(21):
                L.reset()
                L.prefill(x[:1])
                B.ds4c_profile_enable([B.KCLASS_POOL])
                L.prefill(x[1:T])
                m_, c_ = B.ds4c_profile_read()
                B.ds4c_profile_enable(False)
                if c_[B.KCLASS_POOL]:
                    ts.append(m_[B.KCLASS_POOL] / c_[B.KCLASS_POOL])
            B.ds4c_profile_evict(0, 0)
            cold[write] = sorted(ts)[len(ts) // 2] if ts else 0.0
        del scratch
        pl_cnt, cr_cnt = len(pl), len(cr)
        _, pl_bytes, _, _ = layer_algorithmic(w.layer, 1, T - 1)
        pl_avg = sorted(pl)[len(pl) // 2] if pl else 0.0
        pl_gbs = pl_bytes / (pl_avg * 1e-3) / 1e9
        cold_gbs = {k: pl_bytes / (v * 1e-3) / 1e9 if v else 0.0 for k, v in cold.items()}
        # The HBM fraction is the cold figure (the projection output read from
        # HBM); the warm figure, whose reads partly hit the caches, is given
        # beside it as such.
        out["plain_pool_roofline"] = {
            "bound": "hbm", "achieved": cold_gbs[False], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": cold_gbs[False] / PEAK_HBM_GBS,
            "kernel": "pool_r4_kernel" if w.layer.ratio == 4 else "pool_r128_partial_kernel + pool_r128_finish_kernel",
            "measured": f"median of 21 calls of {T - 1} tokens from n0 = 1, cold: a 1 GiB buffer read between each "
                        f"call's projection and pool launches (the caches hold clean lines)",
            "avg_ms": cold[False], "algorithmic_bytes": pl_bytes,
            "traffic": read_traffic(args.workload, "plain_pool_hbm_bytes_per_launch"),
            "cache_warm": {"achieved": pl_gbs, "avg_ms": pl_avg,
                           "measured": f"median of {pl_cnt} calls, warm: the pool reads the projection written just "
                                       f"before, partly from the caches (not an HBM figure)"},
            "cold_write_evict": {"achieved": cold_gbs[True], "frac": cold_gbs[True] / PEAK_HBM_GBS,
                                 "avg_ms": cold[True],
                                 "measured": "median of 21 calls, a 1 GiB buffer written between each call's "
                                             "projection and pool launches (the pool also pays the write-back "
                                             "of the dirty lines it displaces)"}}
        if cr_cnt:
            out["plain_pool_roofline"]["carry"] = {
                "kernel": "pool_r4_carry_kernel", "avg_ms": sorted(cr)[len(cr) // 2],
                "algorithmic_bytes": carry_bytes(w.layer, 1, T - 1)}
    if not args.no_cpu_baseline:
        n_cpu = min(T, 4096)
        if w.layer is not None:
            out["cpu_baseline"] = cpu_baseline(w.layer, x_np[:n_cpu], params[0], one_thread=True)
        else:
            # Whole-stack rate: time one layer of each ratio on the oracle
            # (prefill over a 4096-token sample; with decode steps, also a
            # sample of single-token steps after it, two ratio-4 window
            # boundaries included) and weight by how many layers of each
            # ratio the stack has and how many tokens of each kind a step has.
            import oracle
            from tests._helpers import oracle_spec

            step_s, parts = 0.0, []
            for r in (4, 128):
                l_r = next(l for l, s in shapes if s is not None and s.ratio == r)
                n_r = sum(1 for _, s in shapes if s is not None and s.ratio == r)
                b = cpu_baseline(shapes[l_r][1], x_np[:n_cpu], params[l_r], budget_s=6.0)
                step_s += n_r * T / b["value"]
                part = f"ratio {r}: prefill {b['value']:.0f} tokens/s per layer"
                if Td:
                    spec = oracle_spec(shapes[l_r][1], params[l_r])
                    st = oracle.new_layer_state(spec)
                    oracle.prefill(spec, st, x_np[:n_cpu])
                    nd, td0 = 8, time.perf_counter()
                    for i in range(nd):
                        oracle.decode_one(spec, st, x_np[T + i])
                    dec_s = (time.perf_counter() - td0) / nd
                    step_s += n_r * Td * dec_s
                    part += f", decode {dec_s * 1e3:.1f} ms per token per layer ({nd} steps)"
                parts.append(part + f", x {n_r} layers")
            out["cpu_baseline"] = {"value": (T + Td) / step_s, "unit": "tokens/s", "cores": b["cores"],
                                   "kind": "oracle",
                                   "sample": f"{n_cpu}-token prefill steps of one layer of each ratio, about 6 s "
                                             f"each{', then single-token decode steps' if Td else ''}, combined "
                                             f"over the stack and a step's {T} prefill + {Td} decode tokens "
                                             f"({'; '.join(parts)}); float64 NumPy",
                                   "cpu_model": b.get("cpu_model"), "blas": b.get("blas"),
                                   "cpus_visible": b.get("cpus_visible")}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
