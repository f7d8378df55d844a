"""Throughput of the compressed-KV compressor on one MI355X.

A step is one ds4c_compress_prefill call over one 4096-token chunk of a
layer (projection GEMM + fused store/pool/norm/RoPE/codec/append/frontier
kernel), starting at position 0 each time (the frontier counters are reset on
the host; a call at position 0 reads nothing from the frontier).  Inputs are
resident in HBM before timing.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload r4_flash|r128_flash]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def algorithmic(shape, T):
    """GEMM flops and pool-kernel bytes of one call at position 0."""
    lanes = [shape.d_attn] + ([shape.d_index] if shape.d_index else [])
    W = [shape.coff * d for d in lanes]
    N = 2 * sum(W)
    flops = 2.0 * T * N * shape.hidden
    n = T
    n_emit = T // shape.ratio
    c = n % shape.ratio
    m = n - c
    if shape.ratio == 4:
        live = (4 if m >= 4 else 0) + c
    else:
        live = c
    bytes_ = (T * N * 4                                  # kv + score read once
              + shape.ratio * sum(W) * 4                  # APE
              + n_emit * sum(lanes) * 4                   # rows written
              + live * sum(W) * 2 * 4)                    # frontier written
    return flops, bytes_, n_emit * len(lanes), N


def cpu_baseline(workload, x, params, budget_s=12.0):
    """The oracle as it is, timed on this host over whole 4096-token steps."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from tests._helpers import oracle_spec

    spec = oracle_spec(workload.layer, params)
    steps, t0 = 0, time.perf_counter()
    while True:
        st = oracle.new_layer_state(spec)
        oracle.prefill(spec, st, x)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 50:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": steps * len(x) / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{steps} full {len(x)}-token prefill steps of the same layer ({el:.1f} s); "
                      f"float64 NumPy, BLAS threads {threads}, Python recurrence single-threaded"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="r4_flash", choices=["r4_flash", "r128_flash"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus must be 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from compressed_kv_attention_compressor_amd import binding as B
    from compressed_kv_attention_compressor_amd import synth
    from compressed_kv_attention_compressor_amd.layer import CompressorLayer

    w = synth.WORKLOADS[args.workload]
    shape, T = w.layer, w.tokens
    params = synth.layer_params(w.wid, 0, shape)
    x_np = synth.hidden_states(w.wid, shape.hidden, 0, T, shape.dtype)
    layer = CompressorLayer(shape.ratio, shape.hidden, params, dtype=shape.dtype, n_rot=shape.n_rot,
                            rope_base=shape.rope_base, rms_eps=shape.rms_eps, max_tokens=T)
    x = torch.from_numpy(x_np).to("cuda", torch.bfloat16 if shape.dtype == "bf16" else torch.float32)
    layer.reserve(T)
    flops, pool_bytes, rows_per_step, N = algorithmic(shape, T)

    def step():
        f = layer.frontier
        f.n_tokens = f.n_comp = f.n_index_comp = 0
        layer.prefill(x)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    B.ds4c_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms, cnt = B.ds4c_profile_read()
    B.ds4c_profile_enable(False)

    gemm_ms = ms[B.KCLASS_PROJ] / max(cnt[B.KCLASS_PROJ], 1)
    pool_ms = ms[B.KCLASS_POOL] / max(cnt[B.KCLASS_POOL], 1)
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    pool_gbs = pool_bytes / (pool_ms * 1e-3) / 1e9
    peak = PEAK_BF16_TFLOPS if shape.dtype == "bf16" else PEAK_FP32_TFLOPS
    tokens_per_s = args.steps * T / el

    out = {
        "metric": "compressor tokens/sec + compressed rows/sec; % HBM and MFMA peak (1 GPU)",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": el / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": shape.dtype,
        "data": "synthetic (seeded N(0,1) hidden states, N(0,0.02) weights, N(0,0.1) APE)",
        "config": {"workload": w.name, "ratio": shape.ratio, "tokens": T, "hidden": shape.hidden,
                   "head_dim": shape.d_attn, "index_head_dim": shape.d_index, "chunk": T,
                   "gemm_mnk": [T, N, shape.hidden]},
        "rows_per_s": args.steps * rows_per_step / el,
        "roofline": {"bound": "mfma", "achieved": gemm_tflops, "peak": peak, "unit": "TFLOP/s",
                     "frac": gemm_tflops / peak, "traffic": None, "kernel": "proj_gemm",
                     "avg_ms": gemm_ms},
        "pool_roofline": {"bound": "hbm", "achieved": pool_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": pool_gbs / PEAK_HBM_GBS, "traffic": None, "kernel": "pool",
                          "avg_ms": pool_ms, "algorithmic_bytes": pool_bytes},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x_np, params)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
