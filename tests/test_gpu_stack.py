"""The Flash- and Pro-pattern layer stacks through the native stack entry points.

32 layers (Flash: 0-1 uncompressed; Pro: 0-1 ratio 128; then even ratio 4,
odd ratio 128), hidden 4096,
head_dim 512 / indexer 128, bf16, independent weights per layer, every layer
fed the same hidden states.  One 4096-token chunk, and a 65536-token prompt in
16 chunks of 4096 followed by 256 single-token decode steps, at full size.
Row counts and counters are checked for every layer.  The one-chunk stack
compares every row of every layer; the long run compares, on every layer,
every row of the last prefill chunk and every row the decode steps emit, plus
sampled rows of earlier chunks (chunk edges, first rows), all against the
oracle's closed window form computed from the same inputs; the final frontier
of every layer is compared with the oracle's closed form.
"""

import numpy as np
import pytest
import torch

import oracle
from compressed_kv_attention_compressor_amd import binding as B
from compressed_kv_attention_compressor_amd import synth
from compressed_kv_attention_compressor_amd.layer import CompressorLayer, CompressorStack
from tests._helpers import oracle_spec
from tests.compare import check_attn_rows, check_index_rows, check_prequant

pytestmark = pytest.mark.gpu


def build_stack(workload, total_tokens):
    layers, specs = [], []
    for l in range(workload.n_layers):
        r = B.ds4c_layer_ratio(workload.variant, l)
        assert r == oracle.layer_compress_ratio(l, ("flash", "pro")[workload.variant])
        shape = synth.stack_layer_shape(r)
        if shape is None:
            layers.append(None)
            specs.append(None)
            continue
        p = synth.layer_params(workload.wid, l, shape)
        layers.append(CompressorLayer(r, shape.hidden, p, dtype=shape.dtype, max_tokens=total_tokens))
        specs.append((shape, oracle_spec(shape, p)))
    return CompressorStack(layers), specs


def token_maps(spec, x, toks):
    """Projections of the given absolute positions, as {kind: {p: row}} maps."""
    toks = sorted(set(t for t in toks if t >= 0))
    kv, sc = {}, {}
    for lane in spec.lanes():
        pk, ps = oracle.project(lane, x[toks])
        kv[lane.kind] = dict(zip(toks, pk))
        sc[lane.kind] = dict(zip(toks, ps))
    return kv, sc


def check_layer_rows(L, shape, spec, x, ks, n):
    r = shape.ratio
    toks = set()
    for k in ks:
        toks.update(range(4 * k - 4, 4 * k + 4) if r == 4 else range(128 * k, 128 * k + 128))
    m = n - n % r
    toks.update(range(m - 4 if r == 4 else m, n))
    kv, sc = token_maps(spec, x, toks)
    for lane in spec.lanes():
        k_name = lane.kind
        pre, fin = oracle.window_rows(spec, lane, kv[k_name], sc[k_name], ks)
        got = L.rows[k_name][torch.tensor(ks, device=L.rows[k_name].device)].cpu().numpy()
        if k_name == "attn":
            nst = check_attn_rows(got, fin, None, pre, shape.n_rot, f"attn rows {ks}")
        else:
            nst = check_index_rows(got, fin, None, pre, f"index rows {ks}")
        if nst:
            print(f"[straddle] {k_name}: {nst} codec blocks in {len(ks)} rows", flush=True)
    closed = oracle.frontier_from_tokens(spec, n, kv, sc)
    views = L.frontier_views()
    for lane in spec.lanes():
        kv_g, sc_g = (t.cpu().numpy() for t in views[lane.kind])
        kv_o, sc_o = closed[lane.kind]
        for row, _p in oracle.compressor.live_frontier_rows(r, n):
            check_prequant(kv_g[row], kv_o[row], f"frontier kv row {row}")
            check_prequant(sc_g[row], sc_o[row], f"frontier score row {row}")


def test_stack32_one_chunk():
    w = synth.WORKLOADS["stack32"]
    T = w.tokens
    print(f"[stack] {w.name}", flush=True)
    stack, specs = build_stack(w, T)
    x = synth.hidden_states(w.wid, 4096, 0, T, "bf16")
    stack.prefill(torch.from_numpy(x).to("cuda", torch.bfloat16))
    torch.cuda.synchronize()
    for l, L in enumerate(stack.layers):
        if L is None:
            continue
        r = L.ratio
        assert (L.frontier.n_tokens, L.frontier.n_comp, L.frontier.n_index_comp) == (T, T // r, T // 4 if r == 4 else 0)
        print(f"[stack] layer {l} ratio {r}: all {T // r} rows", flush=True)
        check_layer_rows(L, specs[l][0], specs[l][1], x, list(range(T // r)), T)


def test_stack32_long_prefill_then_decode():
    w = synth.WORKLOADS["stack32_long"]
    T, Td = w.tokens, w.decode_tokens
    print(f"[stack] {w.name}", flush=True)
    stack, specs = build_stack(w, T + Td)
    x = synth.hidden_states(w.wid, 4096, 0, T + Td, "bf16")
    xd = torch.from_numpy(x).to("cuda", torch.bfloat16)
    stack.prefill(xd[:T])  # 16 chunks of 4096 inside the library
    stack.decode(xd[T:T + Td])  # 256 single-token steps inside the library
    torch.cuda.synchronize()
    n = T + Td
    for l, L in enumerate(stack.layers):
        if L is None:
            continue
        r = L.ratio
        assert (L.frontier.n_tokens, L.frontier.n_comp, L.frontier.n_index_comp) == (n, n // r, n // 4 if r == 4 else 0)
        # every row of the last prefill chunk and of the decode steps; edges
        # and first rows of earlier chunks
        last_chunk = (T - 4096) // r
        edges = [0, 1, 1023 // (r // 4), 1024 // (r // 4), 8191 // (r // 4), 8192 // (r // 4)]
        ks = sorted(set(edges) | set(range(last_chunk, n // r)))
        print(f"[stack] layer {l} ratio {r}: {len(ks)} rows", flush=True)
        check_layer_rows(L, specs[l][0], specs[l][1], x, ks, n)


def test_stack32_pro_ragged_prompt_then_decode():
    """Pro schedule: a 5000-token prompt (chunks of 4096 and 904: the short chunk
    takes the plain K-split projection on ratio-4 layers and the fused path on
    ratio-128 layers), then 7 decode steps."""
    w = synth.WORKLOADS["stack32_pro"]
    T, Td = 5000, 7
    print(f"[stack] {w.name}: {T} prompt tokens in chunks of 4096, {Td} decode steps", flush=True)
    stack, specs = build_stack(w, T + Td)
    assert all(L is not None for L in stack.layers)
    x = synth.hidden_states(w.wid, 4096, 0, T + Td, "bf16")
    xd = torch.from_numpy(x).to("cuda", torch.bfloat16)
    stack.prefill(xd[:T], chunk_cap=4096)
    for i in range(Td):
        stack.decode_one(xd[T + i])
    torch.cuda.synchronize()
    n = T + Td
    for l, L in enumerate(stack.layers):
        r = L.ratio
        assert (L.frontier.n_tokens, L.frontier.n_comp, L.frontier.n_index_comp) == (n, n // r, n // 4 if r == 4 else 0)
        if l not in (0, 1, 2, 3, 30, 31):
            continue
        ks = [0, 1, 1023, 1024, 1025, 1249, 1250] if r == 4 else [0, 31, 32, 38]
        check_layer_rows(L, specs[l][0], specs[l][1], x, ks, n)
