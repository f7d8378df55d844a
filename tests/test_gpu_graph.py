"""GPU: the library's calls captured in HIP graphs replay exactly like eager calls.

The decode steps of a two-layer stack (ratio 4 and ratio 128, bf16, crossing
window boundaries of both ratios), whole prefill calls of single layers (the
fused paths), and an indexer call with a mixed-attention call are captured
once and replayed several times.  Between the
replays the program does its own eager work: frontier re-initialisation, an
eager prefill, unrelated torch kernels and synchronisations.  After every
replay the emitted rows and the frontier tensors (or the selection and the
attention output) must equal the eager run's bit for bit.  The library records no memset nodes (its frontier
initialisation is a fill kernel), so nothing here depends on how a captured
memset replays.
"""

import pytest
import torch

from compressed_kv_attention_compressor_amd import synth
from compressed_kv_attention_compressor_amd.layer import CompressorLayer, CompressorStack

pytestmark = pytest.mark.gpu

R4 = synth.LayerShape(ratio=4, hidden=256, d_attn=512, d_index=128, dtype="bf16")
R128 = synth.LayerShape(ratio=128, hidden=256, d_attn=512, d_index=0, dtype="bf16")
WID = 120  # workload id of these inputs


def _layer(shape, l, n):
    p = synth.layer_params(WID, l, shape, random_norm=True)
    return CompressorLayer(shape.ratio, shape.hidden, p, dtype=shape.dtype, n_rot=shape.n_rot,
                           rope_base=shape.rope_base, rms_eps=shape.rms_eps, max_tokens=n)


def _state(layers, n):
    out = []
    for L in layers:
        out += [v[:n // L.ratio].clone() for v in L.rows.values()]
        out += [t.clone() for pair in L.frontier_views().values() for t in pair]
    return out


def _poison(layers):
    for L in layers:
        for v in L.rows.values():
            v.fill_(float("nan"))


def _eager_noise():
    """Unrelated eager work of the program between replays."""
    a = torch.randn(512, 512, device="cuda")
    (a @ a).sum().item()


def _same(got, ref):
    return len(got) == len(ref) and all(torch.equal(a, b) for a, b in zip(got, ref))


def test_stack_decode_graph_replays_match_eager():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    T, Td = 120, 12  # decode positions 120..131: ratio-4 rows at 123, 127, 131; ratio-128 row at 127
    n = T + Td
    x = torch.from_numpy(synth.hidden_states(WID, 256, 0, n, "bf16")).to("cuda", torch.bfloat16)
    layers = [_layer(R4, 0, n), _layer(R128, 1, n)]
    stack = CompressorStack(layers)

    def reinit():
        for L in layers:
            L.reset()

    reinit()
    stack.prefill(x[:T])
    stack.decode(x[T:n])
    torch.cuda.synchronize()
    assert [(L.frontier.n_tokens, L.frontier.n_comp) for L in layers] == [(n, n // 4), (n, n // 128)]
    ref = _state(layers, n)

    reinit()
    stack.prefill(x[:T])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        stack.decode(x[T:n])  # enqueued into the graph, not run
    for rep in range(3):
        print(f"[graph] stack decode replay {rep}", flush=True)
        _poison(layers)
        reinit()
        stack.prefill(x[:T])
        _eager_noise()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(_state(layers, n), ref), f"replay {rep}"


@pytest.mark.parametrize("shape", [R4, R128], ids=["r4", "r128"])
def test_prefill_graph_replays_match_eager(shape):
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    T = 1100  # on a window boundary and long enough for the fused paths of both ratios
    x = torch.from_numpy(synth.hidden_states(WID + 1, 256, 0, T, "bf16")).to("cuda", torch.bfloat16)
    L = _layer(shape, 2, T)
    L.reset()
    L.prefill(x)
    torch.cuda.synchronize()
    ref = _state([L], T)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        L.reset()
        L.prefill(x)
    for rep in range(3):
        print(f"[graph] ratio {shape.ratio} prefill replay {rep}", flush=True)
        _poison([L])
        L.reset()
        L.prefill(x[:T // 2])  # eager work on the same layer: a different state before the replay
        _eager_noise()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(_state([L], T), ref), f"replay {rep}"


def test_indexer_and_mixed_attention_graph_replays_match_eager():
    """An indexer call over two 32768-row chunks (score, per-chunk select and
    final select launches) and a mixed-attention call, captured together and
    replayed with unrelated eager work and poisoned outputs in between."""
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    from compressed_kv_attention_compressor_amd import binding as B

    n, H, Dh, k = 40000, 64, 128, 512
    q_np, w_np, rows_np = synth.indexer_inputs(WID + 2, n, H, Dh)
    q, hw, rows = (torch.from_numpy(a).cuda() for a in (q_np, w_np, rows_np))
    idx = torch.empty(k, dtype=torch.int32, device="cuda")
    sc = torch.empty(k, dtype=torch.float32, device="cuda")
    ws = torch.empty(B.ds4c_indexer_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
    nc, D, ring_cap = 4096, 512, 128
    qa_np, ring_np, comp_np, topk_np = synth.mixed_attention_inputs(WID + 3, nc, H, D, ring_cap, k)
    qa, ring, comp = (torch.from_numpy(a).cuda() for a in (qa_np, ring_np, comp_np))
    topk = torch.from_numpy(topk_np).cuda()
    out = torch.empty(H, D, dtype=torch.float32, device="cuda")
    wsa = torch.empty(B.ds4c_mixed_attention_workspace_bytes(H, D, ring_cap, k), dtype=torch.uint8, device="cuda")
    qpos = 4 * nc - 1

    def calls():
        s = torch.cuda.current_stream().cuda_stream
        B.ds4c_indexer_topk(q.data_ptr(), hw.data_ptr(), H, Dh, rows.data_ptr(), n, k, idx.data_ptr(),
                            sc.data_ptr(), 0, 0, ws.data_ptr(), ws.numel(), s)
        B.ds4c_mixed_attention(qa, ring, qpos + 1 - ring_cap, qpos, ring_cap, comp, topk, qpos, 4, out, wsa, s)

    calls()
    torch.cuda.synchronize()
    ref = [idx.clone(), sc.clone(), out.clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()  # enqueued into the graph, not run
    for rep in range(3):
        print(f"[graph] indexer + mixed attention replay {rep}", flush=True)
        idx.fill_(-1)
        sc.fill_(float("nan"))
        out.fill_(float("nan"))
        ws.fill_(0xAB)
        _eager_noise()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same([idx, sc, out], ref), f"replay {rep}"
