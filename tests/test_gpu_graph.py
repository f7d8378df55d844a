"""GPU: the library's calls captured in HIP graphs replay exactly like eager calls.

The decode steps of a two-layer stack (ratio 4 and ratio 128, bf16, crossing
window boundaries of both ratios) and whole prefill calls of single layers
(the fused paths) are captured once and replayed several times.  Between the
replays the program does its own eager work: frontier re-initialisation, an
eager prefill, unrelated torch kernels and synchronisations.  After every
replay the emitted rows and the frontier tensors must equal the eager run's
bit for bit.  The library records no memset nodes (its frontier
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
