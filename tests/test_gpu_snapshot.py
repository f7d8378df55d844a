"""Stack snapshot (the compressor sections of a session payload) on the GPU.

A Pro-schedule stack at small shapes is run to a mid-window position, saved,
restored into a second stack whose state was scribbled on first, and both
stacks continue with the same calls: rows, frontiers and a second snapshot
must then be bitwise equal (the same kernels run on the same inputs).  The
blob's header, counts, row sections and canonical frontier rows are checked
against the device state and against the oracle's closed frontier form.
"""

import struct

import numpy as np
import pytest
import torch

import oracle
from compressed_kv_attention_compressor_amd import binding as B
from compressed_kv_attention_compressor_amd import synth
from compressed_kv_attention_compressor_amd.layer import CompressorLayer, CompressorStack
from tests._helpers import oracle_spec
from tests.compare import check_prequant

pytestmark = pytest.mark.gpu

SHAPES = {4: synth.LayerShape(ratio=4, hidden=256, d_attn=128, d_index=64, dtype="bf16"),
          128: synth.LayerShape(ratio=128, hidden=256, d_attn=256, d_index=0, dtype="bf16")}
WID = 60


def make_stack(n_layers=6, max_tokens=2048, d128=256):
    layers, specs = [], []
    for l in range(n_layers):
        r = B.ds4c_layer_ratio(1, l)  # Pro: 128, 128, 4, 128, 4, 128
        shape = SHAPES[r] if r == 4 else synth.LayerShape(ratio=128, hidden=256, d_attn=d128, d_index=0, dtype="bf16")
        p = synth.layer_params(WID, l, shape, random_norm=True)
        layers.append(CompressorLayer(r, 256, p, dtype="bf16", max_tokens=max_tokens))
        specs.append((shape, p))
    return CompressorStack(layers), specs


def run(stack, xd, plan):
    t = 0
    for step in plan:
        if step > 0:
            stack.prefill(xd[t:t + step])
            t += step
        else:
            for _ in range(-step):
                stack.decode_one(xd[t])
                t += 1
    return t


def test_snapshot_round_trip_and_continue():
    print("[snapshot] 6-layer Pro stack, save at 1003 tokens, restore, continue", flush=True)
    x = synth.hidden_states(WID, 256, 0, 1600, "bf16")
    xd = torch.from_numpy(x).to("cuda", torch.bfloat16)
    a, specs = make_stack()
    n = run(a, xd, [1000, -3])
    blob = a.snapshot()
    torch.cuda.synchronize()
    L = len(a.layers)
    assert len(blob) == B.ds4c_stack_snapshot_bytes(a.c_layers, n)
    magic, ver, nl, zero, nt = struct.unpack_from("<IIIIQ", blob, 0)
    assert (magic, ver, nl, zero, nt) == (0x53345344, 1, L, 0, n)
    counts = struct.unpack_from(f"<{2 * L}I", blob, 24 + 16 * L)
    assert list(counts[:L]) == [n // layer.ratio for layer in a.layers]
    assert list(counts[L:]) == [n // 4 if layer.ratio == 4 else 0 for layer in a.layers]
    body = np.frombuffer(blob, dtype="<f4", offset=24 + 24 * L)
    # sections in payload order: attention rows, attention frontiers, indexer rows, indexer frontiers
    off = 0
    sections = {}
    for kind in ("attn_rows", "attn_fr", "index_rows", "index_fr"):
        for l, layer in enumerate(a.layers):
            lane = "attn" if kind.startswith("attn") else "index"
            if lane not in layer.kinds:
                continue
            if kind.endswith("rows"):
                m = layer.live_rows(lane).numel()
                sections[(kind, l)] = body[off:off + m]
            else:
                kv, sc = layer.frontier_views()[lane]
                m = kv.numel()
                sections[(kind, l)] = (body[off:off + m].reshape(kv.shape), body[off + m:off + 2 * m].reshape(kv.shape))
                m *= 2
            off += m
    assert off == body.size
    for l, layer in enumerate(a.layers):
        r = layer.ratio
        spec = oracle_spec(*specs[l])
        for lane in layer.kinds:
            rows = sections[(("attn" if lane == "attn" else "index") + "_rows", l)]
            assert np.array_equal(rows, layer.live_rows(lane).cpu().numpy().ravel())
            kv_b, sc_b = sections[(("attn" if lane == "attn" else "index") + "_fr", l)]
            kv_g, sc_g = (t.cpu().numpy() for t in layer.frontier_views()[lane])
            live = {row for row, _ in oracle.compressor.live_frontier_rows(r, n)}
            for row in range(kv_g.shape[0]):
                if row in live:
                    assert np.array_equal(kv_b[row], kv_g[row]) and np.array_equal(sc_b[row], sc_g[row])
                else:
                    assert not kv_b[row].any() and np.isneginf(sc_b[row]).all()
        # live frontier rows against the oracle's closed form
        toks = list(range(max(0, n - n % r - (4 if r == 4 else 0)), n))
        kv, sc = {}, {}
        for lane in spec.lanes():
            pk, ps = oracle.project(lane, x[toks])
            kv[lane.kind], sc[lane.kind] = dict(zip(toks, pk)), dict(zip(toks, ps))
        closed = oracle.frontier_from_tokens(spec, n, kv, sc)
        for lane in spec.lanes():
            kv_b, sc_b = sections[(("attn" if lane.kind == "attn" else "index") + "_fr", l)]
            for row, _p in oracle.compressor.live_frontier_rows(r, n):
                check_prequant(kv_b[row], closed[lane.kind][0][row], f"layer {l} {lane.kind} kv row {row}")
                check_prequant(sc_b[row], closed[lane.kind][1][row], f"layer {l} {lane.kind} score row {row}")

    b, _ = make_stack()
    run(b, xd, [37, -2])  # scribble on b's rows and frontiers
    b.restore(blob)
    assert [layer.frontier.n_tokens for layer in b.layers] == [n] * L
    for la, lb in zip(a.layers, b.layers):
        for k in la.kinds:
            assert torch.equal(la.live_rows(k), lb.live_rows(k))
    plan = [1, 300, -5, 128, 97]
    run(a, xd[n:], plan)
    run(b, xd[n:], plan)
    torch.cuda.synchronize()
    for la, lb in zip(a.layers, b.layers):
        assert (la.frontier.n_tokens, la.frontier.n_comp, la.frontier.n_index_comp) == \
               (lb.frontier.n_tokens, lb.frontier.n_comp, lb.frontier.n_index_comp)
        for k in la.kinds:
            assert torch.equal(la.live_rows(k), lb.live_rows(k))
    assert a.snapshot() == b.snapshot()


def test_snapshot_refused_by_a_different_stack():
    print("[snapshot] refusal", flush=True)
    x = synth.hidden_states(WID, 256, 0, 300, "bf16")
    xd = torch.from_numpy(x).to("cuda", torch.bfloat16)
    a, _ = make_stack()
    run(a, xd, [300])
    blob = a.snapshot()
    c, _ = make_stack(d128=128)  # ratio-128 layers with another head dim
    with pytest.raises(B.DS4CError) as e:
        c.restore(blob)
    assert e.value.status == B.DS4C_EFORMAT
    assert all(layer.frontier.n_tokens == 0 for layer in c.layers)
    small, _ = make_stack(max_tokens=128)  # row buffers too small for 300 tokens
    with pytest.raises(B.DS4CError) as e:
        small.restore(blob)
    assert e.value.status == B.DS4C_ECAP
