"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Every case runs the same seeded inputs through both and compares
element by element with the rules of tests/compare.py: pre-codec values
within 2e-3 relative, codec outputs within one code, row counts, counters
and frontier -inf positions exact.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from compressed_kv_attention_compressor_amd import synth
from compressed_kv_attention_compressor_amd.layer import CompressorLayer
from tests._helpers import oracle_spec
from tests.compare import check_attn_rows, check_index_rows, check_prequant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _tdtype(shape):
    return torch.bfloat16 if shape.dtype == "bf16" else torch.float32


def make_gpu_layer(shape, params, max_tokens):
    return CompressorLayer(shape.ratio, shape.hidden, params, dtype=shape.dtype, n_rot=shape.n_rot,
                           rope_base=shape.rope_base, rms_eps=shape.rms_eps, max_tokens=max_tokens)


def run_gpu(shape, params, x, plan):
    """plan: list of chunk sizes; a negative entry -n means n single decode steps."""
    layer = make_gpu_layer(shape, params, len(x))
    xd = torch.from_numpy(x).to("cuda", _tdtype(shape))
    pre = {k: [] for k in layer.kinds}
    t = 0
    for step in plan:
        if step >= 0:
            got = layer.prefill(xd[t:t + step], prequant=True)
            t += step
        else:
            got = {k: [] for k in layer.kinds}
            for _ in range(-step):
                one = layer.decode_one(xd[t], prequant=True)
                for k in layer.kinds:
                    got[k].append(one[k])
                t += 1
            got = {k: torch.cat(v) for k, v in got.items()}
        for k in layer.kinds:
            pre[k].append(got[k].cpu().numpy())
    assert t == len(x)
    torch.cuda.synchronize()
    out = {
        "rows": {k: layer.live_rows(k).cpu().numpy() for k in layer.kinds},
        "pre": {k: np.concatenate(v) for k, v in pre.items()},
        "frontier": {k: (kv.cpu().numpy(), sc.cpu().numpy()) for k, (kv, sc) in layer.frontier_views().items()},
        "counters": (layer.frontier.n_tokens, layer.frontier.n_comp, layer.frontier.n_index_comp),
        "layer": layer,
    }
    return out


def run_oracle(shape, params, x):
    spec = oracle_spec(shape, params)
    st = oracle.new_layer_state(spec)
    oracle.prefill(spec, st, x)
    return spec, st


def compare_all(shape, g, spec, st, n):
    r = shape.ratio
    assert g["counters"] == (n, n // r, n // 4 if r == 4 else 0)
    for lane in spec.lanes():
        k = lane.kind
        o_rows = np.array(st.lanes[k].rows).reshape(-1, lane.head_dim)
        o_pre = np.array(st.lanes[k].prequant).reshape(-1, lane.head_dim)
        assert g["rows"][k].shape == o_rows.shape
        check_prequant(g["pre"][k], o_pre, f"{k} prequant")
        if k == "attn":
            nst = check_attn_rows(g["rows"][k], o_rows, g["pre"][k], o_pre, shape.n_rot)
        else:
            nst = check_index_rows(g["rows"][k], o_rows, g["pre"][k], o_pre)
        _say(f"[straddle] {k}: {nst} of {o_rows.size // (64 if k == 'attn' else 32)} codec blocks")
        # live frontier rows, pre-quant tolerance; -inf positions exact
        kv_g, sc_g = g["frontier"][k]
        for row, _tok in oracle.compressor.live_frontier_rows(r, n):
            kv_o, sc_o = st.lanes[k].kv[row], st.lanes[k].score[row]
            assert np.array_equal(np.isneginf(sc_g[row]), np.isneginf(sc_o))
            fin = np.isfinite(sc_o)
            check_prequant(kv_g[row], kv_o, f"{k} frontier kv row {row}")
            check_prequant(sc_g[row][fin], sc_o[fin], f"{k} frontier score row {row}")


def _workload(name):
    w = synth.WORKLOADS[name]
    p = synth.layer_params(w.wid, 0, w.layer)
    x = synth.hidden_states(w.wid, w.layer.hidden, 0, w.tokens, w.layer.dtype)
    return w, p, x


@pytest.mark.parametrize("name", ["r4_small", "r4_flash", "r128_flash"])
def test_workload_one_call(name):
    _say(f"[parity] {name} one call")
    w, p, x = _workload(name)
    g = run_gpu(w.layer, p, x, [len(x)])
    spec, st = run_oracle(w.layer, p, x)
    compare_all(w.layer, g, spec, st, len(x))


SMALL = {
    "r4_d128": synth.LayerShape(ratio=4, hidden=256, d_attn=128, d_index=64, dtype="f32"),
    "r4_d512_bf16": synth.LayerShape(ratio=4, hidden=256, d_attn=512, d_index=128, dtype="bf16"),
    "r4_d256_idx512": synth.LayerShape(ratio=4, hidden=128, d_attn=256, d_index=512, dtype="bf16"),
    "r128_d512": synth.LayerShape(ratio=128, hidden=256, d_attn=512, d_index=0, dtype="bf16"),
    "r128_d128_f32": synth.LayerShape(ratio=128, hidden=192, d_attn=128, d_index=0, dtype="f32"),
    # three 64-wide K tiles: the ratio-128 projection's odd-tile tail
    "r128_d256_h192_bf16": synth.LayerShape(ratio=128, hidden=192, d_attn=256, d_index=0, dtype="bf16"),
    # a 128-dim RoPE tail: two FP8 blocks on the attention lane, the whole indexer row rotated
    "r4_d256_rot128": synth.LayerShape(ratio=4, hidden=256, d_attn=256, d_index=128, dtype="bf16", n_rot=128),
    # RoPE over the whole row: no FP8 dims on the attention lane
    "r128_d128_rot128_f32": synth.LayerShape(ratio=128, hidden=192, d_attn=128, d_index=0, dtype="f32", n_rot=128),
}


def _small(name, n, seed=0, random_norm=True):
    shape = SMALL[name]
    p = synth.layer_params(90 + list(SMALL).index(name), 0, shape, seed=seed, random_norm=random_norm)
    x = synth.hidden_states(90 + list(SMALL).index(name), shape.hidden, 0, n, shape.dtype, seed=seed)
    return shape, p, x


PLANS = {
    "ragged": [1, 3, 5, 127, 129, 2, 64, 300, 69],
    "decode_mix": [3, -6, 130, -3, 1, 120, -130, 337],
    "aligned": [256, 256, 188],
    # calls on window boundaries spanning several 256-token tiles, short tails
    "aligned_long": [4, 600, 64, 5, 3],
    # fused calls over several 256-token tiles whose length leaves 7 tokens for
    # the ratio-4 frontier (T % 4 == 3) in a 3-token last tile, the second
    # starting from the frontier the decode steps left; at ratio 128 the first
    # leaves 3 tokens of an open window
    "fused_ragged": [1027, -5, 1031, 2],
}


@pytest.mark.parametrize("plan", list(PLANS))
@pytest.mark.parametrize("name", list(SMALL))
def test_chunked_and_decode(name, plan):
    n = sum(abs(s) for s in PLANS[plan])
    _say(f"[parity] {name} plan {plan} n={n}")
    shape, p, x = _small(name, n)
    g = run_gpu(shape, p, x, PLANS[plan])
    spec, st = run_oracle(shape, p, x)
    compare_all(shape, g, spec, st, n)


def random_plan(seed, n_calls=10):
    """A seeded mix of call kinds: short prefills (1-7 tokens), ragged ones
    (8-599), runs of single decode steps, and window-multiple lengths (4,
    128, 256, 1100: on a window boundary these take the fused paths, which
    need more than 1024 tokens at ratio 4 and more than 256 at ratio 128)."""
    rng = np.random.default_rng(seed)
    plan = []
    for _ in range(n_calls):
        kind = int(rng.integers(0, 4))
        if kind == 0:
            plan.append(int(rng.integers(1, 8)))
        elif kind == 1:
            plan.append(int(rng.integers(8, 600)))
        elif kind == 2:
            plan.append(-int(rng.integers(1, 10)))
        else:
            plan.append(int(rng.choice([4, 128, 256, 1100])))
    return plan


@pytest.mark.parametrize("seed", [11, 12, 13])
@pytest.mark.parametrize("name", list(SMALL))
def test_random_chunk_plans(name, seed):
    plan = random_plan(1000 * list(SMALL).index(name) + seed)
    n = sum(abs(s) for s in plan)
    _say(f"[parity] {name} random plan {plan} n={n}")
    shape, p, x = _small(name, n, seed=seed)
    g = run_gpu(shape, p, x, plan)
    spec, st = run_oracle(shape, p, x)
    compare_all(shape, g, spec, st, n)


# The largest hidden size the boundary accepts (16384), and fp32 at 4096:
# decode dot products then run over several unrolled chunks, the prefill
# GEMM over its longest K loop.
LARGE_K = {
    "r4_h16384_bf16": (synth.LayerShape(ratio=4, hidden=16384, d_attn=128, d_index=64, dtype="bf16"), [5, -7, 9, -3]),
    "r128_h4096_f32": (synth.LayerShape(ratio=128, hidden=4096, d_attn=128, d_index=0, dtype="f32"), [100, -40, 20]),
}


@pytest.mark.parametrize("name", list(LARGE_K))
def test_large_hidden_decode(name):
    shape, plan = LARGE_K[name]
    n = sum(abs(s) for s in plan)
    _say(f"[parity] {name} plan {plan} n={n}")
    wid = 80 + list(LARGE_K).index(name)
    p = synth.layer_params(wid, 0, shape)
    x = synth.hidden_states(wid, shape.hidden, 0, n, shape.dtype)
    g = run_gpu(shape, p, x, plan)
    spec, st = run_oracle(shape, p, x)
    compare_all(shape, g, spec, st, n)


@pytest.mark.parametrize("name", ["r4_d128", "r128_d512"])
def test_single_tokens_and_tiny_calls(name):
    _say(f"[parity] {name} tiny calls")
    shape, p, x = _small(name, 260, seed=3)
    plan = [1] * 9 + [-1] * 7 + [0, 2, 0] + [242]
    g = run_gpu(shape, p, x, plan)
    spec, st = run_oracle(shape, p, x)
    compare_all(shape, g, spec, st, 260)


@pytest.mark.parametrize("name", ["r4_d512_bf16", "r128_d512"])
def test_save_load_continue(name):
    _say(f"[parity] {name} save/load")
    shape, p, x = _small(name, 600, seed=5)
    xd = torch.from_numpy(x).to("cuda", _tdtype(shape))
    spec_full, st_full = run_oracle(shape, p, x)
    for cut in (0, 3, 131, 259):
        a = make_gpu_layer(shape, p, 600)
        pre_a = a.prefill(xd[:cut], prequant=True)
        blob = a.save()
        # the blob's header and live rows match the oracle's canonical frontier
        spec, st = run_oracle(shape, p, x[:cut])
        hdr = np.frombuffer(blob[:32], dtype="<u4")
        cnt = np.frombuffer(blob[32:56], dtype="<u8")
        assert list(hdr) == [0x46345344, 1, shape.ratio, shape.coff, shape.d_attn, shape.d_index, 64, 0]
        assert list(cnt) == [cut, cut // shape.ratio, cut // 4 if shape.ratio == 4 else 0]
        body = np.frombuffer(blob[56:], dtype="<f4")
        canon = oracle.canonical_frontier(spec, st)
        off = 0
        for lane in spec.lanes():
            kv_o, sc_o = canon[lane.kind]
            m = kv_o.size
            kv_g = body[off:off + m].reshape(kv_o.shape)
            sc_g = body[off + m:off + 2 * m].reshape(sc_o.shape)
            off += 2 * m
            assert np.array_equal(np.isneginf(sc_g), np.isneginf(sc_o))
            fin = np.isfinite(sc_o)
            check_prequant(kv_g, kv_o, "blob kv")
            check_prequant(sc_g[fin], sc_o[fin], "blob score")
        assert off == body.size
        # a second save of the same state is byte-identical
        assert a.save() == blob
        # load into a fresh layer (with garbage in its frontier) and continue
        b = make_gpu_layer(shape, p, 600)
        b.prefill(xd[300:300 + 37])  # scribble on b's frontier first
        b.load(blob)
        assert b.frontier.n_tokens == cut
        b.rows = {k: v.clone() for k, v in b.rows.items()}
        for k in b.kinds:
            b.rows[k][: cut // shape.ratio] = a.rows[k][: cut // shape.ratio]
        pre_b = b.prefill(xd[cut:], prequant=True)
        torch.cuda.synchronize()
        # The continued state matches the oracle's uninterrupted run.  (The
        # rows are bitwise equal to `full`'s only when both runs use the same
        # projection tiling; a call that starts on a window boundary takes
        # the fused path, so they are compared at the parity tolerances.)
        g = {
            "rows": {k: b.live_rows(k).cpu().numpy() for k in b.kinds},
            "pre": {k: np.concatenate([pre_a[k].cpu().numpy(), pre_b[k].cpu().numpy()]) for k in b.kinds},
            "frontier": {k: (kv.cpu().numpy(), sc.cpu().numpy()) for k, (kv, sc) in b.frontier_views().items()},
            "counters": (b.frontier.n_tokens, b.frontier.n_comp, b.frontier.n_index_comp),
            "layer": b,
        }
        compare_all(shape, g, spec_full, st_full, 600)


# Flash-size calls of every length class: a call with few output tiles runs
# the plain projection with K split over up to 16 ranges (planes added in a
# second launch), a long call on a window boundary pools in the projection
# epilogue, and ragged lengths cover partial tiles on both paths.
FLASH_PLANS = {
    "r4_flash": [1, 3, 256, 127, 1, 1536, 2172],
    "r128_flash": [1, 127, 64, 64, 2500, 1340],
}


@pytest.mark.parametrize("name", list(FLASH_PLANS))
def test_flash_short_and_ragged_calls(name):
    plan = FLASH_PLANS[name]
    _say(f"[parity] {name} plan {plan}")
    w, p, x = _workload(name)
    assert sum(plan) == len(x)
    g = run_gpu(w.layer, p, x, plan)
    spec, st = run_oracle(w.layer, p, x)
    compare_all(w.layer, g, spec, st, len(x))


def test_deterministic_and_overwrites_poison():
    _say("[parity] determinism")
    w, p, x = _workload("r4_flash")
    xd = torch.from_numpy(x).to("cuda", torch.bfloat16)
    outs = []
    for _ in range(2):
        layer = make_gpu_layer(w.layer, p, len(x))
        for v in layer.rows.values():
            v.fill_(float("nan"))
        layer.prefill(xd)
        torch.cuda.synchronize()
        for k in layer.kinds:
            assert torch.isfinite(layer.live_rows(k)).all()
        outs.append({k: layer.live_rows(k).clone() for k in layer.kinds})
    for k in outs[0]:
        assert torch.equal(outs[0][k], outs[1][k])


@pytest.mark.parametrize("name", list(FLASH_PLANS))
def test_short_calls_are_deterministic(name):
    """The K-split projection adds its planes in a fixed order: two runs of the
    same ragged plan give bitwise-equal rows and frontiers."""
    _say(f"[parity] {name} short-call determinism")
    w, p, x = _workload(name)
    plan = [1, 3, 64, 127, 256, 600]
    runs = [run_gpu(w.layer, p, x[:sum(plan)], plan) for _ in range(2)]
    for k in runs[0]["rows"]:
        assert np.array_equal(runs[0]["rows"][k], runs[1]["rows"][k])
        assert np.array_equal(runs[0]["pre"][k], runs[1]["pre"][k])
        for a_, b_ in zip(runs[0]["frontier"][k], runs[1]["frontier"][k]):
            assert np.array_equal(a_, b_)


def test_row_zero_of_ratio4_pools_current_half_only():
    """Equal scores (zero gate weights and APE) make row 0 the mean of 4 tokens."""
    _say("[parity] equal-score row 0")
    shape = SMALL["r4_d128"]
    p = synth.layer_params(99, 0, shape)
    for k in p:
        p[k]["wgate"][:] = 0
        p[k]["ape"][:] = 0
    x = synth.hidden_states(99, shape.hidden, 0, 12, "f32")
    g = run_gpu(shape, p, x, [12])
    spec, st = run_oracle(shape, p, x)
    compare_all(shape, g, spec, st, 12)


# Score edge cases through every path (fused and plain prefill of both
# ratios, decode steps): every score of every window shifted by +-1000 (the
# pool's max subtraction; e^1000 overflows without it), and one entry per
# window planted 60 above the rest (the pool then returns that entry's kv).
# The oracle's pins hold both cases to closed forms; here the GPU must match
# the oracle on the same extreme inputs.
EDGE_PLANS = {"ragged": PLANS["ragged"], "decode_mix": PLANS["decode_mix"], "aligned_long": PLANS["aligned_long"]}


def _edge_params(shape, p, mode):
    p = {k: {kk: (vv.copy() if isinstance(vv, np.ndarray) else vv) for kk, vv in v.items()} for k, v in p.items()}
    for kind, lane in p.items():
        d = lane["head_dim"]
        if mode == "shift+1000":
            lane["ape"] += np.float32(1000.0)
        elif mode == "shift-1000":
            lane["ape"] -= np.float32(1000.0)
        else:
            # ratio 4: the current half's token at p % 4 == 2 (columns [D, 2D));
            # ratio 128: the token at p % 128 == 5
            row = 2 if shape.ratio == 4 else 5
            c0 = d if shape.ratio == 4 else 0
            lane["ape"][row, c0:c0 + d] += np.float32(60.0)
    return p


@pytest.mark.parametrize("mode", ["shift+1000", "shift-1000", "argmax+60"])
@pytest.mark.parametrize("plan", list(EDGE_PLANS))
@pytest.mark.parametrize("name", ["r4_d512_bf16", "r128_d512"])
def test_score_extremes(name, plan, mode):
    n = sum(abs(s) for s in EDGE_PLANS[plan])
    _say(f"[parity] {name} plan {plan} scores {mode} n={n}")
    shape, p, x = _small(name, n, seed=7)
    p = _edge_params(shape, p, mode)
    g = run_gpu(shape, p, x, EDGE_PLANS[plan])
    spec, st = run_oracle(shape, p, x)
    compare_all(shape, g, spec, st, n)
    if mode == "argmax+60":
        # the planted entry dominates: the pooled value (before the norm) of
        # every full window is that token's kv to within e^-60 of the rest
        lane = spec.attn
        pooled = np.array(st.lanes["attn"].pooled)
        kv_all, _ = oracle.project(lane, x)
        d, r = lane.head_dim, shape.ratio
        for k in range(1, len(pooled)):
            t = 4 * k + 2 if r == 4 else 128 * k + 5
            want = kv_all[t][d:2 * d] if r == 4 else kv_all[t][:d]
            assert np.allclose(pooled[k], want, rtol=1e-12, atol=1e-12)
