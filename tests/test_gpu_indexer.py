"""Indexer scoring and top-k on the GPU against the oracle (oracle/indexer.py).

Each case checks, through the C ABI:
* the rotated, quantised query against the oracle's (one E2M1 code per
  value with equal block exponents; straddling blocks at the coarser grid);
* every row's score against the float64 score of the GPU's own query, within
  2e-3 of max(|score|, rms of all scores);
* the top-k rows and their order exactly against the oracle's selection on
  the GPU's float32 scores (equal scores: lower row first), and the output
  scores bitwise against the score array;
* the oracle's whole pipeline from the raw query: rows selected by one side
  only must score within the tolerance of the k-th best.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import indexer
from compressed_kv_attention_compressor_amd import binding as B
from compressed_kv_attention_compressor_amd import synth
from compressed_kv_attention_compressor_amd.layer import CompressorLayer
from tests.compare import REL_TOL, check_index_rows, check_prequant

pytestmark = pytest.mark.gpu


def run_gpu(q, w, rows, k):
    H, Dh = q.shape
    n = rows.shape[0]
    dev = "cuda"
    qd = torch.from_numpy(np.ascontiguousarray(q)).to(dev)
    wd = torch.from_numpy(np.ascontiguousarray(w)).to(dev)
    rd = torch.from_numpy(np.ascontiguousarray(rows)).to(dev) if n else torch.empty(0, device=dev)
    m = min(n, k)
    idx = torch.full((max(m, 1),), -7, dtype=torch.int32, device=dev)
    sc = torch.full((max(m, 1),), float("nan"), dtype=torch.float32, device=dev)
    q_hat = torch.full((H, Dh), float("nan"), dtype=torch.float32, device=dev)
    scores = torch.full((max(n, 1),), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(B.ds4c_indexer_workspace_bytes(n, k), dtype=torch.uint8, device=dev)
    B.ds4c_indexer_topk(qd.data_ptr(), wd.data_ptr(), H, Dh, rd.data_ptr() if n else 0, n, k, idx.data_ptr(),
                        sc.data_ptr(), q_hat.data_ptr(), scores.data_ptr(), ws.data_ptr(), ws.numel(),
                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return (idx[:m].cpu().numpy(), sc[:m].cpu().numpy(), q_hat.cpu().numpy(), scores[:n].cpu().numpy())


def check(q, w, rows, k, what):
    n = rows.shape[0]
    g_idx, g_sc, g_qhat, g_scores = run_gpu(q, w, rows, k)
    if n == 0:  # nothing is launched
        assert g_idx.size == 0 and np.isnan(g_qhat).all()
        return
    o_qhat = indexer.qat_query(q)
    check_index_rows(g_qhat, o_qhat, None, q.astype(np.float64), f"{what} q_hat")
    o_scores = indexer.scores(g_qhat, w, rows)
    check_prequant(g_scores, o_scores, f"{what} scores")
    want = indexer.topk(g_scores, k)
    assert np.array_equal(g_idx.astype(np.int64), want), what
    assert np.array_equal(g_sc.view(np.uint32), g_scores[g_idx].view(np.uint32)), what
    # the oracle's own pipeline from the raw query
    _, s_full, o_top = indexer.select(q, w, rows, k)
    if len(o_top) < n:
        scale = max(float(np.sqrt(np.mean(s_full ** 2))), 1e-30)
        kth = float(s_full[o_top[-1]])
        for j in set(g_idx.tolist()) ^ set(o_top.tolist()):
            assert abs(float(s_full[j]) - kth) <= REL_TOL * max(abs(kth), scale), (what, j)
    else:
        assert sorted(g_idx.tolist()) == list(range(n))


CASES = {
    # name: (rows, k, heads, head_dim)
    "c5_end_state": (16448, 512, 64, 128),
    "max_rows": (131072, 512, 64, 128),
    "one_row": (1, 512, 64, 128),
    "tiny": (5, 3, 4, 64),
    "k_equals_rows": (512, 512, 64, 128),
    "k_plus_one": (513, 512, 8, 128),
    "two_chunks_odd_k": (4097, 37, 16, 64),
    "many_chunks_small_k": (100000, 64, 32, 128),
    "two_chunks_k1": (40000, 1, 64, 128),
    "one_full_chunk": (32768, 512, 64, 128),
    "no_rows": (0, 16, 64, 128),
}


@pytest.mark.parametrize("name", list(CASES))
def test_indexer_matches_oracle(name):
    n, k, H, Dh = CASES[name]
    print(f"[indexer] {name}: rows {n} k {k} heads {H} dims {Dh}", flush=True)
    q, w, rows = synth.indexer_inputs(40 + list(CASES).index(name), n, H, Dh)
    check(q, w, rows, k, name)


def test_indexer_ties_go_to_the_lower_row():
    print("[indexer] ties", flush=True)
    q, w, rows = synth.indexer_inputs(50, 3000, 64, 128)
    rows[1000:1500] = rows[0:500]          # identical rows: bitwise-equal scores
    rows[2000:2100] = rows[1200:1300]
    check(q, w, rows, 512, "ties")
    g_idx, _, _, g_scores = run_gpu(q, w, rows, 512)
    for j in range(500):
        assert g_scores[j] == g_scores[1000 + j]


def test_indexer_crowded_top_byte():
    """Rows that are one row scaled by factors within 0.1 %: a score scales
    with its row (the ReLU commutes with a positive factor), so all 40000
    scores share one top byte: the first radix digit leaves every key of both
    chunks (32768 and 7232 rows) in the k-th key's bucket, and the later
    digits, which the score order rests on, do all the narrowing."""
    print("[indexer] crowded top byte", flush=True)
    q, w, rows = synth.indexer_inputs(53, 40000, 64, 128)
    scale = 1.0 + 1e-3 * np.random.default_rng(53).random(40000, dtype=np.float64)
    rows = (rows[:1].astype(np.float64) * scale[:, None]).astype(np.float32)
    check(q, w, rows, 512, "crowded top byte")
    _, _, _, g_scores = run_gpu(q, w, rows, 512)
    tops = np.unique(g_scores.view(np.uint32) >> 24)
    assert len(tops) == 1, tops


def test_indexer_over_compressor_rows():
    """The indexer rows a Flash ratio-4 layer writes for a 4096-token chunk (1024 rows)."""
    print("[indexer] over the r4_flash layer's indexer rows", flush=True)
    w_ = synth.WORKLOADS["r4_flash"]
    shape = w_.layer
    p = synth.layer_params(w_.wid, 0, shape)
    x = synth.hidden_states(w_.wid, shape.hidden, 0, w_.tokens, shape.dtype)
    layer = CompressorLayer(shape.ratio, shape.hidden, p, dtype=shape.dtype, max_tokens=w_.tokens)
    layer.prefill(torch.from_numpy(x).to("cuda", torch.bfloat16))
    torch.cuda.synchronize()
    rows = layer.live_rows("index").cpu().numpy()
    assert rows.shape == (1024, 128)
    q, w, _ = synth.indexer_inputs(51, 0, 64, 128)
    check(q, w, rows, 512, "compressor rows")


def test_indexer_is_deterministic():
    """Survivors are gathered with LDS atomics in an order that depends on
    the waves' timing, then sorted (keys are unique): the output is the same
    on every run."""
    print("[indexer] determinism", flush=True)
    q, w, rows = synth.indexer_inputs(52, 100000, 64, 128)
    a = run_gpu(q, w, rows, 512)
    b = run_gpu(q, w, rows, 512)
    for x_, y_ in zip(a, b):
        assert np.array_equal(x_.view(np.uint32) if x_.dtype == np.float32 else x_,
                              y_.view(np.uint32) if y_.dtype == np.float32 else y_)
