"""Ratio-4 indexed mixed attention (Part 3 §7) on the GPU against the oracle.

Tolerance: the kernels compute in float32.  A logit's unscaled dot product
of D = 512 N(0, 1) products has magnitude about sqrt(D) ~ 23; float32
accumulation adds a random-walk error of about sqrt(D) * 2^-24 * 23 ~ 3e-5,
which the 1/sqrt(D) scale brings to ~1.3e-6 per logit.  The weights use the
hardware base-2 exponential (relative error below 1e-6), so each weight is
good to a few 1e-6 relative, and the output, a convex combination of rows
with entries below 6 in magnitude, to ~5e-6 absolute: atol = 2e-5 with
rtol = 1e-5 leaves a factor 4 without hiding a wrong row (a missing or
extra row moves outputs by 1e-3 or more at these sizes, checked below by
planting one in the oracle's list).
"""

import numpy as np
import pytest
import torch

from compressed_kv_attention_compressor_amd import binding as B
from compressed_kv_attention_compressor_amd import synth
from oracle import mixed_attention as MA

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-5, 1e-5


def run_gpu(q, ring, first, last, window, comp, topk, qpos, ratio=4):
    dev = "cuda"
    qd = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float32)).to(dev)
    rd = torch.from_numpy(np.ascontiguousarray(ring, dtype=np.float32)).to(dev)
    cd = torch.from_numpy(np.ascontiguousarray(comp, dtype=np.float32).reshape(-1, q.shape[1])).to(dev)
    td = torch.from_numpy(np.asarray(topk, dtype=np.int32)).to(dev)
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device=dev)
    n = B.ds4c_mixed_attention_workspace_bytes(q.shape[0], q.shape[1], ring.shape[0], len(topk))
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
    B.ds4c_mixed_attention(qd, rd, first, last, window, cd, td, qpos, ratio, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check(q, ring, first, last, window, comp, topk, qpos, ratio=4):
    got = run_gpu(q, ring, first, last, window, comp, topk, qpos, ratio)
    ref = MA.mixed_attention(q, ring, first, last, window, comp, topk, qpos, ratio)
    np.testing.assert_allclose(got, ref, rtol=RTOL, atol=ATOL)
    return got, ref


def test_flash_decode_query_full_size():
    """64 heads x 512 dims, the last decode token of the long prompt (position
    65,791): 128 raw rows and the top 512 of 16,448 compressed rows."""
    print("[mixed] flash: H 64, D 512, ring 128, 16448 rows, k 512, qpos 65791", flush=True)
    q, ring, comp, topk = synth.mixed_attention_inputs(8, 16448)
    got, ref = check(q, ring, 65664, 65791, 128, comp, topk, 65791)
    err = np.abs(got - ref).max()
    print(f"[mixed] max abs error {err:.2e}", flush=True)
    # A planted mistake in the reference (one selected row dropped) is caught.
    bad = MA.mixed_attention(q, ring, 65664, 65791, 128, comp, topk[1:], 65791)
    assert np.abs(got - bad).max() > 10 * ATOL


@pytest.mark.parametrize("D", [64, 128, 256, 512])
@pytest.mark.parametrize("H", [8, 24])
def test_head_shapes_with_ragged_splits(D, H):
    """37 raw rows + 100 list entries: five splits of 32 items, the last
    ragged; the ring wraps (positions 1000..1036 in a ring of 48)."""
    print(f"[mixed] H {H} D {D}: 37 raw + 100 listed", flush=True)
    q, ring, comp, topk = synth.mixed_attention_inputs(60, 300, n_heads=H, head_dim=D, ring_cap=48, k=100, seed=D)
    check(q, ring, 1000, 1036, 64, comp, topk, 1036)


def test_walk_rules_on_the_device():
    print("[mixed] negative entries, early end, duplicates, window inside the ring", flush=True)
    q, ring, comp, topk = synth.mixed_attention_inputs(61, 50, n_heads=16, head_dim=128, ring_cap=64, k=40)
    lst = topk.copy()
    lst[3] = -1
    lst[7] = -5
    lst[10] = lst[11]             # a duplicate
    lst[25] = 50                  # first entry >= visible (50 rows visible at qpos 199): ends the walk
    lst[26] = 2                   # after the end: not attended
    check(q, ring, 150, 203, 20, comp, lst, 199)
    # Window 0 covers every held position; qpos inside the held range.
    check(q, ring, 150, 203, 0, comp, lst, 180)


def test_long_list_ends_past_the_first_scan_pass():
    """1200 entries: the end of the walk (entry 900) lies in the second scan
    pass of 512 entries; 10 raw + 1200 listed items make 38 splits, so the
    merge takes two passes of 32."""
    print("[mixed] k 1200, walk ends at entry 900", flush=True)
    q, ring, comp, topk = synth.mixed_attention_inputs(64, 1900, n_heads=8, head_dim=64, ring_cap=16, k=1200)
    lst = topk.copy()
    lst[900] = 1900
    check(q, ring, 7590, 7599, 16, comp, lst, 7599)


def test_empty_sets_give_zeros_and_single_sets():
    print("[mixed] empty and one-sided calls", flush=True)
    q, ring, comp, topk = synth.mixed_attention_inputs(62, 10, n_heads=8, head_dim=64, ring_cap=16, k=8)
    # Nothing held, nothing listed.
    got = run_gpu(q, ring, 5, 4, 16, comp[:0], np.zeros(0, np.int32), 2)
    assert not got.any()
    # Only negative entries and no raw rows.
    got = run_gpu(q, ring, 5, 4, 16, comp, np.full(8, -1, np.int32), 39)
    assert not got.any()
    # Raw rows only (k = 0), compressed rows only (no raw row held).
    check(q, ring, 30, 39, 16, comp, np.zeros(0, np.int32), 39)
    check(q, ring, 5, 4, 16, comp, topk, 39)
    # No compressed row visible yet (qpos 2): the list ends at its first entry.
    check(q, ring, 0, 2, 16, comp[:0], topk, 2)


def test_ratio_128_visibility():
    print("[mixed] ratio 128: rows visible at qpos 383", flush=True)
    q, ring, comp, topk = synth.mixed_attention_inputs(63, 3, n_heads=8, head_dim=512, ring_cap=128, k=3)
    check(q, ring, 256, 383, 128, comp, topk, 383, ratio=128)


def test_repeated_calls_are_bitwise_equal():
    q, ring, comp, topk = synth.mixed_attention_inputs(8, 16448)
    a = run_gpu(q, ring, 65664, 65791, 128, comp, topk, 65791)
    b = run_gpu(q, ring, 65664, 65791, 128, comp, topk, 65791)
    assert np.array_equal(a, b)


def test_chain_compressor_indexer_attention():
    """The three calls in sequence with every intermediate left on the device:
    a Flash ratio-4 layer compresses a 4096-token chunk (1024 rows per lane),
    the indexer selects 512 of its indexer rows for a query, and the
    query at position 4095 attends the 128 raw window rows plus the selected
    attention rows.  The selection is checked against the oracle's on the
    GPU's own scores, the attention against the oracle on the same rows."""
    from oracle import indexer

    print("[mixed] chain: r4_flash prefill -> indexer top-512 -> mixed attention", flush=True)
    w_ = synth.WORKLOADS["r4_flash"]
    shape = w_.layer
    p = synth.layer_params(w_.wid, 0, shape)
    x = synth.hidden_states(w_.wid, shape.hidden, 0, w_.tokens, shape.dtype)
    from compressed_kv_attention_compressor_amd.layer import CompressorLayer
    layer = CompressorLayer(shape.ratio, shape.hidden, p, dtype=shape.dtype, max_tokens=w_.tokens)
    layer.prefill(torch.from_numpy(x).to("cuda", torch.bfloat16))
    n = layer.frontier.n_index_comp
    assert n == 1024 and layer.frontier.n_comp == 1024
    dev = "cuda"
    # Indexer over the layer's indexer rows, straight from the row buffer.
    qi, wi, _ = synth.indexer_inputs(52, 0, 64, 128)
    qid, wid = torch.from_numpy(qi).to(dev), torch.from_numpy(wi).to(dev)
    k = 512
    idx = torch.empty(k, dtype=torch.int32, device=dev)
    isc = torch.empty(k, dtype=torch.float32, device=dev)
    scores = torch.empty(n, dtype=torch.float32, device=dev)
    iws = torch.empty(B.ds4c_indexer_workspace_bytes(n, k), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    B.ds4c_indexer_topk(qid.data_ptr(), wid.data_ptr(), 64, 128, layer.rows["index"].data_ptr(), n, k,
                        idx.data_ptr(), isc.data_ptr(), 0, scores.data_ptr(), iws.data_ptr(), iws.numel(), stream)
    # Mixed attention over the layer's attention rows with that selection.
    q, ring, _, _ = synth.mixed_attention_inputs(53, 1, n_heads=64, head_dim=512, ring_cap=128, k=1)
    qd, rd = torch.from_numpy(q).to(dev), torch.from_numpy(ring).to(dev)
    comp = layer.rows["attn"][:1024]
    out = torch.full((64, 512), float("nan"), dtype=torch.float32, device=dev)
    aws = torch.empty(B.ds4c_mixed_attention_workspace_bytes(64, 512, 128, k), dtype=torch.uint8, device=dev)
    B.ds4c_mixed_attention(qd, rd, 3968, 4095, 128, comp, idx, 4095, 4, out, aws, stream)
    torch.cuda.synchronize()
    g_idx, g_scores = idx.cpu().numpy(), scores.cpu().numpy()
    assert np.array_equal(g_idx.astype(np.int64), indexer.topk(g_scores, k))
    ref = MA.mixed_attention(q, ring, 3968, 4095, 128, comp.cpu().numpy(), g_idx, 4095, 4)
    np.testing.assert_allclose(out.cpu().numpy(), ref, rtol=RTOL, atol=ATOL)
