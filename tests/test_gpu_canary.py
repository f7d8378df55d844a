"""Output-buffer discipline on the GPU: canary guards and poisoned outputs.

Every buffer the library writes (compressed rows, pre-codec rows, frontier
state, workspace, attention output) is placed inside a larger allocation
whose guard regions, before and after, hold a canary pattern; the outputs
themselves start poisoned with the same pattern (a NaN bit pattern).  After
each call:
* every guard region still holds the canary (nothing written out of range);
* every row the call emits holds no canary (fully overwritten), and rows past
  the new row count still hold it (nothing written beyond the count).
The calls cover the plain and fused prefill paths of both ratios, decode
steps with and without a window boundary, and mixed attention.
"""

import numpy as np
import pytest
import torch

from compressed_kv_attention_compressor_amd import binding as B
from compressed_kv_attention_compressor_amd import synth
from compressed_kv_attention_compressor_amd.layer import CompressorLayer

pytestmark = pytest.mark.gpu

CANARY = 0x7FA5A5A5            # a NaN bit pattern
G_ROWS, G_BYTES = 8, 4096      # guard sizes: rows for row buffers, bytes for byte buffers


def guarded_rows(n, d):
    big = torch.full(((2 * G_ROWS + n) * d,), CANARY, dtype=torch.int32, device="cuda")
    return big, big.view(torch.float32)[G_ROWS * d:(G_ROWS + n) * d].view(n, d)


def _pattern_bytes(n):
    return np.tile(np.frombuffer(np.array([CANARY], dtype=np.int32).tobytes(), dtype=np.uint8), n // 4)


def guarded_bytes(n):
    total = 2 * G_BYTES + (n + 3) // 4 * 4
    big = torch.from_numpy(_pattern_bytes(total).copy()).to("cuda")
    return big, big[G_BYTES:G_BYTES + n]


def guards_intact_bytes(big, n):
    v = big.cpu().numpy()
    pat = _pattern_bytes(v.size)
    return np.array_equal(v[:G_BYTES], pat[:G_BYTES]) and np.array_equal(v[G_BYTES + n:], pat[G_BYTES + n:])


def guards_intact_rows(big, n, d):
    v = big.cpu().numpy()
    return (v[:G_ROWS * d] == CANARY).all() and (v[(G_ROWS + n) * d:] == CANARY).all()


def is_canary(t):
    return t.contiguous().view(torch.int32) == CANARY


class Guarded:
    """A layer whose rows, frontier state and workspace live inside guarded
    allocations (the layer object only supplies the descriptor)."""

    def __init__(self, shape, wid, max_tokens):
        p = synth.layer_params(wid, 0, shape, random_norm=True)
        self.L = CompressorLayer(shape.ratio, shape.hidden, p, dtype=shape.dtype, max_tokens=max_tokens)
        self.shape = shape
        L = self.L
        self.cap = L.cap
        self.rows = {}
        for k in L.kinds:
            self.rows[k] = guarded_rows(self.cap, L.head_dim[k])
        n_state = B.ds4c_frontier_bytes(L.layer)
        self.state_big, self.state = guarded_bytes(n_state)
        L.frontier.state = self.state.data_ptr()
        self.n_state = n_state
        n_ws = B.ds4c_workspace_bytes(L.layer, max_tokens)
        self.ws_big, self.ws = guarded_bytes(n_ws)
        self.n_ws = n_ws
        B.ds4c_frontier_init(L.layer, L.frontier, 0)

    def rows_ptr(self, k):
        return self.rows[k][1].data_ptr() if k in self.rows else 0

    def prefill(self, x):
        L = self.L
        n0 = L.frontier.n_tokens
        n_emit = (n0 + x.shape[0]) // L.ratio - n0 // L.ratio
        pre = {k: guarded_rows(max(n_emit, 1), L.head_dim[k]) for k in L.kinds}
        B.ds4c_compress_prefill(L.layer, L.frontier, x.data_ptr(), x.shape[0],
                                self.rows_ptr("attn"), self.cap, self.rows_ptr("index"),
                                self.cap if "index" in self.rows else 0, self.ws.data_ptr(), self.n_ws,
                                pre["attn"][1].data_ptr(), pre["index"][1].data_ptr() if "index" in pre else 0, 0)
        torch.cuda.synchronize()
        return n_emit, pre

    def decode(self, x):
        L = self.L
        pos = L.frontier.n_tokens
        n_emit = 1 if (pos + 1) % L.ratio == 0 else 0
        pre = {k: guarded_rows(1, L.head_dim[k]) for k in L.kinds}
        B.ds4c_compress_decode_one(L.layer, L.frontier, x.data_ptr(), self.rows_ptr("attn"), self.cap,
                                   self.rows_ptr("index"), self.cap if "index" in self.rows else 0,
                                   pre["attn"][1].data_ptr(), pre["index"][1].data_ptr() if "index" in pre else 0, 0)
        torch.cuda.synchronize()
        return n_emit, pre

    def check(self, n_emit, pre):
        L = self.L
        for k in L.kinds:
            big, view = self.rows[k]
            d = L.head_dim[k]
            assert guards_intact_rows(big, self.cap, d), f"{k} rows guard"
            n = L.frontier.n_comp if k == "attn" else L.frontier.n_index_comp
            assert not is_canary(view[:n]).any(), f"{k} rows [0, {n}) not fully written"
            assert is_canary(view[n:]).all(), f"{k} rows past {n} written"
            pbig, pview = pre[k]
            assert guards_intact_rows(pbig, pview.shape[0], d), f"{k} pre-codec guard"
            assert not is_canary(pview[:n_emit]).any(), f"{k} pre-codec rows not fully written"
        assert guards_intact_bytes(self.state_big, self.n_state), "frontier state guard"
        assert guards_intact_bytes(self.ws_big, self.n_ws), "workspace guard"


@pytest.mark.parametrize("ratio", [4, 128])
def test_prefill_and_decode_stay_inside_their_buffers(ratio):
    shape = (synth.LayerShape(ratio=4, hidden=256, d_attn=128, d_index=64, dtype="bf16") if ratio == 4 else
             synth.LayerShape(ratio=128, hidden=256, d_attn=256, d_index=0, dtype="bf16"))
    x = synth.hidden_states(70 + ratio, 256, 0, 6000, "bf16")
    xd = torch.from_numpy(x).to("cuda", torch.bfloat16)
    g = Guarded(shape, 70 + ratio, max_tokens=6000)
    t = 0
    # One token (decode path), a call from inside a window (plain path),
    # calls that start on a window boundary long enough for the fused path,
    # then decode steps across a boundary.
    plan = [1, 599, 1448, 2048, -9] if ratio == 4 else [1, 383, 1664, 2560, -130]
    for step in plan:
        if step > 0:
            print(f"[canary] ratio {ratio}: prefill {step} tokens from {t}", flush=True)
            n_emit, pre = g.prefill(xd[t:t + step])
            g.check(n_emit, pre)
            t += step
        else:
            print(f"[canary] ratio {ratio}: {-step} decode steps from {t}", flush=True)
            for _ in range(-step):
                n_emit, pre = g.decode(xd[t].contiguous())
                g.check(n_emit, pre)
                t += 1
    assert g.L.frontier.n_tokens == t


def test_mixed_attention_output_stays_inside_its_buffer():
    print("[canary] mixed attention, 24 heads x 256 dims", flush=True)
    q, ring, comp, topk = synth.mixed_attention_inputs(71, 300, n_heads=24, head_dim=256, ring_cap=48, k=100)
    dev = "cuda"
    qd, rd, cd = (torch.from_numpy(a).to(dev) for a in (q, ring, comp))
    td = torch.from_numpy(topk).to(dev)
    big, out = guarded_rows(24, 256)
    n = B.ds4c_mixed_attention_workspace_bytes(24, 256, 48, 100)
    ws_big, ws = guarded_bytes(n)
    B.ds4c_mixed_attention(qd, rd, 1000, 1036, 64, cd, td, 1036, 4, out, ws)
    torch.cuda.synchronize()
    assert guards_intact_rows(big, 24, 256)
    assert guards_intact_bytes(ws_big, n)
    assert not is_canary(out).any()
