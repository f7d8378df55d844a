"""GPU: the decode GEMV's form for APE tables that lie far apart in memory.

The GEMV reads the indexer lane's APE row as an offset from the attention
lane's when the two are within 2^31 floats of each other, and from its
argument struct otherwise.  This test places a 10 GiB buffer between the two
tables so that the second form runs, and checks that a layer built that way
emits exactly the rows and frontier of a twin whose tables are adjacent.
"""

import numpy as np
import pytest
import torch

from compressed_kv_attention_compressor_amd import binding as B
from compressed_kv_attention_compressor_amd import synth
from compressed_kv_attention_compressor_amd.layer import CompressorLayer

pytestmark = pytest.mark.gpu


def _layer(shape, params, n):
    return CompressorLayer(shape.ratio, shape.hidden, params, dtype=shape.dtype, n_rot=shape.n_rot,
                           rope_base=shape.rope_base, rms_eps=shape.rms_eps, max_tokens=n)


def _run(layer, x, n_prefill, n_decode):
    layer.prefill(x[:n_prefill])
    pre = []
    for t in range(n_prefill, n_prefill + n_decode):
        pre.append(layer.decode_one(x[t], prequant=True))
    torch.cuda.synchronize()
    return pre


def test_far_apart_ape_tables_decode_like_adjacent_ones():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    w = synth.WORKLOADS["r4_small"]
    s = w.layer
    p = synth.layer_params(w.wid, 0, s)
    n_prefill, n_decode = 61, 11  # window boundaries at positions 63, 67 and 71
    x = torch.from_numpy(synth.hidden_states(w.wid, s.hidden, 0, n_prefill + n_decode, s.dtype)).to("cuda")
    near = _layer(s, p, n_prefill + n_decode)
    far = _layer(s, p, n_prefill + n_decode)
    # One 20 GiB buffer: one of its two ends lies at least 10 GiB (2.7e9 floats) from the
    # attention table, and the indexer table is copied there.
    ape_np = np.ascontiguousarray(p["index"]["ape"], dtype=np.float32)
    nbytes = (ape_np.nbytes + 255) // 256 * 256
    spacer = torch.empty((20 << 30) + nbytes, dtype=torch.uint8, device="cuda")
    attn = far.layer.attn.ape
    ends = [0, 20 << 30]
    off = max(ends, key=lambda o: abs(spacer.data_ptr() + o - attn))
    ape_far = spacer[off:off + ape_np.nbytes].view(torch.float32)
    ape_far.copy_(torch.from_numpy(ape_np).view(-1))
    gap = abs(ape_far.data_ptr() - attn) // 4
    assert gap > 2**31 - 1, gap
    print(f"index APE table {gap} floats from the attention table", flush=True)
    lane = far.layer.index
    far.layer.index = B.Lane(lane.head_dim, lane.wkv, lane.wgate, ape_far.data_ptr(), lane.norm_w)
    far._keep.append(spacer)

    got_near = _run(near, x, n_prefill, n_decode)
    got_far = _run(far, x, n_prefill, n_decode)
    for kind in near.kinds:
        assert torch.equal(near.live_rows(kind), far.live_rows(kind)), kind
        for a, b in zip(got_near, got_far):
            assert torch.equal(a[kind], b[kind]), kind
    assert (near.n_tokens, near.frontier.n_comp) == (far.n_tokens, far.frontier.n_comp) == (72, 18)
    assert torch.equal(near.state[256:], far.state[256:])
