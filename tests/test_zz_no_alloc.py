"""The allocation-free indexer entry point against the workspace one.

ds4c_indexer_topk_noalloc runs ds4c_indexer_topk's kernels on the library's
fixed per-device scratch.  Three calls in a row, each smaller than the one
before (the largest call the indexer accepts at k = 512, then a two-chunk and
a one-chunk call): every output must equal the workspace entry point's on the
same inputs bit for bit -- selected rows and their order, their scores, the
rotated quantised query -- and the noalloc call's row scores (kept in the
scratch, not returned) must select the same rows as the returned scores of
the workspace call.  The scratch keeps the previous call's contents, so a
smaller call after a larger one would expose any read of stale scores or
candidate keys.
"""

import numpy as np
import pytest
import torch

from compressed_kv_attention_compressor_amd import binding as B
from compressed_kv_attention_compressor_amd import synth

pytestmark = pytest.mark.gpu

CALLS = [(1 << 20, 512), (40000, 512), (5000, 64)]


def _outputs(n, k, H, Dh, dev):
    m = min(n, k)
    return (torch.full((m,), -7, dtype=torch.int32, device=dev),
            torch.full((m,), float("nan"), dtype=torch.float32, device=dev),
            torch.full((H, Dh), float("nan"), dtype=torch.float32, device=dev))


def test_noalloc_indexer_matches_the_workspace_entry_point():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    dev = "cuda"
    stream = torch.cuda.current_stream().cuda_stream
    for i, (n, k) in enumerate(CALLS):
        print(f"[no-alloc] call {i}: {n} rows, k {k}", flush=True)
        q, w, rows = synth.indexer_inputs(200 + i, n, 64, 128)
        qd, wd, rd = (torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in (q, w, rows))
        # workspace entry point (reference), with the row scores returned
        idx_r, sc_r, qh_r = _outputs(n, k, 64, 128, dev)
        scores_r = torch.full((n,), float("nan"), dtype=torch.float32, device=dev)
        ws = torch.empty(B.ds4c_indexer_workspace_bytes(n, k), dtype=torch.uint8, device=dev)
        B.ds4c_indexer_topk(qd.data_ptr(), wd.data_ptr(), 64, 128, rd.data_ptr(), n, k, idx_r.data_ptr(),
                            sc_r.data_ptr(), qh_r.data_ptr(), scores_r.data_ptr(), ws.data_ptr(), ws.numel(), stream)
        # allocation-free entry point: scores stay in the library's scratch
        idx_g, sc_g, qh_g = _outputs(n, k, 64, 128, dev)
        B.ds4c_indexer_topk_noalloc(qd.data_ptr(), wd.data_ptr(), 64, 128, rd.data_ptr(), n, k, idx_g.data_ptr(),
                                    sc_g.data_ptr(), qh_g.data_ptr(), 0, stream)
        torch.cuda.synchronize()
        assert torch.equal(idx_g, idx_r), f"call {i}: selected rows differ"
        assert torch.equal(sc_g, sc_r), f"call {i}: selected scores differ"
        assert torch.equal(qh_g, qh_r), f"call {i}: rotated query differs"
        # the selection is the top k of the returned scores, ties to the lower row
        s = scores_r.cpu().numpy()
        want = np.lexsort((np.arange(n), -s.astype(np.float64)))[:min(n, k)]
        assert np.array_equal(idx_g.cpu().numpy().astype(np.int64), want), f"call {i}: not the top k"
        assert np.array_equal(sc_g.cpu().numpy(), s[want]), f"call {i}: scores not the selected rows'"
        del ws
