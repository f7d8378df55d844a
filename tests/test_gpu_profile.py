"""Kernel timing through the library's profiling calls, on the GPU.

Timing and the cold-pool eviction must not change what a call computes:
the same calls with timing off, timing on, and timing on with a scratch
buffer written between projection and pooling give bitwise-equal rows and
frontiers (the same kernels run on the same inputs), and the timed classes
record one interval per call.
"""

import pytest
import torch

from compressed_kv_attention_compressor_amd import binding as B
from compressed_kv_attention_compressor_amd import synth
from compressed_kv_attention_compressor_amd.layer import CompressorLayer

pytestmark = pytest.mark.gpu

WID = 61


@pytest.mark.parametrize("ratio", [4, 128])
def test_timing_and_eviction_leave_results_unchanged(ratio):
    print(f"[profile] ratio {ratio}: 1 + 599 tokens, timing off / on / on with read and write eviction", flush=True)
    shape = synth.LayerShape(ratio=ratio, hidden=256, d_attn=128, d_index=64 if ratio == 4 else 0, dtype="bf16")
    p = synth.layer_params(WID, 0, shape, random_norm=True)
    x = synth.hidden_states(WID, 256, 0, 600, "bf16")
    xd = torch.from_numpy(x).to("cuda", torch.bfloat16)
    L = CompressorLayer(ratio, 256, p, dtype="bf16", max_tokens=600)
    scratch = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    results, counts = [], []
    scratch.zero_()
    for mode in ("off", "on", "evict_read", "evict_write"):
        L.reset()
        L.prefill(xd[:1])
        if mode != "off":
            B.ds4c_profile_enable([B.KCLASS_PROJ, B.KCLASS_POOL, B.KCLASS_CARRY])
        if mode.startswith("evict"):
            B.ds4c_profile_evict(scratch.data_ptr(), scratch.numel(), write=mode == "evict_write")
        try:
            L.prefill(xd[1:600])
            torch.cuda.synchronize()
            if mode != "off":
                counts.append(B.ds4c_profile_read()[1])
        finally:
            B.ds4c_profile_evict(0, 0)
            B.ds4c_profile_enable(False)
        results.append({k: L.live_rows(k).clone() for k in L.kinds})
        results[-1]["state"] = L.state.clone()
    for r in results[1:]:
        for k, v in r.items():
            assert torch.equal(v, results[0][k]), k
    for c in counts:
        assert c[B.KCLASS_PROJ] >= 1 and c[B.KCLASS_POOL] == 1
        assert c[B.KCLASS_CARRY] == (1 if ratio == 4 else 0)
    # The write eviction wrote the scratch buffer (word i holds i).
    assert int(scratch[16:20].view(torch.int32)[0]) == 1
