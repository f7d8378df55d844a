"""White-box check of the projection GEMM through the C ABI.

After a prefill call that does not start on a window boundary (the plain
path; one token is prefilled first) the first T*N floats of the workspace
hold the projection [T, N] = x . [wkv_attn; wgate_attn; wkv_index;
wgate_index]^T (scores without APE).  It is compared with the float64 product on the host
against the floating-point error bound of a float32 accumulation:
|g - o| <= 5e-5 * sum_k |x_k w_k|  (about 200x the typical rounding error and
far below what a wrong index, operand or tile would produce).
"""

import numpy as np
import pytest
import torch

from compressed_kv_attention_compressor_amd import synth
from compressed_kv_attention_compressor_amd.layer import CompressorLayer

pytestmark = pytest.mark.gpu

CASES = {
    # name: (shape, tokens) -- chosen so that each tile shape is selected
    "bf16_256x160": (synth.FLASH_R4, 4096),
    "bf16_256x160_ragged_m": (synth.FLASH_R4, 4000),
    "bf16_128x128": (synth.FLASH_R128, 4096),
    "bf16_128x128_ragged": (synth.FLASH_R128, 4000),
    "bf16_64x64": (synth.LayerShape(ratio=4, hidden=256, d_attn=128, d_index=64, dtype="bf16"), 700),
    "f32_64x64": (synth.LayerShape(ratio=4, hidden=256, d_attn=128, d_index=64, dtype="f32"), 1000),
    "bf16_128x128_small_k": (synth.LayerShape(ratio=4, hidden=256, d_attn=512, d_index=128, dtype="bf16"), 700),
    "f32_128x128": (synth.LayerShape(ratio=128, hidden=192, d_attn=512, d_index=0, dtype="f32"), 4000),
    "f32_256x160": (synth.LayerShape(ratio=4, hidden=128, d_attn=512, d_index=128, dtype="f32"), 4000),
    # short calls: K split over 16 / 8 / 4 / 2 ranges, planes added in order
    "bf16_128x128_split8": (synth.FLASH_R4, 64),
    "bf16_128x128_split4": (synth.FLASH_R4, 200),
    "bf16_64x64_split16": (synth.FLASH_R128, 5),
    "bf16_64x64_split2": (synth.FLASH_R128, 300),
    "f32_64x64_split2": (synth.LayerShape(ratio=4, hidden=256, d_attn=128, d_index=64, dtype="f32"), 300),
    "f32_64x64_split8": (synth.LayerShape(ratio=128, hidden=4096, d_attn=128, d_index=0, dtype="f32"), 100),
}


@pytest.mark.parametrize("name", list(CASES))
def test_projection_matches_float64(name):
    shape, T = CASES[name]
    print(f"[projection] {name} T={T}", flush=True)
    wid = 70 + list(CASES).index(name)
    p = synth.layer_params(wid, 0, shape)
    x_all = synth.hidden_states(wid, shape.hidden, 0, T + 1, shape.dtype)
    layer = CompressorLayer(shape.ratio, shape.hidden, p, dtype=shape.dtype, max_tokens=T + 1)
    tdt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    xg = torch.from_numpy(x_all).to("cuda", tdt)
    layer.prefill(xg[:1])
    layer.prefill(xg[1:])
    torch.cuda.synchronize()
    x = x_all[1:]
    kinds = ["attn"] + (["index"] if shape.ratio == 4 else [])
    w = np.concatenate([np.concatenate([p[k]["wkv"], p[k]["wgate"]]) for k in kinds]).astype(np.float64)
    N = w.shape[0]
    got = layer._ws[: T * N * 4].view(torch.float32).view(T, N).cpu().numpy().astype(np.float64)
    x64 = x.astype(np.float64)
    want = x64 @ w.T
    bound = np.abs(x64) @ np.abs(w).T
    err = np.abs(got - want) / bound
    assert float(err.max()) < 5e-5, (name, float(err.max()), np.unravel_index(np.argmax(err), err.shape))
