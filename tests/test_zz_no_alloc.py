"""moe_fused_forward_noalloc (the entry point for callers that cannot
allocate: its workspace is the library's fixed device scratch) against
moe_fused_forward with a workspace of its own, through the C ABI, bit for bit:
two calls in a row on one stream, the second with a smaller input, in every
data mode.  Named to be collected last."""
import ctypes

import numpy as np
import pytest
import torch

from skew_aware_grouped_amd import device, moe, workloads as W

pytestmark = pytest.mark.gpu


def _args(d, out, mode):
    dims = moe.make_dims(d["x"], d["topk_ids"], d["w1"], x_scale=d["x_scale"])
    scales = None
    if mode in (W.MODE_FP8, W.MODE_MXFP8):
        scales = moe.moe_scales(d["x_scale"].data_ptr(), d["w1_scale"].data_ptr(), d["w2_scale"].data_ptr())
    elif mode == W.MODE_INT8:
        scales = moe.moe_scales(d["x_scale"].data_ptr(), None, None)
    return dims, (d["x"].data_ptr(), d["topk_ids"].data_ptr(), d["topk_w"].data_ptr(), d["w1"].data_ptr(),
                  d["w2"].data_ptr(), scales, out.data_ptr())


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@pytest.mark.parametrize("mode", [W.MODE_F32ACT, W.MODE_BF16, W.MODE_FP8, W.MODE_MXFP8, W.MODE_INT8])
def test_noalloc_matches_workspace_entry_point(mode):
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    odt = torch.float32 if mode == W.MODE_F32ACT else torch.bfloat16
    # the second call is smaller: the scratch still holds the first call's
    # (larger) routing tables, task lists and rows
    for shape, seed in (((700, 16, 2, 512, 256), 61), ((90, 8, 3, 256, 256), 62)):
        T, E, k, d_h, d_e = shape
        d = device.upload(W.custom(T, E, k, d_h, d_e, mode, seed=seed, routing=("zipf", 1.2, 2)))
        ref = torch.full((T, d_h), float("nan"), dtype=odt, device="cuda:0")
        got = torch.full((T, d_h), float("nan"), dtype=odt, device="cuda:0")
        dims, a = _args(d, ref, mode)
        need = moe.moe_workspace_bytes(dims)
        assert 0 < need <= moe.MOE_NOALLOC_SCRATCH_BYTES
        ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
        rc = moe.moe_fused_forward(dims, *a, ws.data_ptr(), need, sp)
        assert rc == moe.MOE_OK, moe.moe_error_string(rc)
        dims, a = _args(d, got, mode)
        rc = moe.moe_fused_forward_noalloc(dims, *a, sp)
        assert rc == moe.MOE_OK, moe.moe_error_string(rc)
        torch.cuda.synchronize()
        assert torch.isfinite(ref.float()).all()
        assert torch.equal(_bits(ref), _bits(got)), f"shape {shape}"


def test_noalloc_rejects_dims_beyond_scratch():
    d = moe.moe_dims(mode=moe.MOE_MODE_FP8, num_tokens=8192, num_experts=32, top_k=2, d_hidden=7168,
                     d_expert=2048)
    assert moe.moe_workspace_bytes(d) > moe.MOE_NOALLOC_SCRATCH_BYTES
    p = 1 << 20
    rc = moe.moe_fused_forward_noalloc(d, p, p, p, p, p, moe.moe_scales(p, p, p), p, None)
    assert rc == moe.MOE_ERR_SCRATCH
