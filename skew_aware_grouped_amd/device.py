"""Move a synthetic workload (numpy, from ``workloads``) into device tensors and
run the layer on it.  Marshalling only."""
from __future__ import annotations

import numpy as np

from . import moe
from .workloads import MODE_BF16, MODE_F32ACT, MODE_FP8, MODE_INT8, MODE_MXFP8, MoEWorkload


def upload(w: MoEWorkload, device="cuda:0", packed: bool = False) -> dict:
    """Device copies of the workload's tensors; with ``packed`` the weights are
    rewritten once into the packed tile order (moe_pack_weights)."""
    import torch

    def t(a, dt=None):
        r = torch.from_numpy(np.ascontiguousarray(a)).to(device)
        return r if dt is None else r.view(dt)

    d = {"mode": w.mode}
    if w.mode == MODE_F32ACT:
        d["x"] = t(w.x)
    elif w.mode == MODE_BF16:
        d["x"] = t(w.x.view(np.int16), torch.bfloat16)
    elif w.mode == MODE_INT8:
        d["x"] = t(w.x.astype(np.int8))
    else:
        d["x"] = t(w.x, torch.float8_e4m3fn)
    if w.mode in (MODE_FP8, MODE_MXFP8):  # fp32 block scales or uint8 E8M0 scales
        d["w1"] = t(w.w1, torch.float8_e4m3fn)
        d["w2"] = t(w.w2, torch.float8_e4m3fn)
        d["x_scale"] = t(w.x_scale)
        d["w1_scale"] = t(w.w1_scale)
        d["w2_scale"] = t(w.w2_scale)
    else:
        d["w1"] = t(w.w1.view(np.int16), torch.bfloat16)
        d["w2"] = t(w.w2.view(np.int16), torch.bfloat16)
        d["x_scale"] = d["w1_scale"] = d["w2_scale"] = None
        if w.mode == MODE_INT8:  # one fp32 scale per token
            d["x_scale"] = t(w.x_scale.astype(np.float32))
    d["topk_ids"] = t(w.topk_ids.astype(np.int32))
    d["topk_w"] = t(w.topk_w.astype(np.float32))
    d["weight_layout"] = moe.MOE_WEIGHTS_ROW_MAJOR
    d["activation"] = int(w.activation)
    if packed:
        d["w1"], d["w2"] = moe.pack_weights(d["w1"], d["w2"])
        d["weight_layout"] = moe.MOE_WEIGHTS_PACKED
    return d


def run(d: dict, out=None, workspace=None, stream=None, events=None, launch=moe.MOE_LAUNCH_MULTI):
    return moe.fused_forward(d["x"], d["topk_ids"], d["topk_w"], d["w1"], d["w2"], out=out, x_scale=d["x_scale"],
                             w1_scale=d["w1_scale"], w2_scale=d["w2_scale"], workspace=workspace, stream=stream,
                             events=events, weight_layout=d.get("weight_layout", moe.MOE_WEIGHTS_ROW_MAJOR),
                             activation=d.get("activation", moe.MOE_ACT_SWIGLU), launch=launch)


def out_to_f64(out) -> np.ndarray:
    import torch
    return out.float().cpu().numpy().astype(np.float64)
