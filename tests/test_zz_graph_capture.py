"""The layer call launches without host computation or allocation once its
workspace exists, so a HIP graph can capture it (the property the PipeLink page,
section 4 "Contract-Guided Linking", states for host providers behind a C
interface).  A captured call is replayed on new inputs written into the same
buffers; every replay must equal, bit for bit, an eager call on those inputs
with its own output and workspace.  Eager work and synchronisations run between
the replays.  Named to run last: a capture failure cannot disturb other tests."""
import numpy as np
import pytest
import torch

from skew_aware_grouped_amd import device, moe, workloads as W

pytestmark = pytest.mark.gpu

KEYS = ("x", "topk_ids", "topk_w", "w1", "w2", "x_scale", "w1_scale", "w2_scale")


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


CASES = [(m, moe.MOE_LAUNCH_MULTI) for m in (W.MODE_BF16, W.MODE_FP8, W.MODE_MXFP8, W.MODE_INT8)] + \
        [(m, moe.MOE_LAUNCH_SINGLE) for m in (W.MODE_BF16, W.MODE_FP8, W.MODE_MXFP8)]


@pytest.mark.parametrize("mode,launch", CASES)
def test_graph_replays_match_eager(mode, launch):
    """Both launch forms; the single launch's workspace starts zeroed (its
    synchronisation block), and every replay must leave that block zero again."""
    shape = (200, 8, 2, 256, 256)
    d = device.upload(W.custom(*shape, mode, seed=31))
    dims = moe.make_dims(d["x"], d["topk_ids"], d["w1"], x_scale=d["x_scale"], launch=launch)
    ws_graph = torch.zeros(moe.moe_workspace_bytes(dims), dtype=torch.uint8, device="cuda:0")
    out_graph = torch.empty((shape[0], shape[3]), dtype=torch.bfloat16, device="cuda:0")
    device.run(d, out=out_graph, workspace=ws_graph, launch=launch)  # eager warm-up on the graph's buffers
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        device.run(d, out=out_graph, workspace=ws_graph, launch=launch)
    torch.cuda.synchronize()

    ws_eager = torch.zeros_like(ws_graph)
    for i, seed in enumerate((32, 33, 34, 33)):
        # new routing, weights and activations (the last replay repeats an earlier input)
        new = device.upload(W.custom(*shape, mode, seed=seed))
        for k in KEYS:
            if d[k] is not None:
                d[k].copy_(new[k])
        out_graph.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        eager = device.run(d, workspace=ws_eager, launch=launch)
        torch.cuda.synchronize()
        print(f"graph replay {i} (seed {seed}) mode={mode} launch={launch}", flush=True)
        assert torch.isfinite(out_graph.float()).all()
        assert torch.equal(_bits(out_graph), _bits(eager)), f"replay {i} differs from the eager call"
        if launch == moe.MOE_LAUNCH_SINGLE:
            assert not ws_graph[:moe.MOE_SYNC_BYTES].any(), "synchronisation block not zero after a replay"
