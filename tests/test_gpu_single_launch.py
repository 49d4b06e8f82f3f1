"""GPU parity of the single-launch layer (moe_dims.launch = MOE_LAUNCH_SINGLE:
routing, GEMM-1, GEMM-2 and the combine in one persistent kernel) against the
CPU oracle, through the C ABI.

Same tolerances and row checks as the four-launch tests (test_gpu_forward):
norm-wise max relative error 1e-2 (bf16) / 3e-2 (FP8, MXFP8) over the compared
rows and for every row on its own.  After every call the workspace's
synchronisation block must be all zeros again: the queue, exit, M-tile and
arrival counters reset by the kernel, and no bounded wait ran out."""
import numpy as np
import pytest
import torch

from skew_aware_grouped_amd import device, moe, workloads as W
from tests.test_gpu_forward import EDGE_CASES, FP8_MODES, TOL, _sample_rows, normwise, rowwise

pytestmark = pytest.mark.gpu

MODES = [W.MODE_BF16, W.MODE_FP8, W.MODE_MXFP8]
SINGLE = moe.MOE_LAUNCH_SINGLE


def _sync_words(ws):
    return ws[:moe.MOE_SYNC_BYTES].view(torch.int32).cpu().numpy()


def _run(d, out=None, workspace=None, launch=SINGLE):
    return device.run(d, out=out, workspace=workspace, launch=launch)


def _check(w, oracle, rows=None, label="", packed=False):
    d = device.upload(w, packed=packed)
    out = torch.full((w.T, w.d_h), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    dims = moe.make_dims(d["x"], d["topk_ids"], d["w1"], x_scale=d["x_scale"], launch=SINGLE)
    ws = moe.workspace_for(dims, "cuda:0")
    print(f"single launch {label}: mode={w.mode} T={w.T} E={w.E} k={w.k} {w.d_h}x{w.d_e} packed={packed}",
          flush=True)
    _run(d, out=out, workspace=ws)
    torch.cuda.synchronize()
    words = _sync_words(ws)
    assert words[moe.SYNC_TIMEOUTS_WORD] == 0, "a bounded wait ran out"
    assert not words.any(), f"synchronisation block not back to zero at words {np.nonzero(words)[0][:8]}"
    g = device.out_to_f64(out)
    assert np.isfinite(g).all(), "unwritten or non-finite output rows"
    acc, _ = oracle.forward(w, rows=rows)
    gs = g if rows is None else g[rows]
    err, rerr = normwise(gs, acc), rowwise(gs, acc)
    print(f"  {len(gs)} rows, normwise err {err:.3e}, worst row {rerr:.3e}", flush=True)
    assert err <= TOL[w.mode], err
    assert rerr <= TOL[w.mode], rerr
    return d, out, ws


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("mode", MODES)
def test_single_small_shapes(oracle, mode, packed):
    """Several tiles in every direction, ragged expert groups."""
    _check(W.custom(200, 8, 3, 384, 256, mode, seed=21), oracle, label="small", packed=packed)


@pytest.mark.parametrize("mode", MODES)
def test_single_d_expert_384(oracle, mode):
    _check(W.custom(300, 6, 2, 256, 384, mode, seed=23), oracle, label="d_e=384")


@pytest.mark.parametrize("mode", MODES)
def test_single_clamped_activation(oracle, mode):
    w = W.custom(200, 8, 3, 384, 256, mode, seed=22, activation=W.ACT_SWIGLU_CLAMPED, x_gain=4.0)
    _check(w, oracle, label="clamped")


@pytest.mark.parametrize("case", sorted(EDGE_CASES))
@pytest.mark.parametrize("mode", MODES)
def test_single_edge_cases(oracle, case, mode):
    """One expert, top-8 with repeated ids, 256 experts, every row on one expert
    (several M-tiles of one expert), dropped ids and a token with none valid."""
    c = EDGE_CASES[case]
    rng = np.random.default_rng(9)
    T, E, k = c["T"], c["E"], c["k"]
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    if c.get("ids") == "one":
        ids[:] = E // 2
    if c.get("ids") == "dropped":
        ids[::3, 0] = -1
        ids[1::5, 1] = E + 3
        ids[7, :] = -2
    w = W.custom(T, E, k, 256, 512 if mode in FP8_MODES else 128, mode, seed=13, topk_ids=ids)
    _check(w, oracle, label=case)


@pytest.mark.parametrize("name", ["qwen_bf16"])
def test_single_workload_full_parity(oracle, name):
    _check(W.config(name), oracle, label=name, packed=True)


@pytest.mark.parametrize("name", ["qwen_fp8", "ds_fp8_128", "ds_fp8_512", "ds_fp8_1024", "qwen_mxfp8",
                                  "ds_mxfp8_1024"])
def test_single_workload_sampled(oracle, name):
    w = W.config(name)
    _check(w, oracle, rows=_sample_rows(w), label=name, packed=True)


@pytest.mark.parametrize("mode", MODES)
def test_single_deterministic_and_reusable(mode):
    """Bitwise equal across calls; the same workspace then serves other dims
    (its counters were reset), and the single and four-launch outputs agree
    within the tolerance (the single launch keeps y in fp32)."""
    name = {W.MODE_BF16: "qwen_bf16", W.MODE_FP8: "qwen_fp8", W.MODE_MXFP8: "qwen_mxfp8"}[mode]
    d = device.upload(W.config(name), packed=True)
    a = _run(d).clone()
    b = _run(d).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    small = device.upload(W.custom(90, 5, 2, 256, 256, mode, seed=5))
    s1 = _run(small).clone()
    s4 = _run(small, launch=moe.MOE_LAUNCH_MULTI).clone()
    c = _run(d).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    assert normwise(s1.double().cpu().numpy(), s4.double().cpu().numpy()) <= TOL[mode]
    m = _run(d, launch=moe.MOE_LAUNCH_MULTI)
    torch.cuda.synchronize()
    assert normwise(a.double().cpu().numpy(), m.double().cpu().numpy()) <= TOL[mode]


@pytest.mark.parametrize("mode", MODES)
def test_single_noalloc_matches_workspace_call(mode):
    """The no-allocation entry point with MOE_LAUNCH_SINGLE: its fixed scratch
    starts zeroed, so the synchronisation block needs no initialisation."""
    d = device.upload(W.custom(150, 8, 2, 256, 256, mode, seed=44))
    ref = _run(d).clone()
    dims = moe.make_dims(d["x"], d["topk_ids"], d["w1"], x_scale=d["x_scale"], launch=SINGLE)
    out = torch.full_like(ref, float("nan"))
    scales = None if mode == W.MODE_BF16 else moe.moe_scales(d["x_scale"].data_ptr(), d["w1_scale"].data_ptr(),
                                                              d["w2_scale"].data_ptr())
    for _ in range(2):
        rc = moe.moe_fused_forward_noalloc(dims, d["x"].data_ptr(), d["topk_ids"].data_ptr(), d["topk_w"].data_ptr(),
                                           d["w1"].data_ptr(), d["w2"].data_ptr(), scales, out.data_ptr(),
                                           moe._stream_ptr())
        assert rc == moe.MOE_OK, moe.moe_error_string(rc)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_workspace_init_zeroes_the_sync_block():
    ws = torch.full((moe.MOE_SYNC_BYTES + 4096,), 7, dtype=torch.uint8, device="cuda:0")
    assert moe.moe_workspace_init(ws.data_ptr(), ws.numel(), moe._stream_ptr()) == moe.MOE_OK
    torch.cuda.synchronize()
    assert not ws[:moe.MOE_SYNC_BYTES].any()
    assert (ws[moe.MOE_SYNC_BYTES:] == 7).all()
