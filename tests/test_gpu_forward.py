"""GPU parity of the whole layer (moe_fused_forward through the C ABI) against
the CPU oracle.

Tolerance: norm-wise max relative error max|g - r| / max|r|, 1e-2 in the bf16
modes and 3e-2 in the FP8 and MXFP8 modes, asserted twice: over all compared
rows together and for every compared token row on its own (a row whose
reference is exactly zero, every assignment dropped, must be exactly zero).
At full workload sizes the oracle computes a sample of token rows that meets
every GEMM M-tile: one token from each 64-row slice of every expert's group
(the GEMM-1 and GEMM-2 tasks take 64- or 128-row M-tiles), each expert's last
row and the first row of its last 16-row group block; the full output is then
checked for properties that hold at any size (every row written, finite,
bitwise identical across launches)."""
import numpy as np
import pytest

from skew_aware_grouped_amd import device, moe, workloads as W

pytestmark = pytest.mark.gpu

TOL = {W.MODE_F32ACT: 1e-2, W.MODE_BF16: 1e-2, W.MODE_FP8: 3e-2, W.MODE_MXFP8: 3e-2, W.MODE_INT8: 1e-2}
FP8_MODES = (W.MODE_FP8, W.MODE_MXFP8)


def normwise(got, ref):
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def rowwise(got, ref):
    """Largest per-row norm-wise error max_c|g - r| / max_c|r| over the rows;
    rows whose reference is exactly zero must match exactly."""
    den = np.abs(ref).max(axis=1)
    num = np.abs(got - ref).max(axis=1)
    zero = den == 0
    assert np.all(num[zero] == 0), "a token with no valid assignment has a nonzero output row"
    return float((num[~zero] / den[~zero]).max()) if (~zero).any() else 0.0


SLICE = 64  # rows per sampled slice of an expert's group: the smaller GEMM M-tile


def _sample_rows(w, n=12, seed=0):
    """Token rows to check at full size: a random set, the first and last token,
    and for every active expert one token from each SLICE-row slice of its
    group (its rows in the stable order, ascending flat index p), its last row
    and the first row of its last 16-row group block.  So every M-tile of both
    GEMMs' task lists meets the oracle, including each expert's partial one."""
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(w.T, size=min(n, w.T), replace=False).tolist()) | {0, w.T - 1}
    flat = w.topk_ids.ravel()
    valid = (flat >= 0) & (flat < w.E)
    order = np.argsort(np.where(valid, flat, w.E), kind="stable")  # p grouped by expert, ascending p
    cnt = np.bincount(flat[valid], minlength=w.E)
    start = 0
    for e in range(w.E):
        c = int(cnt[e])
        if c == 0:
            continue
        ps = order[start:start + c]
        start += c
        picks = {int(rng.integers(m0, min(c, m0 + SLICE))) for m0 in range(0, c, SLICE)}
        picks |= {c - 1, (c - 1) // 16 * 16}
        rows |= {int(ps[i]) // w.k for i in picks}
    return sorted(rows)


def _run(w, out=None):
    import torch
    d = device.upload(w)
    o = device.run(d, out=out)
    torch.cuda.synchronize()
    return d, o


def _check(w, oracle, rows=None, label="", packed=False):
    import torch
    d = device.upload(w, packed=packed)
    odt = torch.float32 if w.mode == W.MODE_F32ACT else torch.bfloat16
    out = torch.full((w.T, w.d_h), float("nan"), dtype=odt, device="cuda:0")  # sentinel: every row must be written
    dims = moe.make_dims(d["x"], d["topk_ids"], d["w1"], x_scale=d["x_scale"])
    ws = moe.workspace_for(dims, "cuda:0")
    device.run(d, out=out, workspace=ws)
    torch.cuda.synchronize()
    g = device.out_to_f64(out)
    assert np.isfinite(g).all(), "unwritten or non-finite output rows"
    acc, _ = oracle.forward(w, rows=rows)
    gs = g if rows is None else g[rows]
    err = normwise(gs, acc)
    rerr = rowwise(gs, acc)
    print(f"{label} mode={w.mode} act={w.activation} packed={packed} T={w.T} E={w.E} k={w.k} {w.d_h}x{w.d_e}: "
          f"{len(gs)} rows, normwise err {err:.3e}, worst row {rerr:.3e}", flush=True)
    assert err <= TOL[w.mode], err
    assert rerr <= TOL[w.mode], rerr
    return d, out, g


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("mode", [W.MODE_F32ACT, W.MODE_BF16, W.MODE_FP8, W.MODE_MXFP8, W.MODE_INT8])
def test_small_shapes_full_parity(oracle, mode, packed):
    """Several tiles in every direction with ragged expert groups."""
    w = W.custom(200, 8, 3, 384, 256, mode, seed=21)
    _check(w, oracle, label="small", packed=packed)


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("mode", [W.MODE_F32ACT, W.MODE_BF16, W.MODE_FP8, W.MODE_MXFP8, W.MODE_INT8])
def test_small_shapes_d_expert_384(oracle, mode, packed):
    """d_e = 384: three FP8 / six bf16 GEMM-1 column blocks, ragged expert
    groups up to several M-tiles."""
    w = W.custom(300, 6, 2, 256, 384, mode, seed=23)
    _check(w, oracle, label="d_e=384", packed=packed)


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("mode", [W.MODE_F32ACT, W.MODE_BF16, W.MODE_FP8, W.MODE_MXFP8, W.MODE_INT8])
def test_clamped_activation_small_shapes(oracle, mode, packed):
    """The clamped activation on widened inputs (x scaled by 4: about a tenth
    of the gate and up values lie beyond the clamp), ragged expert groups."""
    w = W.custom(200, 8, 3, 384, 256, mode, seed=22, activation=W.ACT_SWIGLU_CLAMPED, x_gain=4.0)
    _check(w, oracle, label="clamped", packed=packed)


@pytest.mark.parametrize("mode", FP8_MODES)
def test_clamped_activation_wide_kernels(oracle, mode):
    """The clamped activation (x scaled by 4) at 4200 assignments, where both
    FP8 modes run the 8-wave GEMM-1 and GEMM-2; every row compared."""
    w = W.custom(2100, 6, 2, 512, 1024, mode, seed=47, routing=("zipf", 1.1, 1),
                 activation=W.ACT_SWIGLU_CLAMPED, x_gain=4.0)
    _check(w, oracle, label="clamped_wide", packed=True)


@pytest.mark.parametrize("name", ["qwen_bf16", "ds_fp8_1024", "ds_mxfp8_1024"])
def test_clamped_activation_sampled(oracle, name):
    import dataclasses
    w = dataclasses.replace(W.config(name), activation=W.ACT_SWIGLU_CLAMPED)
    _check(w, oracle, rows=_sample_rows(w), label=name + "_clamped", packed=True)


@pytest.mark.parametrize("name", ["tiny", "qwen_bf16"])
def test_workload_full_parity(oracle, name):
    w = W.config(name)
    _check(w, oracle, label=name)


@pytest.mark.parametrize("name", ["qwen_fp8", "ds_fp8_128", "ds_fp8_256", "ds_fp8_512", "ds_fp8_1024", "ds_fp8_8192",
                                  "qwen_mxfp8", "ds_mxfp8_1024", "ds_mxfp8_8192", "qwen_int8", "ds_int8_1024"])
def test_workload_sampled_parity(oracle, name):
    """Full-size workloads on packed weights (the layout bench.py times; the
    row-major layout is bitwise equal, tested below)."""
    print(f"generating {name}", flush=True)
    w = W.config(name)
    _check(w, oracle, rows=_sample_rows(w), label=name, packed=True)


@pytest.mark.parametrize("mode", [W.MODE_F32ACT, W.MODE_BF16, W.MODE_FP8, W.MODE_MXFP8, W.MODE_INT8])
def test_large_batch_routing_path(oracle, mode):
    """T*k = 18000 assignments, above the 16384 the routing kernel keeps in
    LDS: the ids are read twice and row_src is scattered straight to memory,
    and the GEMMs run on that permutation.  Skewed routing with empty
    experts; every output row is compared.  d_e = 1024: in the FP8 modes one
    code of the intermediate that the MFMA's sum puts on the other side of an
    e4m3 rounding boundary than the oracle's fp32 sum moves a whole row by up
    to about 2% at d_e = 256 (measured: 0.16% of the codes differ, each by one
    step), which the per-row bound would see at k = 4; the effect shrinks as
    1/sqrt(d_e)."""
    w = W.custom(4500, 64, 4, 256, 1024, mode, seed=41, routing=("zipf", 1.1, 6))
    _check(w, oracle, label="large_batch")


@pytest.mark.parametrize("mode", FP8_MODES)
def test_fp8_wide_gemm1_with_narrow_gemm2(oracle, mode):
    """8400 assignments take the 8-wave FP8 (MXFP8) GEMM-1; d_h = 384 is not
    a multiple of 256, so GEMM-2 keeps the 4-wave kernel and 128-column tasks
    (its grid then comes from that kernel's occupancy).  Every row compared.
    MXFP8 at d_e = 1024: at d_e = 256 its worst row is 3.1% off, the same
    bit for bit from the 4-wave kernels (rounding flips of the intermediate,
    as in test_large_batch_routing_path)."""
    w = W.custom(4200, 16, 2, 384, 256 if mode == W.MODE_FP8 else 1024, mode, seed=45, routing=("zipf", 1.1, 2))
    _check(w, oracle, label="wide1_narrow2")


def test_more_m_tiles_than_rank_table(oracle):
    """About 1.08 million assignments over 64 experts: more than 8192 GEMM
    M-tiles per task list, so the task builder finds each task's expert by
    binary search instead of its rank table.  Sampled rows cover every
    M-tile."""
    rng = np.random.default_rng(77)
    T, E, k = 270000, 64, 4
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    w = W.custom(T, E, k, 128, 128, W.MODE_BF16, seed=43, topk_ids=ids)
    _check(w, oracle, rows=_sample_rows(w, n=64), label="m_tiles_8k")


@pytest.mark.parametrize("mode", [W.MODE_BF16, W.MODE_FP8, W.MODE_MXFP8, W.MODE_INT8])
def test_determinism_two_launches_and_streams(mode):
    import torch
    w = W.custom(300, 16, 2, 512, 256, mode, seed=5, routing=("zipf", 1.2, 3))
    d = device.upload(w)
    a = device.run(d).clone()
    b = device.run(d).clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())  # inputs were uploaded on the current stream
    with torch.cuda.stream(s):  # the binding gives this stream its own workspace
        c = device.run(d, stream=s).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_workspace_cache_is_per_stream():
    """The binding's cached workspace is never shared between two streams."""
    import torch
    w = W.custom(16, 4, 2, 256, 128, W.MODE_BF16, seed=2)
    d = device.upload(w)
    dims = moe.make_dims(d["x"], d["topk_ids"], d["w1"])
    s = torch.cuda.Stream()
    a = moe.workspace_for(dims, "cuda:0")
    b = moe.workspace_for(dims, "cuda:0", s)
    assert a.data_ptr() != b.data_ptr()
    assert moe.workspace_for(dims, "cuda:0").data_ptr() == a.data_ptr()


EDGE_CASES = {
    "one_token": dict(T=1, E=4, k=2),
    "single_expert": dict(T=100, E=1, k=1),
    "k8_duplicates": dict(T=40, E=3, k=8),
    "e256": dict(T=300, E=256, k=4),
    "all_on_one_expert": dict(T=333, E=16, k=2, ids="one"),
    "dropped_ids": dict(T=64, E=8, k=2, ids="dropped"),
}


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("case", sorted(EDGE_CASES))
@pytest.mark.parametrize("mode", [W.MODE_BF16, W.MODE_FP8, W.MODE_MXFP8, W.MODE_INT8])
def test_edge_cases(oracle, case, mode, packed):
    c = EDGE_CASES[case]
    rng = np.random.default_rng(9)
    T, E, k = c["T"], c["E"], c["k"]
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)  # duplicates allowed
    if c.get("ids") == "one":
        ids[:] = E // 2
    if c.get("ids") == "dropped":
        ids[::3, 0] = -1
        ids[1::5, 1] = E + 3
        ids[7, :] = -2  # a token with no valid assignment -> zero row
    # FP8 modes at d_e = 512: with every slot of a token on one expert, a
    # flipped code of the intermediate repeats in both slots, and at d_e = 256
    # the per-row bound sits at the edge of that flip noise (3.1e-2 measured)
    w = W.custom(T, E, k, 256, 512 if mode in FP8_MODES else 128, mode, seed=13, topk_ids=ids)
    _check(w, oracle, label=case, packed=packed)


def _packed_reference(wt, gated, bn):
    """The packed tile order as the header defines it, by numpy indexing: chunk
    ((tile * R + b) * rows + r) * 8 + s holds chunk s ^ (r & 7) of K block b of
    tile row r (gated tiles: gate rows c*bn.., then up rows d_e + c*bn..)."""
    E, nrows, kbytes = wt.shape
    n_out = nrows // 2 if gated else nrows
    R = kbytes // 128
    w5 = wt.reshape(E, nrows, R, 8, 16)
    c = np.arange(n_out // bn)[:, None, None, None]
    b = np.arange(R)[None, :, None, None]
    r = np.arange(2 * bn if gated else bn)[None, None, :, None]
    s = np.arange(8)[None, None, None, :]
    row = np.where(r < bn, c * bn + r, n_out + c * bn + r - bn) if gated else c * bn + r
    return w5[:, row, b, s ^ (r & 7)].reshape(-1)


@pytest.mark.parametrize("d_e", [256, 384])
@pytest.mark.parametrize("mode", [W.MODE_BF16, W.MODE_FP8, W.MODE_MXFP8])
def test_pack_weights_is_the_stated_permutation(mode, d_e):
    """moe_pack_weights output, byte for byte, against the header's formula."""
    import torch
    w = W.custom(8, 3, 2, 384, d_e, mode, seed=3)
    d = device.upload(w)
    p1, p2 = moe.pack_weights(d["w1"], d["w2"])
    torch.cuda.synchronize()
    L = moe.moe_workspace_layout(moe.make_dims(d["x"], d["topk_ids"], d["w1"], x_scale=d["x_scale"]))
    assert (L.block_n1, L.block_n2) == ((128, 128) if mode in FP8_MODES else (64, 128))

    def raw(t):
        return t.view(torch.uint8).cpu().numpy().reshape(t.shape[0], t.shape[1], -1)

    for src, got, gated, bn in ((d["w1"], p1, True, L.block_n1), (d["w2"], p2, False, L.block_n2)):
        want = _packed_reference(raw(src), gated, bn)
        assert np.array_equal(got.view(torch.uint8).cpu().numpy().reshape(-1), want)


@pytest.mark.parametrize("name", ["tiny", "qwen_bf16", "qwen_fp8", "ds_fp8_128", "ds_fp8_1024", "ds_fp8_8192",
                                  "qwen_mxfp8", "ds_mxfp8_1024", "qwen_int8"])
def test_packed_weights_bitwise_equal_row_major(name):
    """The packed layout changes where the GEMMs read each weight tile from,
    not what they compute: the output is bitwise the row-major one."""
    import torch
    print(f"generating {name}", flush=True)
    w = W.config(name)
    a = device.run(device.upload(w)).clone()
    b = device.run(device.upload(w, packed=True)).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16) if a.dtype != torch.float32 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype != torch.float32 else b.view(torch.int32))


@pytest.mark.parametrize("T,d_e", [(150, 256), (2100, 1024)])
@pytest.mark.parametrize("packed", [False, True])
def test_mxfp8_scales_vary_across_k(oracle, packed, T, d_e):
    """MXFP8 with scale bytes that differ by up to 2^7 between neighbouring
    32-value blocks of K, for x, W1 and W2 alike (still valid MX inputs): the
    output is right only if every 32-value slice of K meets its own scale in
    both operands.  Shifts are kept small enough that no product under- or
    overflows fp32.  300 assignments run the 4-wave GEMMs, 4200 the 8-wave
    ones (whose stages carry the scale words of 256 weight rows)."""
    import dataclasses
    w = W.custom(T, 6, 2, 512, d_e, W.MODE_MXFP8, seed=31, routing=("zipf", 1.1, 2))
    rng = np.random.default_rng(4)

    def shifted(sc, lo, hi):
        d = rng.integers(lo, hi + 1, size=sc.shape[-1])  # one shift per K block
        d = d + rng.integers(-1, 2, size=sc.shape[:-1])[..., None]  # and a small one per row
        return np.clip(sc.astype(np.int32) + d, 1, 254).astype(np.uint8)

    w = dataclasses.replace(w, x_scale=shifted(w.x_scale, -4, 3), w1_scale=shifted(w.w1_scale, -3, 4),
                            w2_scale=shifted(w.w2_scale, -4, 3))
    _check(w, oracle, label="mx_scale_shifts", packed=packed)


def test_empty_batch_is_noop():
    import torch
    w = W.custom(4, 4, 2, 256, 128, W.MODE_BF16, seed=1)
    d = device.upload(w)
    x0 = d["x"][:0]
    out = moe.fused_forward(x0, d["topk_ids"][:0], d["topk_w"][:0], d["w1"], d["w2"])
    torch.cuda.synchronize()
    assert out.shape == (0, 256)


@pytest.mark.parametrize("name", ["qwen_fp8", "ds_fp8_1024", "qwen_bf16", "ds_mxfp8_1024", "qwen_mxfp8", "qwen_int8",
                                  "ds_fp8_8192"])
def test_forward_routing_and_task_list(oracle, name):
    """The workspace after a forward call holds the oracle's counts, padded
    permutation (row_src) and routing weight per padded row, and task lists that
    cover every (group block, column block) pair exactly once."""
    import torch
    w = W.config(name)
    d = device.upload(w)
    dims = moe.make_dims(d["x"], d["topk_ids"], d["w1"], x_scale=d["x_scale"])
    ws = moe.workspace_for(dims, "cuda:0")
    device.run(d, workspace=ws)
    torch.cuda.synchronize()
    L = moe.moe_workspace_layout(dims)
    raw = ws.cpu().numpy()

    def arr(off, n, dt=np.int32):
        return raw[off:off + n * np.dtype(dt).itemsize].view(dt)

    r = oracle.route(w.topk_ids.ravel(), w.E, moe.moe_block_m())
    N = w.T * w.k
    assert np.array_equal(arr(L.counts, w.E), r["counts"])
    assert np.array_equal(arr(L.offsets, w.E + 1), r["offsets"])
    assert np.array_equal(arr(L.padded_offsets, w.E + 1), r["padded_offsets"])
    # the layer writes the padded permutation its GEMMs consume; the compact
    # pos / ppos / sorted_p arrays are moe_route's (tested in test_gpu_route)
    assert np.array_equal(arr(L.row_src, L.n_pad_cap), r["row_src"])
    # routing weight by padded row: a copy of topk_w, exact; 0 on padding rows
    n_pad = int(r["padded_offsets"][-1])
    src = r["row_src"][:n_pad]
    want_w = np.where(src >= 0, w.topk_w.ravel().astype(np.float32)[np.maximum(src, 0)], np.float32(0))
    assert np.array_equal(arr(L.row_w, n_pad, np.float32), want_w)
    ctl = arr(L.stats, 304)
    for lst, off, nb, segw in ((3, L.tasks1, w.d_e // L.block_n1, 272), (4, L.tasks2, w.d_h // L.block_n2, 288)):
        nt = int(ctl[lst])
        seg = ctl[segw:segw + 9]
        assert seg[0] == 0 and seg[8] == nt and np.all(np.diff(seg) >= 0)
        tasks = arr(off, 4 * nt).reshape(nt, 4)
        seen = {}
        for e, row0, nsub, cb in tasks.tolist():
            assert 1 <= nsub <= L.max_row_blocks and 0 <= cb < nb
            for b in range(nsub):
                r0 = row0 + 16 * b
                assert r["padded_offsets"][e] <= r0 < r["padded_offsets"][e + 1]
                seen[(r0, cb)] = seen.get((r0, cb), 0) + 1
        assert len(seen) == r["ntiles"] * nb and set(seen.values()) == {1}
        for x in range(8):
            part = tasks[seg[x]:seg[x + 1]].tolist()
            # longest expert first within each XCD's segment
            counts = [r["counts"][t[0]] for t in part]
            assert counts == sorted(counts, reverse=True)
            # every (expert, column block) group lives in one segment, contiguously
            groups = [(t[0], t[3]) for t in part]
            assert len(set(groups)) == len(list(dict.fromkeys(groups)))
            for g in set(groups):
                idx = [i for i, q in enumerate(groups) if q == g]
                assert idx == list(range(idx[0], idx[0] + len(idx)))
        owner = {}
        for x in range(8):
            for t in tasks[seg[x]:seg[x + 1]].tolist():
                assert owner.setdefault((t[0], t[3]), x) == x
