"""CPU checks of the C-ABI library: it loads, exports every declared entry
point, and its host-side logic (sizes, layout, argument checks) behaves as the
header states.  No call here touches a GPU."""
import ctypes

import pytest

from skew_aware_grouped_amd import moe


def test_library_exports_every_header_symbol():
    L = moe.lib()
    names = moe.header_symbols()
    assert set(names) >= {"moe_fused_forward", "moe_route", "moe_workspace_bytes", "moe_block_m",
                          "moe_route_caps", "moe_workspace_layout", "moe_error_string"}
    for n in names:
        assert hasattr(L, n), n


def test_block_m_and_caps():
    assert moe.moe_block_m() == 16
    assert moe.moe_route_caps(1024, 2, 32) == (2048 + 32 * 15, (2048 + 32 * 15) // 16)
    assert moe.moe_route_caps(1, 2, 32) == (2 + 2 * 15, 2)


def _dims(mode=moe.MOE_MODE_FP8, T=1024, E=32, k=2, d_h=7168, d_e=2048, layout=moe.MOE_WEIGHTS_ROW_MAJOR,
          act=moe.MOE_ACT_SWIGLU, launch=moe.MOE_LAUNCH_MULTI):
    return moe.moe_dims(mode=mode, num_tokens=T, num_experts=E, top_k=k, d_hidden=d_h, d_expert=d_e,
                        weight_layout=layout, activation=act, launch=launch)


def test_workspace_layout_is_disjoint_and_aligned():
    for mode in (0, 1, 2, 3, 4):
        d = _dims(mode=mode)
        L = moe.moe_workspace_layout(d)
        offs = [L.sync, L.counts, L.offsets, L.padded_offsets, L.pos, L.sorted_p, L.ppos, L.row_src, L.row_w,
                L.tile_expert, L.tile_row0, L.stats, L.tasks1, L.tasks2, L.h, L.h_scale, L.y, L.zero, L.x_bf16,
                L.total]
        assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
        N = 2048
        assert L.pos - L.ppos <= 0 and L.sorted_p - L.pos >= 4 * N
        assert L.y + (4 if mode == 0 else 2) * N * 7168 <= L.total
        assert moe.moe_workspace_bytes(d) == L.total


def test_gemm_task_shapes_follow_batch_and_launch():
    """Column blocks and the largest task in the layout: FP8 batches of at
    least 2048 assignments (MXFP8: 4096) take the 8-wave GEMM-1 (16-block
    M-tiles), of at least 1024 the 8-wave GEMM-2 (256-column tasks, when d_h
    is a multiple of 256, the layer runs as four launches and, in MXFP8,
    d_e >= 1024); everything else 8-block tasks and 128-column GEMM-2
    blocks."""
    big = dict(mode=moe.MOE_MODE_FP8, T=8192, E=32, k=2, d_h=7168, d_e=2048)
    L = moe.moe_workspace_layout(_dims(**big))
    assert (L.block_n1, L.block_n2, L.max_row_blocks) == (128, 256, 16)
    L = moe.moe_workspace_layout(_dims(**dict(big, d_h=7296)))  # 57 * 128: GEMM-2 keeps 128 columns
    assert (L.block_n1, L.block_n2, L.max_row_blocks) == (128, 128, 16)
    L = moe.moe_workspace_layout(_dims(**dict(big, T=1024)))  # 2048 assignments: both 8-wave
    assert (L.block_n1, L.block_n2, L.max_row_blocks) == (128, 256, 16)
    L = moe.moe_workspace_layout(_dims(**dict(big, T=600)))  # 1200: the 8-wave GEMM-2 only
    assert (L.block_n1, L.block_n2, L.max_row_blocks) == (128, 256, 16)
    L = moe.moe_workspace_layout(_dims(**dict(big, T=511)))  # 1022: both 4-wave
    assert (L.block_n1, L.block_n2, L.max_row_blocks) == (128, 128, 8)
    L = moe.moe_workspace_layout(_dims(**dict(big, mode=moe.MOE_MODE_MXFP8)))
    assert (L.block_n1, L.block_n2, L.max_row_blocks) == (128, 256, 16)
    L = moe.moe_workspace_layout(_dims(**dict(big, T=511, mode=moe.MOE_MODE_MXFP8)))
    assert (L.block_n1, L.block_n2, L.max_row_blocks) == (128, 128, 8)
    mx = dict(big, mode=moe.MOE_MODE_MXFP8)
    assert moe.moe_workspace_layout(_dims(**dict(mx, T=1024))).block_n2 == 256  # 2048: GEMM-2 only
    assert moe.moe_workspace_layout(_dims(**dict(mx, T=1024, d_h=2048, d_e=768))).block_n2 == 128  # short K
    L = moe.moe_workspace_layout(_dims(**dict(big, mode=moe.MOE_MODE_BF16)))  # 64-column bf16 GEMM-1 tasks
    assert (L.block_n1, L.block_n2, L.max_row_blocks) == (64, 128, 8)
    L = moe.moe_workspace_layout(_dims(**dict(big, T=1024, launch=moe.MOE_LAUNCH_SINGLE)))
    assert L.block_n2 == 128


def test_invalid_dims_rejected():
    assert moe.moe_workspace_bytes(_dims(d_h=100)) == 0
    assert moe.moe_workspace_bytes(_dims(E=0)) == 0
    assert moe.moe_workspace_bytes(_dims(k=9)) == 0
    assert moe.moe_workspace_bytes(_dims(mode=5)) == 0
    assert moe.moe_workspace_bytes(_dims(mode=-1)) == 0
    assert moe.moe_workspace_bytes(_dims(layout=2)) == 0
    assert moe.moe_workspace_bytes(_dims(layout=moe.MOE_WEIGHTS_PACKED)) == moe.moe_workspace_bytes(_dims())
    assert moe.moe_workspace_bytes(_dims(act=2)) == 0
    assert moe.moe_workspace_bytes(_dims(act=moe.MOE_ACT_SWIGLU_CLAMPED)) == moe.moe_workspace_bytes(_dims())


def test_forward_argument_errors_without_gpu():
    p = 1 << 20  # fake, 256-aligned, never dereferenced: checks run before any launch
    big = 1 << 40
    args = dict(x=p, topk_ids=p, topk_w=p, w1=p, w2=p, out=p, workspace=p)
    sc = moe.moe_scales(p, p, p)

    def call(dims, scales=sc, ws_bytes=big, **over):
        a = {**args, **over}
        return moe.moe_fused_forward(dims, a["x"], a["topk_ids"], a["topk_w"], a["w1"], a["w2"], scales, a["out"],
                                     a["workspace"], ws_bytes, None)

    assert call(None) == moe.MOE_ERR_INVALID_ARG
    assert call(_dims(mode=5)) == moe.MOE_ERR_INVALID_ARG
    assert call(_dims(layout=7)) == moe.MOE_ERR_INVALID_ARG
    assert call(_dims(act=-1)) == moe.MOE_ERR_INVALID_ARG
    assert call(_dims(d_h=100)) == moe.MOE_ERR_UNSUPPORTED
    assert call(_dims(E=300)) == moe.MOE_ERR_UNSUPPORTED
    assert call(_dims(T=0)) == moe.MOE_OK  # empty batch: nothing to do
    assert call(_dims(), x=None) == moe.MOE_ERR_INVALID_ARG
    assert call(_dims(), x=p + 4) == moe.MOE_ERR_INVALID_ARG  # misaligned
    assert call(_dims(), scales=None) == moe.MOE_ERR_INVALID_ARG  # FP8 needs scales
    mx = _dims(mode=moe.MOE_MODE_MXFP8)
    assert call(mx, scales=None) == moe.MOE_ERR_INVALID_ARG  # so does MXFP8
    assert call(mx, scales=moe.moe_scales(p, p + 2, p)) == moe.MOE_ERR_INVALID_ARG  # E8M0 rows: 4-byte aligned
    assert call(mx, scales=moe.moe_scales(p, p, 0)) == moe.MOE_ERR_INVALID_ARG
    assert call(_dims(), ws_bytes=16) == moe.MOE_ERR_WORKSPACE
    assert call(_dims(), workspace=None) == moe.MOE_ERR_WORKSPACE
    assert call(_dims(), workspace=p + 64) == moe.MOE_ERR_WORKSPACE  # workspace must be 256-aligned
    for c in range(5):
        assert moe.moe_error_string(c) != "unknown error"


def test_route_argument_errors_without_gpu():
    out = moe.moe_route_out()
    assert moe.moe_route(4, 2, 0, 1 << 20, out, None) == moe.MOE_ERR_INVALID_ARG
    assert moe.moe_route(4, 9, 4, 1 << 20, out, None) == moe.MOE_ERR_INVALID_ARG
    assert moe.moe_route(4, 2, 4, 1 << 20, out, None) == moe.MOE_ERR_INVALID_ARG  # null outputs


def test_pack_weights_argument_errors_without_gpu():
    E, d_h, d_e = 4, 256, 128
    n1 = E * 2 * d_e * d_h * 2  # bf16 bytes of W1
    n2 = E * d_h * d_e * 2
    w1, w2 = 1 << 30, (1 << 30) + n1  # fake, aligned, disjoint; never dereferenced
    p1, p2 = (1 << 31), (1 << 31) + n1
    dims = _dims(mode=moe.MOE_MODE_BF16, T=0, E=E, d_h=d_h, d_e=d_e)

    def call(d=dims, a=w1, b=w2, c=p1, e=p2):
        return moe.moe_pack_weights(d, a, b, c, e, None)

    assert call(d=None) == moe.MOE_ERR_INVALID_ARG
    assert call(d=_dims(mode=moe.MOE_MODE_BF16, E=E, d_h=100, d_e=d_e)) == moe.MOE_ERR_INVALID_ARG
    for bad in (dict(a=None), dict(b=None), dict(c=None), dict(e=None), dict(c=p1 + 8), dict(a=w1 + 4)):
        assert call(**bad) == moe.MOE_ERR_INVALID_ARG, bad
    assert call(c=w1 + 256) == moe.MOE_ERR_INVALID_ARG  # w1_packed overlaps w1
    assert call(e=w1) == moe.MOE_ERR_INVALID_ARG  # w2_packed overlaps w1
    assert call(e=p1 + n1 - 16) == moe.MOE_ERR_INVALID_ARG  # the packed buffers overlap


def test_noalloc_rejects_oversize_before_any_device_call():
    """The no-allocation entry point refuses dims whose workspace exceeds its
    fixed scratch, on the host, before looking up the scratch's address."""
    d = _dims(T=8192)  # 8192 tokens of the 7168/2048 top-2 FP8 layer
    assert moe.moe_workspace_bytes(d) > moe.MOE_NOALLOC_SCRATCH_BYTES
    p = 1 << 20
    rc = moe.moe_fused_forward_noalloc(d, p, p, p, p, p, moe.moe_scales(p, p, p), p, None)
    assert rc == moe.MOE_ERR_SCRATCH
    assert "scratch" in moe.moe_error_string(rc)
    assert moe.moe_fused_forward_noalloc(None, p, p, p, p, p, None, p, None) == moe.MOE_ERR_INVALID_ARG


def test_single_launch_layout_and_envelope():
    """The synchronisation block sits first, at the same place and size for all
    dims; the single launch keeps y in fp32; outside its envelope (F32ACT and
    INT8 modes, more than 2048 assignments, T * d_h / 128 above 65536) the call
    is rejected before any pointer or device is touched."""
    for mode in (1, 2, 3):
        for T, d_h in ((64, 256), (1024, 7168)):
            m = moe.moe_workspace_layout(_dims(mode=mode, T=T, d_h=d_h))
            s = moe.moe_workspace_layout(_dims(mode=mode, T=T, d_h=d_h, launch=moe.MOE_LAUNCH_SINGLE))
            assert m.sync == s.sync == 0 and m.counts == s.counts == moe.MOE_SYNC_BYTES
            assert s.x_bf16 - s.zero == m.x_bf16 - m.zero
            N = T * 2
            assert m.zero - m.y >= 2 * N * d_h and s.zero - s.y >= 4 * N * d_h
    null = (None,) * 6 + (None, None, None, 0, None)
    for mode, T, d_h in ((0, 64, 256), (4, 64, 256), (1, 1025, 256), (2, 1024, 8320)):
        d = _dims(mode=mode, T=T, d_h=d_h, launch=moe.MOE_LAUNCH_SINGLE)
        assert moe.moe_fused_forward(d, *null[1:]) == moe.MOE_ERR_UNSUPPORTED, (mode, T, d_h)
    d = _dims(launch=2)
    assert moe.moe_workspace_bytes(d) == 0
    assert moe.moe_fused_forward(d, *null[1:]) == moe.MOE_ERR_INVALID_ARG
    assert moe.moe_workspace_init(None, moe.MOE_SYNC_BYTES, None) == moe.MOE_ERR_WORKSPACE
    assert moe.moe_workspace_init(256, moe.MOE_SYNC_BYTES - 4, None) == moe.MOE_ERR_WORKSPACE
    assert moe.moe_workspace_init(256 + 16, moe.MOE_SYNC_BYTES, None) == moe.MOE_ERR_WORKSPACE
