// C-ABI host side of the fused MoE library: argument checks, workspace
// layout, persistent-grid sizing and the launch sequence
// route -> GEMM-1 (+SwiGLU) -> GEMM-2 (+routing weight) -> combine.
#include <algorithm>
#include <mutex>

#include "moe_internal.h"

namespace {

using namespace moe;

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool dims_ok(const moe_dims* d) {
    if (!d) return false;
    if (d->mode < MOE_MODE_F32ACT || d->mode > MOE_MODE_INT8) return false;
    if (d->num_tokens < 0 || d->num_experts < 1 || d->num_experts > kMaxExperts) return false;
    if (d->top_k < 1 || d->top_k > 8) return false;
    if ((int64_t)d->num_tokens * d->top_k >= ((int64_t)1 << 31)) return false;
    if (d->d_hidden < 128 || d->d_hidden % 128 || d->d_expert < 128 || d->d_expert % 128) return false;
    if (d->weight_layout != MOE_WEIGHTS_ROW_MAJOR && d->weight_layout != MOE_WEIGHTS_PACKED) return false;
    if (d->activation != MOE_ACT_SWIGLU && d->activation != MOE_ACT_SWIGLU_CLAMPED) return false;
    if (d->launch != MOE_LAUNCH_MULTI && d->launch != MOE_LAUNCH_SINGLE) return false;
    return true;
}

static_assert(MOE_SYNC_BYTES == 4u * kSyncWords, "synchronisation block size");

// the single launch's envelope (dims already valid)
bool single_ok(const moe_dims* d) {
    const int64_t N = (int64_t)d->num_tokens * d->top_k;
    return (d->mode == MOE_MODE_BF16 || d->mode == MOE_MODE_FP8 || d->mode == MOE_MODE_MXFP8) && N <= kLayerMaxN &&
           (int64_t)d->num_tokens * (d->d_hidden / 128) <= kSyncArriveWords;
}

void route_caps(int64_t N, int64_t E, int64_t* n_pad_cap, int64_t* tile_cap) {
    *n_pad_cap = N + (E < N ? E : N) * (kBlockM - 1);
    *tile_cap = *n_pad_cap / kBlockM;
}

void layout_of(const moe_dims* d, moe_ws_layout* L) {
    const int64_t N = (int64_t)d->num_tokens * d->top_k;
    const int64_t E = d->num_experts;
    route_caps(N, E, &L->n_pad_cap, &L->tile_cap);
    // M-tiles: each expert's blocks grouped 8 at a time (GEMM-1; GEMM-2 outside
    // MXFP8 mode), or kSmallRowBlocks when 8-block tiles would leave too few
    // tasks: both lists are sized for the smaller tiles
    const int64_t mtile_cap1 = L->tile_cap / kSmallRowBlocks + (E < N ? E : N);
    const int64_t mtile_cap2 = mtile_cap1;
    L->block_n1 = gemm1_block_n(d->mode);
    const bool wide2 =
        fp8_wide2(d->mode, d->launch, d->num_tokens, d->top_k, d->num_experts, d->d_hidden, d->d_expert);
    L->block_n2 = gemm2_block_n(d->mode, wide2);
    // the largest task of either list, in group blocks
    L->max_row_blocks = std::max(gemm1_max_row_blocks(d->mode, d->num_tokens, d->top_k, d->d_hidden, d->d_expert),
                                 gemm2_row_blocks(d->mode, wide2));
    L->task1_cap = mtile_cap1 * (d->d_expert / L->block_n1);
    L->task2_cap = mtile_cap2 * (d->d_hidden / L->block_n2);
    const size_t hb = mode_fp8(d->mode) ? 1 : 2;
    const size_t yb = d->mode == MOE_MODE_F32ACT || d->launch == MOE_LAUNCH_SINGLE ? 4 : 2;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align_up(o + (bytes ? bytes : 1));
        return at;
    };
    // the synchronisation block of the single launch comes first, at the same
    // place and size for all dims
    L->sync = take(MOE_SYNC_BYTES);
    L->counts = take(4 * E);
    L->offsets = take(4 * (E + 1));
    L->padded_offsets = take(4 * (E + 1));
    L->pos = take(4 * N);
    L->sorted_p = take(4 * N);
    L->ppos = take(4 * N);
    L->row_src = take(4 * L->n_pad_cap);
    L->row_w = take(4 * L->n_pad_cap);
    L->tile_expert = take(4 * L->tile_cap);
    L->tile_row0 = take(4 * L->tile_cap);
    L->stats = take(4 * kCtlWords);
    L->tasks1 = take(16 * L->task1_cap);
    L->tasks2 = take(16 * L->task2_cap);
    L->h = take(hb * L->n_pad_cap * d->d_expert);
    // FP8: fp32 per row per 128 columns; MXFP8: one E8M0 byte per row per 32 columns
    L->h_scale = take(d->mode == MOE_MODE_FP8     ? 4 * L->n_pad_cap * (d->d_expert / kQ)
                      : d->mode == MOE_MODE_MXFP8 ? L->n_pad_cap * (d->d_expert / 32)
                                                  : 0);
    L->y = take(yb * N * d->d_hidden);
    L->zero = take(kZeroBytes);
    // F32ACT: x rounded to bf16 once; INT8: the codes widened to bf16 (exact);
    // the bf16 GEMMs then run on it
    L->x_bf16 = take(d->mode == MOE_MODE_F32ACT || d->mode == MOE_MODE_INT8 ? 2 * (size_t)d->num_tokens * d->d_hidden
                                                                            : 0);
    L->total = o;
}

// Per-device cache of the chip size and of the GEMM kernels' occupancy.
// Slots 4 and 5 hold the 8-wave FP8 and MXFP8 GEMM-1 and GEMM-2 (fp8_wide, fp8_wide2).
struct DeviceInfo {
    bool ready = false;
    int cus = 0;
    int occ1[6] = {0, 0, 0, 0, 0, 0};
    int occ2[6] = {0, 0, 0, 0, 0, 0};
    int occ_layer[4] = {0, 0, 0, 0};  // single-launch kernel, by mode (BF16, FP8, MXFP8)
};
std::mutex g_mu;
DeviceInfo g_dev[64];

// occ_layer (may be null): resident workgroups per CU of the single-launch kernel
hipError_t device_info(int mode, bool wide, bool wide2, int* cus, int* occ1, int* occ2, int* occ_layer = nullptr) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    DeviceInfo& di = g_dev[dev];
    if (!di.ready) {
        err = hipDeviceGetAttribute(&di.cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (err != hipSuccess) return err;
        for (int m = 0; m < 6; ++m) {
            err = gemm_occupancy(m < 4 ? m : m == 4 ? MOE_MODE_FP8 : MOE_MODE_MXFP8, m >= 4, &di.occ1[m], &di.occ2[m]);
            if (err != hipSuccess) return err;
            if (di.occ1[m] < 1) di.occ1[m] = 1;
            if (di.occ2[m] < 1) di.occ2[m] = 1;
        }
        for (int m = MOE_MODE_BF16; m <= MOE_MODE_MXFP8; ++m) {
            err = layer_occupancy(m, &di.occ_layer[m]);
            if (err != hipSuccess) return err;
            if (di.occ_layer[m] < 1) di.occ_layer[m] = 1;
        }
        di.ready = true;
    }
    *cus = di.cus;
    if (occ_layer) *occ_layer = di.occ_layer[mode_fp8(mode) ? mode : MOE_MODE_BF16];
    const int wide_slot = mode == MOE_MODE_MXFP8 ? 5 : 4;
    *occ1 = di.occ1[wide ? wide_slot : gemm_mode(mode)];
    *occ2 = di.occ2[wide2 ? wide_slot : gemm_mode(mode)];
    return hipSuccess;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Workspace of moe_fused_forward_noalloc, for callers that cannot allocate
// device memory.  A file-scope device array: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code `scratch` names a host-side stand-in, not device memory, so it is never
// passed to a kernel or copy: the device address comes from
// hipGetSymbolAddress, taken once per device (with that device current) and
// kept in g_scratch.
__device__ __attribute__((aligned(256))) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];
void* g_scratch[64] = {};

hipError_t scratch_of_current_device(void** p) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* q = nullptr;
        err = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
        if (err != hipSuccess) return err;
        if (!q || ((uintptr_t)q & (kAlign - 1))) return hipErrorInvalidSymbol;
        g_scratch[dev] = q;
    }
    *p = g_scratch[dev];
    return hipSuccess;
}

template <typename T>
T* at(void* base, size_t off) {
    return reinterpret_cast<T*>(static_cast<char*>(base) + off);
}

}  // namespace

extern "C" {

const char* moe_error_string(int code) {
    switch (code) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_HIP: return "HIP launch or query failed";
        case MOE_ERR_SCRATCH: return "workspace these dims need exceeds the fixed scratch of the no-allocation entry point";
        default: return "unknown error";
    }
}

int32_t moe_block_m(void) { return kBlockM; }

int moe_route_caps(int32_t num_tokens, int32_t top_k, int32_t num_experts, int64_t* n_pad_cap, int64_t* tile_cap) {
    if (!n_pad_cap || !tile_cap || num_tokens < 0 || top_k < 1 || num_experts < 1) return MOE_ERR_INVALID_ARG;
    route_caps((int64_t)num_tokens * top_k, num_experts, n_pad_cap, tile_cap);
    return MOE_OK;
}

int moe_workspace_layout(const moe_dims* dims, moe_ws_layout* layout) {
    if (!layout || !dims_ok(dims)) return MOE_ERR_INVALID_ARG;
    layout_of(dims, layout);
    return MOE_OK;
}

size_t moe_workspace_bytes(const moe_dims* dims) {
    if (!dims_ok(dims)) return 0;
    moe_ws_layout L;
    layout_of(dims, &L);
    return L.total;
}

int moe_route(int32_t num_tokens, int32_t top_k, int32_t num_experts, const int32_t* topk_ids,
              const moe_route_out* out, void* stream) {
    if (!out || num_tokens < 0 || top_k < 1 || top_k > 8 || num_experts < 1 || num_experts > kMaxExperts)
        return MOE_ERR_INVALID_ARG;
    if ((int64_t)num_tokens * top_k >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    if (!out->counts || !out->offsets || !out->padded_offsets || !out->row_src || !out->tile_expert ||
        !out->tile_row0 || !out->stats)
        return MOE_ERR_INVALID_ARG;
    const int64_t N = (int64_t)num_tokens * top_k;
    if (N > 0 && (!topk_ids || !out->pos || !out->sorted_p || !out->ppos)) return MOE_ERR_INVALID_ARG;
    RouteArgs a{};
    a.ids = topk_ids;
    a.N = (int32_t)N;
    a.E = num_experts;
    route_caps(N, num_experts, &a.n_pad_cap, &a.tile_cap);
    a.nb1 = a.nb2 = 0;
    a.mb1_max = kMaxRowBlocks1;
    a.full = 1;
    a.counts = out->counts;
    a.offsets = out->offsets;
    a.padded_offsets = out->padded_offsets;
    a.pos = out->pos;
    a.sorted_p = out->sorted_p;
    a.ppos = out->ppos;
    a.row_src = out->row_src;
    a.tile_expert = out->tile_expert;
    a.tile_row0 = out->tile_row0;
    a.ctl = out->stats;  // only words 0..3 are written when no task lists are built
    if (launch_route(a, static_cast<hipStream_t>(stream)) != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
}

static int forward_impl(const moe_dims* dims, const void* x, const int32_t* topk_ids, const float* topk_w,
                        const void* w1, const void* w2, const moe_scales* scales, void* out, void* workspace,
                        size_t workspace_bytes, void* stream, void* const* events) {
    if (!dims) return MOE_ERR_INVALID_ARG;
    if (!dims_ok(dims)) {
        // shape fields present but outside the envelope
        if (dims->mode < 0 || dims->mode > MOE_MODE_INT8 || dims->num_tokens < 0 || dims->num_experts < 1 || dims->top_k < 1 ||
            dims->d_hidden <= 0 || dims->d_expert <= 0 ||
            (dims->weight_layout != MOE_WEIGHTS_ROW_MAJOR && dims->weight_layout != MOE_WEIGHTS_PACKED) ||
            (dims->activation != MOE_ACT_SWIGLU && dims->activation != MOE_ACT_SWIGLU_CLAMPED) ||
            (dims->launch != MOE_LAUNCH_MULTI && dims->launch != MOE_LAUNCH_SINGLE))
            return MOE_ERR_INVALID_ARG;
        return MOE_ERR_UNSUPPORTED;
    }
    const int mode = dims->mode;
    const int64_t T = dims->num_tokens;
    if (T == 0) return MOE_OK;
    const bool single = dims->launch == MOE_LAUNCH_SINGLE;
    if (single && !single_ok(dims)) return MOE_ERR_UNSUPPORTED;
    if (!x || !topk_ids || !topk_w || !w1 || !w2 || !out) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w1) || !aligned16(w2) || !aligned16(out) || !aligned16(topk_ids) ||
        !aligned16(topk_w))
        return MOE_ERR_INVALID_ARG;
    if (mode_fp8(mode) && (!scales || !scales->x_scale || !scales->w1_scale || !scales->w2_scale))
        return MOE_ERR_INVALID_ARG;
    // INT8: one fp32 scale per token (4-byte aligned)
    if (mode == MOE_MODE_INT8 && (!scales || !scales->x_scale || ((uintptr_t)scales->x_scale & 3)))
        return MOE_ERR_INVALID_ARG;
    // MXFP8 scale rows are loaded 4 bytes at a time
    if (mode == MOE_MODE_MXFP8 && (((uintptr_t)scales->x_scale | (uintptr_t)scales->w1_scale | (uintptr_t)scales->w2_scale) & 3))
        return MOE_ERR_INVALID_ARG;
    moe_ws_layout L;
    layout_of(dims, &L);
    if (!workspace || workspace_bytes < L.total || ((uintptr_t)workspace & (kAlign - 1))) return MOE_ERR_WORKSPACE;

    int cus = 0, occ1 = 1, occ2 = 1;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (single) {
        int occ = 1;
        if (device_info(mode, false, false, &cus, &occ1, &occ2, &occ) != hipSuccess) return MOE_ERR_HIP;
        const int64_t N = T * dims->top_k;
        const int64_t E = dims->num_experts;
        const int mtb = layer_mtile_blocks(mode);
        // at most one workgroup per task
        const int64_t mtiles = L.tile_cap / mtb + std::min<int64_t>(E, N);
        const int64_t tasks = mtiles * (dims->d_expert / L.block_n1 + dims->d_hidden / L.block_n2);
        const int grid = (int)std::max<int64_t>(std::min<int64_t>(tasks, (int64_t)cus * occ), 1);
        LayerArgs la{};
        la.g1.x = x;
        la.g1.x_scale = mode_fp8(mode) ? scales->x_scale : nullptr;
        la.g1.w1 = w1;
        la.g1.w1_scale = mode_fp8(mode) ? scales->w1_scale : nullptr;
        la.g1.h = at<void>(workspace, L.h);
        la.g1.h_scale = mode_fp8(mode) ? at<unsigned char>(workspace, L.h_scale) : nullptr;
        la.g1.topk_w = topk_w;
        la.g1.k = dims->top_k;
        la.g1.d_h = dims->d_hidden;
        la.g1.d_e = dims->d_expert;
        la.g1.packed = dims->weight_layout == MOE_WEIGHTS_PACKED;
        la.g1.act = dims->activation;
        la.g2.h = la.g1.h;
        la.g2.h_scale = la.g1.h_scale;
        la.g2.w2 = w2;
        la.g2.w2_scale = mode_fp8(mode) ? scales->w2_scale : nullptr;
        la.g2.y = at<void>(workspace, L.y);
        la.g2.d_h = dims->d_hidden;
        la.g2.d_e = dims->d_expert;
        la.g2.packed = la.g1.packed;
        la.ids = topk_ids;
        la.sync = at<int32_t>(workspace, L.sync);
        la.out = out;
        la.T = (int32_t)T;
        la.N = (int32_t)N;
        la.E = dims->num_experts;
        la.k = dims->top_k;
        la.nb1 = dims->d_expert / L.block_n1;
        la.nb2 = dims->d_hidden / L.block_n2;
        hipEvent_t e0 = events ? static_cast<hipEvent_t>(events[0]) : nullptr;
        hipEvent_t e1 = events ? static_cast<hipEvent_t>(events[1]) : nullptr;
        if (launch_layer(mode, la, grid, s, e0, e1) != hipSuccess) return MOE_ERR_HIP;
        for (int i = 2; events && i < 8; ++i)
            if (hipEventRecord(static_cast<hipEvent_t>(events[i]), s) != hipSuccess) return MOE_ERR_HIP;
        return MOE_OK;
    }
    const bool wide = fp8_wide(mode, T, dims->top_k, dims->d_hidden, dims->d_expert);
    const bool wide2 =
        fp8_wide2(mode, dims->launch, T, dims->top_k, dims->num_experts, dims->d_hidden, dims->d_expert);
    if (device_info(mode, wide, wide2, &cus, &occ1, &occ2) != hipSuccess) return MOE_ERR_HIP;
    // timing events of launch i (route, GEMM-1, GEMM-2, combine), or none
    auto ev = [&](int i) -> hipEvent_t { return events ? static_cast<hipEvent_t>(events[i]) : nullptr; };
    const int32_t E = dims->num_experts, k = dims->top_k, d_h = dims->d_hidden, d_e = dims->d_expert;

    RouteArgs r{};
    r.ids = topk_ids;
    r.N = (int32_t)(T * k);
    r.E = E;
    r.n_pad_cap = L.n_pad_cap;
    r.tile_cap = L.tile_cap;
    r.nb1 = d_e / L.block_n1;
    r.nb2 = d_h / L.block_n2;
    r.min_tasks1 = cus * occ1;
    r.mb1_max = wide ? kMaxRowBlocksFp8G1 : kMaxRowBlocks1;
    r.mb2 = gemm2_row_blocks(mode, wide2);
    r.mix1 = mode != MOE_MODE_FP8 && !wide;
    // GEMM-2's tasks are short: 128-row tiles only when every workgroup slot
    // still gets two tasks (Qwen shapes at 1024 tokens stay at 64-row tiles);
    // the 8-wave FP8 kernel's 256-row tiles when every slot gets one
    r.min_tasks2 = (wide2 ? 1 : 2) * cus * occ2;
    // persistent grids: at most one workgroup per task, at most what fits on the chip
    const int grid1 = (int)std::max<int64_t>(std::min<int64_t>(L.task1_cap, (int64_t)cus * occ1), 1);
    const int grid2 = (int)std::max<int64_t>(std::min<int64_t>(L.task2_cap, (int64_t)cus * occ2), 1);
    r.grid1 = grid1;
    r.grid2 = grid2;
    r.counts = at<int32_t>(workspace, L.counts);
    r.offsets = at<int32_t>(workspace, L.offsets);
    r.padded_offsets = at<int32_t>(workspace, L.padded_offsets);
    r.pos = at<int32_t>(workspace, L.pos);
    r.sorted_p = at<int32_t>(workspace, L.sorted_p);
    r.ppos = at<int32_t>(workspace, L.ppos);
    r.row_src = at<int32_t>(workspace, L.row_src);
    r.tile_expert = at<int32_t>(workspace, L.tile_expert);
    r.tile_row0 = at<int32_t>(workspace, L.tile_row0);
    r.ctl = at<int32_t>(workspace, L.stats);
    r.tasks1 = at<int4>(workspace, L.tasks1);
    r.tasks2 = at<int4>(workspace, L.tasks2);
    r.zero = at<unsigned char>(workspace, L.zero);
    if (launch_route(r, s, ev(0), ev(1)) != hipSuccess) return MOE_ERR_HIP;
    const void* xg = x;
    if (mode == MOE_MODE_F32ACT) {
        uint16_t* xb = at<uint16_t>(workspace, L.x_bf16);
        if (launch_x_to_bf16(static_cast<const float*>(x), xb, T * d_h, s) != hipSuccess) return MOE_ERR_HIP;
        xg = xb;
    } else if (mode == MOE_MODE_INT8) {
        uint16_t* xb = at<uint16_t>(workspace, L.x_bf16);
        if (launch_i8_to_bf16(static_cast<const int8_t*>(x), xb, T * d_h, s) != hipSuccess) return MOE_ERR_HIP;
        xg = xb;
    }

    Gemm1Args g1{};
    g1.x = xg;
    g1.x_scale = mode_fp8(mode) ? scales->x_scale : nullptr;
    g1.w1 = w1;
    g1.w1_scale = mode_fp8(mode) ? scales->w1_scale : nullptr;
    g1.row_src = r.row_src;
    g1.tasks = r.tasks1;
    g1.ctl = r.ctl;
    g1.zero = r.zero;
    g1.h = at<void>(workspace, L.h);
    g1.h_scale = mode_fp8(mode) ? at<unsigned char>(workspace, L.h_scale) : nullptr;
    g1.topk_w = topk_w;
    g1.row_w = at<float>(workspace, L.row_w);
    g1.x_row_scale = mode == MOE_MODE_INT8 ? static_cast<const float*>(scales->x_scale) : nullptr;
    g1.k = k;
    g1.d_h = d_h;
    g1.d_e = d_e;
    g1.packed = dims->weight_layout == MOE_WEIGHTS_PACKED;
    g1.act = dims->activation;
    if (launch_gemm1(gemm_mode(mode), wide, g1, grid1, s, ev(2), ev(3)) != hipSuccess) return MOE_ERR_HIP;

    Gemm2Args g2{};
    g2.h = g1.h;
    g2.h_scale = g1.h_scale;
    g2.w2 = w2;
    g2.w2_scale = mode_fp8(mode) ? scales->w2_scale : nullptr;
    g2.row_src = r.row_src;
    g2.row_w = g1.row_w;
    g2.tasks = r.tasks2;
    g2.ctl = r.ctl;
    g2.zero = r.zero;
    g2.y = at<void>(workspace, L.y);
    g2.d_h = d_h;
    g2.d_e = d_e;
    g2.packed = dims->weight_layout == MOE_WEIGHTS_PACKED;
    if (launch_gemm2(gemm_mode(mode), wide2, g2, grid2, s, ev(4), ev(5)) != hipSuccess) return MOE_ERR_HIP;

    CombineArgs c{};
    c.y = g2.y;
    c.ids = topk_ids;
    c.out = out;
    c.T = (int32_t)T;
    c.k = k;
    c.E = E;
    c.d_h = d_h;
    if (launch_combine(gemm_mode(mode), c, s, ev(6), ev(7)) != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
}

// ------------------------------------------------------------- backward
// Workspace of moe_fused_backward: routing arrays, transposed weights, the
// recomputed gate/up accumulators and every intermediate of the backward.
struct BwdLayout {
    size_t counts, offsets, padded_offsets, pos, sorted_p, ppos, row_src, tile_expert, tile_row0, stats;
    size_t w1t, w2t, gu, q, h, dgu, dxp, dgut, xpt, dyt, ht, total;
    int64_t n_pad_cap, tile_cap, ldt;
};

static void bwd_layout_of(const moe_dims* d, BwdLayout* L) {
    const int64_t N = (int64_t)d->num_tokens * d->top_k, E = d->num_experts, d_h = d->d_hidden, d_e = d->d_expert;
    route_caps(N, E, &L->n_pad_cap, &L->tile_cap);
    L->ldt = (L->n_pad_cap + 63) / 64 * 64;  // row length of the transposed (K = padded rows) operands
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align_up(o + (bytes ? bytes : 1));
        return at;
    };
    L->counts = take(4 * E);
    L->offsets = take(4 * (E + 1));
    L->padded_offsets = take(4 * (E + 1));
    L->pos = take(4 * N);
    L->sorted_p = take(4 * N);
    L->ppos = take(4 * N);
    L->row_src = take(4 * L->n_pad_cap);
    L->tile_expert = take(4 * L->tile_cap);
    L->tile_row0 = take(4 * L->tile_cap);
    L->stats = take(4 * kCtlWords);
    L->w1t = take(2 * (size_t)E * 2 * d_e * d_h);
    L->w2t = take(2 * (size_t)E * d_h * d_e);
    L->gu = take(4 * (size_t)L->n_pad_cap * 2 * d_e);
    L->q = take(4 * (size_t)L->n_pad_cap * d_e);
    L->h = take(2 * (size_t)L->n_pad_cap * d_e);
    L->dgu = take(2 * (size_t)L->n_pad_cap * 2 * d_e);
    L->dxp = take(4 * (size_t)L->n_pad_cap * d_h);
    L->dgut = take(2 * (size_t)2 * d_e * L->ldt);
    L->xpt = take(2 * (size_t)d_h * L->ldt);
    L->dyt = take(2 * (size_t)d_h * L->ldt);
    L->ht = take(2 * (size_t)d_e * L->ldt);
    L->total = o;
}

static bool bwd_dims_ok(const moe_dims* d) {
    return dims_ok(d) && d->mode == MOE_MODE_BF16 && d->weight_layout == MOE_WEIGHTS_ROW_MAJOR &&
           d->activation == MOE_ACT_SWIGLU;
}

int moe_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
    if (!workspace || workspace_bytes < MOE_SYNC_BYTES || ((uintptr_t)workspace & (kAlign - 1))) return MOE_ERR_WORKSPACE;
    if (launch_sync_clear(static_cast<int32_t*>(workspace), static_cast<hipStream_t>(stream)) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

int moe_pack_weights(const moe_dims* dims, const void* w1, const void* w2, void* w1_packed, void* w2_packed,
                     void* stream) {
    if (!dims) return MOE_ERR_INVALID_ARG;
    moe_dims d = *dims;
    d.weight_layout = MOE_WEIGHTS_ROW_MAJOR;  // the packing itself ignores the field
    if (!dims_ok(&d)) return MOE_ERR_INVALID_ARG;
    if (!w1 || !w2 || !w1_packed || !w2_packed) return MOE_ERR_INVALID_ARG;
    if (!aligned16(w1) || !aligned16(w2) || !aligned16(w1_packed) || !aligned16(w2_packed)) return MOE_ERR_INVALID_ARG;
    const int64_t eb = mode_fp8(d.mode) ? 1 : 2;
    const int64_t E = d.num_experts, d_h = d.d_hidden, d_e = d.d_expert;
    const int64_t b1 = E * 2 * d_e * d_h * eb, b2 = E * d_h * d_e * eb;
    auto overlap = [](const void* a, int64_t na, const void* b, int64_t nb) {
        const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
        return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
    };
    if (overlap(w1_packed, b1, w1, b1) || overlap(w1_packed, b1, w2, b2) || overlap(w2_packed, b2, w1, b1) ||
        overlap(w2_packed, b2, w2, b2) || overlap(w1_packed, b1, w2_packed, b2))
        return MOE_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (launch_pack(w1, w1_packed, E, d_e, d_h * eb, gemm1_block_n(d.mode), true, s) != hipSuccess)
        return MOE_ERR_HIP;
    if (launch_pack(w2, w2_packed, E, d_h, d_e * eb, gemm2_block_n(d.mode, false), false, s) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

int moe_fused_forward(const moe_dims* dims, const void* x, const int32_t* topk_ids, const float* topk_w,
                      const void* w1, const void* w2, const moe_scales* scales, void* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
    return forward_impl(dims, x, topk_ids, topk_w, w1, w2, scales, out, workspace, workspace_bytes, stream,
                        nullptr);
}

int moe_fused_forward_noalloc(const moe_dims* dims, const void* x, const int32_t* topk_ids, const float* topk_w,
                              const void* w1, const void* w2, const moe_scales* scales, void* out, void* stream) {
    // the size check comes first: a rejected call touches no device
    if (dims && dims_ok(dims) && dims->num_tokens > 0) {
        moe_ws_layout L;
        layout_of(dims, &L);
        if (L.total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
    }
    if (dims && dims->num_tokens == 0 && dims_ok(dims)) return MOE_OK;
    void* ws = nullptr;
    if (dims && dims_ok(dims)) {
        if (scratch_of_current_device(&ws) != hipSuccess) {
            (void)hipGetLastError();
            return MOE_ERR_HIP;
        }
    }
    // invalid dims fall through to forward_impl's own checks (ws may be null
    // then; it is rejected before any use)
    return forward_impl(dims, x, topk_ids, topk_w, w1, w2, scales, out, ws, MOE_NOALLOC_SCRATCH_BYTES, stream,
                        nullptr);
}

size_t moe_backward_workspace_bytes(const moe_dims* dims) {
    if (!bwd_dims_ok(dims)) return 0;
    BwdLayout L;
    bwd_layout_of(dims, &L);
    return L.total;
}

int moe_fused_backward(const moe_dims* dims, const void* x, const int32_t* topk_ids, const float* topk_w,
                       const void* w1, const void* w2, const void* dout, float* dx, float* dw1, float* dw2,
                       float* dtopk_w, void* workspace, size_t workspace_bytes, void* stream) {
    if (!dims) return MOE_ERR_INVALID_ARG;
    if (!dims_ok(dims)) return MOE_ERR_INVALID_ARG;
    if (!bwd_dims_ok(dims)) return MOE_ERR_UNSUPPORTED;
    const int64_t T = dims->num_tokens;
    if (T == 0) return MOE_OK;
    if (!x || !topk_ids || !topk_w || !w1 || !w2 || !dout || !dx || !dw1 || !dw2 || !dtopk_w)
        return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w1) || !aligned16(w2) || !aligned16(dout) || !aligned16(dx) ||
        !aligned16(dw1) || !aligned16(dw2) || !aligned16(topk_ids) || !aligned16(topk_w) || !aligned16(dtopk_w))
        return MOE_ERR_INVALID_ARG;
    BwdLayout L;
    bwd_layout_of(dims, &L);
    if (!workspace || workspace_bytes < L.total || ((uintptr_t)workspace & (kAlign - 1))) return MOE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int32_t E = dims->num_experts, k = dims->top_k, d_h = dims->d_hidden, d_e = dims->d_expert;
    const int64_t N = T * k;

    RouteArgs r{};
    r.ids = topk_ids;
    r.N = (int32_t)N;
    r.E = E;
    r.n_pad_cap = L.n_pad_cap;
    r.tile_cap = L.tile_cap;
    r.nb1 = r.nb2 = 0;
    r.mb1_max = kMaxRowBlocks1;
    r.full = 1;
    r.counts = at<int32_t>(workspace, L.counts);
    r.offsets = at<int32_t>(workspace, L.offsets);
    r.padded_offsets = at<int32_t>(workspace, L.padded_offsets);
    r.pos = at<int32_t>(workspace, L.pos);
    r.sorted_p = at<int32_t>(workspace, L.sorted_p);
    r.ppos = at<int32_t>(workspace, L.ppos);
    r.row_src = at<int32_t>(workspace, L.row_src);
    r.tile_expert = at<int32_t>(workspace, L.tile_expert);
    r.tile_row0 = at<int32_t>(workspace, L.tile_row0);
    r.ctl = at<int32_t>(workspace, L.stats);
    if (launch_route(r, s) != hipSuccess) return MOE_ERR_HIP;
    const int32_t* poff = r.padded_offsets;
    const uint16_t* xb = static_cast<const uint16_t*>(x);
    const uint16_t* w1b = static_cast<const uint16_t*>(w1);
    const uint16_t* w2b = static_cast<const uint16_t*>(w2);
    const uint16_t* db = static_cast<const uint16_t*>(dout);
    uint16_t* w1t = at<uint16_t>(workspace, L.w1t);
    uint16_t* w2t = at<uint16_t>(workspace, L.w2t);
    float* gu = at<float>(workspace, L.gu);
    float* q = at<float>(workspace, L.q);
    uint16_t* h = at<uint16_t>(workspace, L.h);
    uint16_t* dgu = at<uint16_t>(workspace, L.dgu);
    float* dxp = at<float>(workspace, L.dxp);
    uint16_t* dgut = at<uint16_t>(workspace, L.dgut);
    uint16_t* xpt = at<uint16_t>(workspace, L.xpt);
    uint16_t* dyt = at<uint16_t>(workspace, L.dyt);
    uint16_t* ht = at<uint16_t>(workspace, L.ht);
    const int R = (int)L.n_pad_cap;
    bool ok = true;
    // transposed weights: W1^T [E][d_h][2 d_e], W2^T [E][d_e][d_h]
    ok = ok && launch_transpose(w1b, d_h, (int64_t)2 * d_e * d_h, w1t, 2 * d_e, (int64_t)2 * d_e * d_h, 2 * d_e, d_h,
                                E, nullptr, 1, nullptr, nullptr, s) == hipSuccess;
    ok = ok && launch_transpose(w2b, d_e, (int64_t)d_h * d_e, w2t, d_h, (int64_t)d_h * d_e, d_h, d_e, E, nullptr, 1,
                                nullptr, nullptr, s) == hipSuccess;
    // recompute [g u] per padded row; q = dout . W2[e]
    ok = ok && launch_bwd_gemm_rows(xb, d_h, r.row_src, k, w1b, d_h, (int64_t)2 * d_e * d_h, gu, 2 * d_e, 2 * d_e, d_h,
                                    r.tile_expert, r.tile_row0, r.ctl, L.tile_cap, s) == hipSuccess;
    ok = ok && launch_bwd_gemm_rows(db, d_h, r.row_src, k, w2t, d_h, (int64_t)d_e * d_h, q, d_e, d_e, d_h,
                                    r.tile_expert, r.tile_row0, r.ctl, L.tile_cap, s) == hipSuccess;
    // h, dg, du, dtopk_w
    ok = ok && launch_bwd_act(gu, q, r.row_src, poff + E, topk_w, h, dgu, dtopk_w, d_e, L.n_pad_cap, s) == hipSuccess;
    // dX per row, then per token over its slots (also zeroes dtopk_w of dropped slots)
    ok = ok && launch_bwd_gemm_rows(dgu, 2 * d_e, nullptr, 1, w1t, 2 * d_e, (int64_t)2 * d_e * d_h, dxp, d_h, d_h,
                                    2 * d_e, r.tile_expert, r.tile_row0, r.ctl, L.tile_cap, s) == hipSuccess;
    ok = ok && launch_bwd_dx(dxp, r.ppos, topk_ids, dx, dtopk_w, (int)T, k, E, d_h, s) == hipSuccess;
    // K-contiguous operands of the weight gradients (K = an expert's padded rows)
    ok = ok && launch_transpose(dgu, 2 * d_e, 0, dgut, L.ldt, 0, R, 2 * d_e, 1, nullptr, 1, nullptr, poff + E, s) ==
                   hipSuccess;
    ok = ok && launch_transpose(xb, d_h, 0, xpt, L.ldt, 0, R, d_h, 1, r.row_src, k, nullptr, poff + E, s) ==
                   hipSuccess;
    ok = ok && launch_transpose(db, d_h, 0, dyt, L.ldt, 0, R, d_h, 1, r.row_src, k, topk_w, poff + E, s) ==
                   hipSuccess;
    ok = ok && launch_transpose(h, d_e, 0, ht, L.ldt, 0, R, d_e, 1, nullptr, 1, nullptr, poff + E, s) == hipSuccess;
    // dW1[e] = [dg du]^T . x rows; dW2[e] = (w dout)^T . h rows
    ok = ok && launch_bwd_gemm_experts(dgut, L.ldt, xpt, L.ldt, dw1, d_h, (int64_t)2 * d_e * d_h, E, 2 * d_e, d_h,
                                       poff, s) == hipSuccess;
    ok = ok && launch_bwd_gemm_experts(dyt, L.ldt, ht, L.ldt, dw2, d_e, (int64_t)d_h * d_e, E, d_h, d_e, poff, s) ==
                   hipSuccess;
    return ok ? MOE_OK : MOE_ERR_HIP;
}

int moe_fused_forward_profiled(const moe_dims* dims, const void* x, const int32_t* topk_ids, const float* topk_w,
                               const void* w1, const void* w2, const moe_scales* scales, void* out,
                               void* workspace, size_t workspace_bytes, void* stream, void* const* events) {
    if (!events) return MOE_ERR_INVALID_ARG;
    for (int i = 0; i < 8; ++i)
        if (!events[i]) return MOE_ERR_INVALID_ARG;
    return forward_impl(dims, x, topk_ids, topk_w, w1, w2, scales, out, workspace, workspace_bytes, stream,
                        events);
}

}  // extern "C"
