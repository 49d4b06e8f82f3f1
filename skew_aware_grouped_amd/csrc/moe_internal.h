// Internal declarations shared by the HIP translation units of the fused MoE
// library (kernels and the C-ABI host code).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_fused.h"

namespace moe {

// Rows per group block.  Equal to the M size of the 16x16 MFMA tiles, so a
// cold expert with a handful of tokens pads to at most 15 rows.
constexpr int kBlockM = 16;
// A GEMM-1 task covers up to kMaxRowBlocks1 consecutive group blocks of one
// expert (128 rows), so a hot expert's W1 is streamed once per 128 of its
// rows, or kSmallRowBlocks when 128-row tiles would leave too few tasks.  A
// GEMM-2 task covers up to gemm2_row_blocks(mode) blocks: 8 in the bf16 and
// FP8 modes, 4 in MXFP8 mode (its 128-row body would need more registers than
// two workgroups per CU leave).  The kernels carry one fully unrolled body per
// block count.
constexpr int kMaxRowBlocks1 = 8;
constexpr int kMaxRowBlocks2 = 8;
constexpr int kSmallRowBlocks = 4;
constexpr int kMaxRowBlocks = kMaxRowBlocks1;
// FP8 GEMM-1 runs its own kernel: 8 waves (two per SIMD, so one wave's
// block-scale promotion overlaps the other's MFMAs) and tasks of up to 16
// group blocks (256 rows), so that each weight byte brought into LDS feeds
// twice the rows: the per-CU rate of direct-to-LDS loads, not HBM, bounds
// this kernel at large batches.
constexpr int kMaxRowBlocksFp8G1 = 16;
constexpr int kGemm1Fp8Waves = 8;
constexpr int kGemm1Fp8Threads = 64 * kGemm1Fp8Waves;
// It serves batches of at least kFp8WideMinAssignments routed rows (64 rows
// per expert on average at 32 experts; measured: at 2048 assignments of the
// DeepSeek shapes it is 13% faster than the 4-wave kernel, at 1024 3%
// slower); smaller FP8 batches take the 4-wave kernel, whose stage loads and
// epilogue are shorter per task.
// The 8-wave kernel addresses x, one expert's W1 and the scales with 32-bit
// offsets from uniform bases, so it also needs T*d_h and 2*d_e*d_h below 2^31.
constexpr int64_t kFp8WideMinAssignments = 2048;
// MXFP8 runs the same kernels with its scale bytes (four loads of scale words
// per stage more) from kMxWideMinAssignments (measured at 2048 assignments
// of the Qwen shapes: 41 us against the 4-wave kernel's 35; at 8192 tokens of
// the DeepSeek shapes 491 against 680).
constexpr int64_t kMxWideMinAssignments = 4096;
inline bool fp8_wide(int mode, int64_t T, int64_t k, int64_t d_h, int64_t d_e) {
    const int64_t min_n = mode == MOE_MODE_MXFP8 ? kMxWideMinAssignments : kFp8WideMinAssignments;
    return (mode == MOE_MODE_FP8 || mode == MOE_MODE_MXFP8) && T * k >= min_n && T * d_h < ((int64_t)1 << 31) &&
           2 * d_e * d_h < ((int64_t)1 << 31);
}
inline int gemm1_max_row_blocks(int mode, int64_t T, int64_t k, int64_t d_h, int64_t d_e) {
    return fp8_wide(mode, T, k, d_h, d_e) ? kMaxRowBlocksFp8G1 : kMaxRowBlocks1;
}
// FP8 GEMM-2 from kFp8Wide2MinAssignments routed rows on (four launches
// only: the single launch keeps its own task shapes) runs an 8-wave kernel on
// the same geometry: tasks of up to 16 group blocks by 256 output columns, so
// it needs d_h a multiple of 256 and n_pad*d_e below 2^31 (32-bit offsets
// into h).  Measured at 1024 DeepSeek-shaped assignments: 97 -> 86 us.
// MXFP8 takes it only with d_e of at least 1024 (K blocks enough to carry a
// 256x256 task's fixed costs; measured at 2048 assignments: DeepSeek shapes,
// d_e = 2048, 134 -> 114 us; Qwen shapes, d_e = 768, 21.5 -> 24 us).
constexpr int64_t kFp8Wide2MinAssignments = 1024;
inline bool fp8_wide2(int mode, int launch, int64_t T, int64_t k, int64_t E, int64_t d_h, int64_t d_e) {
    const int64_t n_pad = T * k + (E < T * k ? E : T * k) * (kBlockM - 1);
    return (mode == MOE_MODE_FP8 || (mode == MOE_MODE_MXFP8 && d_e >= 1024)) && launch == MOE_LAUNCH_MULTI &&
           T * k >= kFp8Wide2MinAssignments &&
           d_h % 256 == 0 && n_pad * d_e < ((int64_t)1 << 31);
}
constexpr int kMaxRowBlocksFp8G2 = 16;
// Workgroup of the GEMM kernels: 4 wave64s, one per SIMD.
constexpr int kGemmWaves = 4;
constexpr int kGemmThreads = 64 * kGemmWaves;
// Routing runs in one workgroup of 16 waves.
constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kMaxExperts = 256;
constexpr int kQ = 128;  // FP8 block-scale granularity
// Bytes of zeros kept in the workspace: padding rows of a group block read
// their operand (and FP8 row scale) from here.
constexpr int kZeroBytes = 256;

// Control block of the workspace (int32 words): statistics, then the
// per-XCD task queues of the two GEMM kernels.  Each queue has its own
// 64-byte line for its counter so the eight XCDs' atomics do not share one.
enum {
    kStatDropped = 0,
    kStatTiles,
    kStatPadRows,
    kStatTasks1,
    kStatTasks2,
    kStatCount = 8,
    kXcds = 8,          // XCDs of an MI355X; a task list is split into this many segments
    kQueueStride = 16,  // words between two queue counters
    kCtlQueue1 = 16,    // GEMM-1 counters: [kCtlQueue1 + kQueueStride * x]
    kCtlQueue2 = kCtlQueue1 + kXcds * kQueueStride,
    kCtlSeg1 = kCtlQueue2 + kXcds * kQueueStride,  // GEMM-1 segment starts [kXcds + 1]
    kCtlSeg2 = kCtlSeg1 + 16,                       // GEMM-2 segment starts [kXcds + 1]
    kCtlWords = kCtlSeg2 + 16
};

// First task of GEMM workgroup g, assigned without the queue: workgroup g
// takes task j = g / kXcds of segment x = g % kXcds if that segment has more
// than j tasks (workgroups are dispatched to the XCDs in turn, so x is
// normally the workgroup's own XCD).  Returns how many tasks of segment x are
// taken that way, where the segment's queue counter starts.
__host__ __device__ inline int static_tasks(int grid, int x, int seg_len) {
    const int n = (grid - x + kXcds - 1) / kXcds;  // workgroups g < grid with g % kXcds == x
    return n < seg_len ? n : seg_len;
}

// Output columns per GEMM task.  GEMM-1 FP8 needs 128 so that one task owns
// a whole 128-column requantisation group of the intermediate and a single
// block row of W1's scales; bf16 GEMM-1 uses 64; GEMM-2 uses 128 (one W2
// scale block row).
constexpr bool mode_fp8(int mode) { return mode == MOE_MODE_FP8 || mode == MOE_MODE_MXFP8; }  // e4m3 operands
// The GEMM kernels of a mode: INT8 tokens run the bf16 GEMMs on their widened codes
inline int gemm_mode(int mode) { return mode == MOE_MODE_INT8 ? MOE_MODE_BF16 : mode; }
inline int gemm1_block_n(int mode) { return mode_fp8(mode) ? 128 : 64; }
inline int gemm2_block_n(int, bool wide2) { return wide2 ? 256 : 128; }
inline int gemm2_row_blocks(int mode, bool wide2) {
    return wide2 ? kMaxRowBlocksFp8G2 : mode == MOE_MODE_MXFP8 ? kSmallRowBlocks : kMaxRowBlocks2;
}

struct RouteArgs {
    const int32_t* ids;
    int32_t N, E;
    int64_t n_pad_cap, tile_cap;
    int32_t nb1, nb2;  // column blocks of GEMM-1 / GEMM-2; 0 = do not build task lists
    int32_t min_tasks1;  // GEMM-1 takes its largest M-tiles only if that leaves this many tasks
    int32_t mb1_max;     // largest GEMM-1 M-tile in group blocks (gemm1_max_row_blocks)
    int32_t mb2;         // largest GEMM-2 M-tile in group blocks (gemm2_row_blocks)
    int32_t min_tasks2;  // GEMM-2 takes 8-block M-tiles only if that leaves this many tasks
    int32_t mix1;        // GEMM-1 may mix 8- and 4-block M-tiles (not in FP8 mode, whose 128-row epilogue is long)
    int32_t grid1, grid2;  // workgroups of the GEMM kernels (their first tasks are assigned statically)
    int32_t full;          // also write pos, ppos, sorted_p and the block map (the layer consumes row_src and task lists)
    int32_t *counts, *offsets, *padded_offsets, *pos, *sorted_p, *ppos, *row_src, *tile_expert, *tile_row0;
    int32_t* ctl;  // control block [kCtlWords]
    int4* tasks1;
    int4* tasks2;
    unsigned char* zero;  // kZeroBytes to clear (may be null)
};

struct Gemm1Args {
    const void* x;  // e4m3 codes or bf16 [T, d_h]
    const void* x_scale;  // FP8: fp32 [T, d_h/128]; MXFP8: E8M0 bytes [T, d_h/32]
    const void* w1;
    const void* w1_scale;  // FP8: fp32 128x128 block scales; MXFP8: E8M0 bytes per row per 32
    const int32_t* row_src;
    const int4* tasks;
    int32_t* ctl;
    const unsigned char* zero;
    void* h;
    void* h_scale;  // FP8: fp32 [n_pad, d_e/128]; MXFP8: E8M0 bytes [n_pad, d_e/32]
    const float* topk_w;  // [T*k] routing weights
    float* row_w;         // [n_pad] routing weight of each padded row (0 on padding), written by column block 0
    const float* x_row_scale;  // INT8 mode: fp32 [T], one per token, applied to GEMM-1's accumulators; else null
    int32_t k, d_h, d_e;
    int32_t packed;  // W1 in the packed tile order
    int32_t act;     // MOE_ACT_*
};

struct Gemm2Args {
    const void* h;
    const void* h_scale;
    const void* w2;
    const void* w2_scale;
    const int32_t* row_src;
    const float* row_w;  // from GEMM-1
    const int4* tasks;
    int32_t* ctl;
    const unsigned char* zero;
    void* y;
    int32_t d_h, d_e;
    int32_t packed;  // W2 in the packed tile order
};

// ---------------------------------------------------------- single launch
// moe_dims.launch == MOE_LAUNCH_SINGLE: the whole layer in one persistent
// kernel (moe_layer.hip).  Its envelope: BF16, FP8 or MXFP8 data, at most
// kLayerMaxN routed assignments, T * (d_h / 128) at most kSyncArriveWords.
constexpr int kLayerMaxN = 2048;
// M-tiles of the single launch, in group blocks: 128 rows in the bf16 modes,
// 64 in the FP8 ones (their GEMM-1 task requantises h, which costs more per
// row at 128 rows)
inline int layer_mtile_blocks(int mode) { return mode_fp8(mode) ? kSmallRowBlocks : kMaxRowBlocks1; }
// Synchronisation block at the start of every workspace (int32 words), the
// same size for all dims so that no call's other sections ever overlap it.
// It holds zeros before the first single-launch call on a workspace and every
// such call leaves it zero: the queue and exit counters and the M-tile
// counters are reset by the last workgroup to finish, each arrival counter by
// the workgroup that completes it.  The four-launch path never touches it.
enum {
    kSyncQueue = 0,        // task queue counter (own 128-byte line)
    kSyncExit = 32,        // workgroups finished
    kSyncTimeouts = 64,    // bounded waits that ran out (diagnostic, never reset by the kernel)
    kSyncZero = 96,        // 256 bytes of zeros: padding rows read their operand here
    kSyncDone = 256,       // [group block] GEMM-1 column blocks stored for the GEMM-2 M-tile starting there
    kSyncDoneWords = 512,  // >= (kLayerMaxN + kMaxExperts * 15) / 16
    kSyncArrive = kSyncDone + kSyncDoneWords,  // [token * (d_h / 128) + column block] y rows stored
    kSyncArriveWords = 65536,
    kSyncWords = kSyncArrive + kSyncArriveWords
};

struct LayerArgs {
    Gemm1Args g1;  // x, x_scale, w1, w1_scale, h, h_scale, topk_w, k, d_h, d_e, packed, act
    Gemm2Args g2;  // h, h_scale, w2, w2_scale, y (fp32 [T*k, d_h]), d_h, d_e, packed
    const int32_t* ids;
    int32_t* sync;  // kSyncWords
    void* out;      // bf16 [T, d_h]
    int32_t T, N, E, k, nb1, nb2;
};

struct CombineArgs {
    const void* y;
    const int32_t* ids;
    void* out;
    int32_t T, k, E, d_h;
};

// Launchers.  With t0/t1 (timing events created by the caller) the kernel's
// own start and end are recorded, as the dispatch sees them.
hipError_t launch_route(const RouteArgs& a, hipStream_t s, hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
// x fp32 -> bf16 (round to nearest even), n elements, multiple of 8
hipError_t launch_x_to_bf16(const float* x, uint16_t* xb, int64_t n, hipStream_t s);
// int8 codes -> bf16 (exact), n elements, multiple of 16
hipError_t launch_i8_to_bf16(const int8_t* x, uint16_t* xb, int64_t n, hipStream_t s);
// W (row-major [E][rows][K bytes]) -> packed tile order for tasks of `bn`
// output columns (gated: gate and up rows of a column block together)
hipError_t launch_pack(const void* w, void* wp, int64_t E, int64_t n_out, int64_t k_bytes, int bn, bool gated,
                       hipStream_t s);
// wide: FP8 and MXFP8 only, the 8-wave kernels (fp8_wide, fp8_wide2)
hipError_t launch_gemm1(int mode, bool wide, const Gemm1Args& a, int grid, hipStream_t s, hipEvent_t t0 = nullptr,
                        hipEvent_t t1 = nullptr);
hipError_t launch_gemm2(int mode, bool wide, const Gemm2Args& a, int grid, hipStream_t s, hipEvent_t t0 = nullptr,
                        hipEvent_t t1 = nullptr);
hipError_t launch_combine(int mode, const CombineArgs& a, hipStream_t s, hipEvent_t t0 = nullptr,
                          hipEvent_t t1 = nullptr);
// Backward pass (BF16 mode; see moe_backward.hip).  Row GEMM: C rows are the
// 16-row group blocks of the padded layout; expert GEMM: per expert, K over
// its padded rows.
hipError_t launch_bwd_gemm_rows(const uint16_t* A, int64_t lda, const int32_t* a_rows, int a_div, const uint16_t* B,
                                int64_t ldb, int64_t b_estride, float* C, int64_t ldc, int N, int K,
                                const int32_t* tile_expert, const int32_t* tile_row0, const int32_t* ctl,
                                int64_t tile_cap, hipStream_t s);
hipError_t launch_bwd_gemm_experts(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, float* C,
                                   int64_t ldc, int64_t c_estride, int E, int M, int N, const int32_t* poff,
                                   hipStream_t s);
hipError_t launch_transpose(const uint16_t* in, int64_t ldi, int64_t in_bstride, uint16_t* out, int64_t ldo,
                            int64_t out_bstride, int R, int C, int batch, const int32_t* rows, int map_div,
                            const float* roww, const int32_t* n_used, hipStream_t s);
hipError_t launch_bwd_act(const float* GU, const float* Q, const int32_t* row_src, const int32_t* poff_end,
                          const float* topk_w, uint16_t* H, uint16_t* dGU, float* dtopk_w, int d_e, int64_t n_pad_cap,
                          hipStream_t s);
hipError_t launch_bwd_dx(const float* dXp, const int32_t* ppos, const int32_t* ids, float* dx, float* dtopk_w, int T,
                         int k, int E, int d_h, hipStream_t s);

// The single-launch layer kernel (grid: at most its resident capacity) and its
// occupancy; sync_clear zeroes a synchronisation block.
hipError_t launch_layer(int mode, const LayerArgs& a, int grid, hipStream_t s, hipEvent_t t0 = nullptr,
                        hipEvent_t t1 = nullptr);
hipError_t layer_occupancy(int mode, int* blocks_per_cu);
hipError_t launch_sync_clear(int32_t* sync, hipStream_t s);

// Resident workgroups per CU of the persistent GEMM kernels (occupancy query;
// wide: the 8-wave FP8 or MXFP8 GEMM-1 and GEMM-2).
hipError_t gemm_occupancy(int mode, bool wide, int* g1_blocks_per_cu, int* g2_blocks_per_cu);

}  // namespace moe
