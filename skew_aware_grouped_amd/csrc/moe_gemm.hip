// Persistent grouped-GEMM kernels of the four-launch layer (GEMM-1 with the
// activation epilogue, GEMM-2 with the routing-weight epilogue, the 8-wave FP8
// GEMM-1), the top-k combine, and the small conversion and packing kernels.
// The task body they share is gemm_task (moe_gemm_task.h).
#include "moe_gemm_task.h"

namespace moe {
namespace {


template <int MODE>
__global__ __launch_bounds__(kGemmThreads) void gemm1_kernel(Gemm1Args a) {
    constexpr int GM = MODE == MOE_MODE_F32ACT ? MOE_MODE_BF16 : MODE;  // x arrives as bf16
    constexpr int RING = Cfg<GM, true>::kRing;
    __shared__ __attribute__((aligned(16))) unsigned char smem[RING];
    __shared__ QueueLds q;
    const int xcd = my_xcd();
    if (threadIdx.x <= kXcds) q.seg[threadIdx.x] = a.ctl[kCtlSeg1 + threadIdx.x];
    if (threadIdx.x == 0) q.mask = 0;
    lds_barrier();
    if (threadIdx.x >= 64 * kSchedWave) {
        Sched sch{a.ctl, kCtlQueue1, a.tasks, a.row_src, nullptr, &q, xcd};
        sch.first();
        sch.load_rows(0);
        sch.publish();
    }
    lds_barrier();
    for (int par = 0;; par ^= 1) {
        // readfirstlane: the task is the same for every thread, and the
        // compiler must know it, or it treats the task loop as divergent and
        // may split a thread-0 region next to the loop's back-edge off the
        // loop while the other lanes iterate on a stale task
        const int t = __builtin_amdgcn_readfirstlane(q.slot);
        if (t < 0) break;
        const int e = __builtin_amdgcn_readfirstlane(q.task.x), row0 = __builtin_amdgcn_readfirstlane(q.task.y);
        const int nsub = __builtin_amdgcn_readfirstlane(q.task.z), cb = __builtin_amdgcn_readfirstlane(q.task.w);
        Sched sch{a.ctl, kCtlQueue1, a.tasks, a.row_src, nullptr, &q, xcd};
#define MOE_G1(NS)                                                                                                \
    gemm_task<GM, true, NS, RING>(a.x, a.x_scale, a.row_src, a.k, a.w1, a.w1_scale, a.zero, e, row0, cb, a.d_h, a.d_e, \
                                  a.packed != 0, smem, &a, nullptr, sch, q.rows[par], q.roww[par], par)
        switch (nsub) {
            case 1: MOE_G1(1); break;
            case 2: MOE_G1(2); break;
            case 3: MOE_G1(3); break;
            case 4: MOE_G1(4); break;
            case 5: MOE_G1(5); break;
            case 6: MOE_G1(6); break;
            case 7: MOE_G1(7); break;
            default: MOE_G1(8); break;
        }
#undef MOE_G1
    }
}

template <int MODE>
__global__ __launch_bounds__(kGemmThreads) void gemm2_kernel(Gemm2Args a) {
    constexpr int RING = Cfg<MODE, false>::kRing;
    __shared__ __attribute__((aligned(16))) unsigned char smem[RING];
    __shared__ QueueLds q;
    const int xcd = my_xcd();
    if (threadIdx.x <= kXcds) q.seg[threadIdx.x] = a.ctl[kCtlSeg2 + threadIdx.x];
    if (threadIdx.x == 0) q.mask = 0;
    lds_barrier();
    if (threadIdx.x >= 64 * kSchedWave) {
        Sched sch{a.ctl, kCtlQueue2, a.tasks, a.row_src, a.row_w, &q, xcd};
        sch.first();
        sch.load_rows(0);
        sch.publish();
    }
    lds_barrier();
    for (int par = 0;; par ^= 1) {
        const int t = __builtin_amdgcn_readfirstlane(q.slot);  // uniform, as in gemm1_kernel
        if (t < 0) break;
        const int e = __builtin_amdgcn_readfirstlane(q.task.x), row0 = __builtin_amdgcn_readfirstlane(q.task.y);
        const int nsub = __builtin_amdgcn_readfirstlane(q.task.z), cb = __builtin_amdgcn_readfirstlane(q.task.w);
        Sched sch{a.ctl, kCtlQueue2, a.tasks, a.row_src, a.row_w, &q, xcd};
#define MOE_G2(NS)                                                                                                 \
    gemm_task<MODE, false, NS, RING>(a.h, a.h_scale, a.row_src, 1, a.w2, a.w2_scale, a.zero, e, row0, cb, a.d_e, a.d_h, \
                                     a.packed != 0, smem, nullptr, &a, sch, q.rows[par], q.roww[par], par)
        // 128-row tasks outside MXFP8 mode (gemm2_row_blocks)
        if constexpr (MODE != MOE_MODE_MXFP8) {
            switch (nsub) {
                case 1: MOE_G2(1); break;
                case 2: MOE_G2(2); break;
                case 3: MOE_G2(3); break;
                case 4: MOE_G2(4); break;
                case 5: MOE_G2(5); break;
                case 6: MOE_G2(6); break;
                case 7: MOE_G2(7); break;
                default: MOE_G2(8); break;
            }
        } else {
            switch (nsub) {
                case 1: MOE_G2(1); break;
                case 2: MOE_G2(2); break;
                case 3: MOE_G2(3); break;
                default: MOE_G2(4); break;
            }
        }
#undef MOE_G2
    }
}

// ---------------------------------------------- FP8 / MXFP8 GEMM-1 (8 waves)
// Block-scaled FP8 GEMM-1 with SwiGLU and the per-row-per-128 requantisation
// of h, for tasks of up to 16 group blocks (256 rows) by 128 output columns
// (256 weight rows: 128 gate, 128 up).  Eight waves, two per SIMD: wave
// (wm, wn) = (w / 4, w % 4) owns output columns [32 wn, 32 wn + 32) (two
// 16-column fragments, gate and up) of the task's row blocks wm, wm + 2,
// wm + 4, ...  Each K block of every row block is one 16x16x128 MFMA per
// fragment from zero, promoted into the fp32 accumulator with (row scale of
// x) * (block scale of W1) -- one FMA per accumulator element.  With two
// waves per SIMD the promotion of one wave runs while the other's MFMAs do,
// so the body needs no software pipelining of its own.
//
// A stage (one K block) holds the 256 weight rows (32 KB), the task's token
// rows (2 KB per group block) and their row scales; 256-row tasks bring in 64
// KB per 16.8 MFLOP, where 128-row ones bring 48 KB per 8.4: the per-CU rate
// of direct-to-LDS loads (about 66-74 GB/s with eight issuing waves, measured)
// bounds this kernel before HBM or the MFMAs do.  The four waves of wave row
// 0, one per SIMD, issue the stage loads: a wave that issues direct-to-LDS
// loads waits while the CU's address unit works through them (about 1 KB
// per 16 cycles), and on each SIMD the other wave's MFMAs run meanwhile.  The
// last wave is the scheduler (as in gemm_task) and computes.
//
// The MXFP8 form (gemm1_mxfp8_kernel, the same task code with MX set) keeps
// the geometry: its stages also carry the E8M0 scale words of the 256 weight
// rows, the scaled MFMA accumulates in place (no promotion), and h is
// requantised per row per 32 columns, one MX block per wave.
struct G1F8 {
    static constexpr int kWaves = kGemm1Fp8Waves;
    static constexpr int kSched = kWaves - 1;
    static constexpr int kLoaders = 4;  // waves 0..3: one per SIMD
    static constexpr int kStoreThreads = 64 * kSched;
    static constexpr int kMaxRows = 16 * kMaxRowBlocksFp8G1;
    static_assert((kMaxRows + 63) / 64 <= kLoaders, "one row-scale load of 64 rows per loading wave");
    static constexpr int kBN = 128;
    static constexpr int kBRows = 2 * kBN;
    static constexpr int kBAll = kBRows / 8;                         // B loads per stage
    static constexpr int kBMax = (kBAll + kLoaders - 1) / kLoaders;  // per loading wave, at most
    static constexpr int kAMax = (2 * kMaxRowBlocksFp8G1 + kLoaders - 1) / kLoaders;
    static constexpr int kStageB = kBRows * kRowBytes;
    // row scales of up to 256 rows (4 B each), then the gate and up block scales
    static constexpr int kScaleBlk = 4 * kMaxRows;
    static constexpr int kStageS = kScaleBlk + 16;
    // MXFP8: the K block's four E8M0 bytes of each A row (one 4-byte word per
    // row, in the positions of the FP8 row scales), then of each B row (row r
    // at word kScaleBlk / 4 + r)
    static constexpr int kStageSMx = kScaleBlk + 4 * kBRows;
    static constexpr int stage_bytes(int nsub, bool mx = false) {
        return kStageB + 16 * nsub * kRowBytes + (mx ? kStageSMx : kStageS);
    }
    static constexpr int kRing = 160 * 1024 - 5 * 1024;
    static constexpr int stages(int nsub, bool mx = false) {
        return kRing / stage_bytes(nsub, mx) < 8 ? kRing / stage_bytes(nsub, mx) : 8;
    }
    static constexpr int kEpiRow = kBN;  // one e4m3 byte per column
};
static_assert(G1F8::kEpiRow * G1F8::kMaxRows + 4 * G1F8::kMaxRows * 4 <= G1F8::kRing,
              "epilogue staging must fit in the ring");
static_assert(G1F8::stages(kMaxRowBlocksFp8G1) >= 2 && G1F8::stages(kMaxRowBlocksFp8G1, true) >= 2,
              "ring too small");
static_assert(G1F8::stage_bytes(1) % 16 == 0 && G1F8::stage_bytes(1, true) % 16 == 0, "stages 16-byte aligned");

// Row blocks of the task that wave row wm computes: wm, wm + 2, ...
template <int NSUB, int WM>
struct G1F8Rows {
    static constexpr int n = WM == 0 ? (NSUB + 1) / 2 : NSUB / 2;
};

// One K block of the FP8 GEMM-1 for a wave owning NW row blocks
// (2 i + wm, i < NW), with the weight fragment as the MFMA's first operand:
// lane (lr, lg) of a 16x16 result holds token row lr of the row block and
// weight columns 4 lg .. 4 lg + 3 of the fragment, so each lane promotes
// with one row scale per row block (times the K block's gate or up block
// scale).  The row scales of the wave's row blocks sit at stage positions
// 16 lr + 8 wm + i (the loads place them so): two 16-byte reads per K block.
// The A fragment of block i + 1 is read while block i's MFMAs run; the
// other wave of the SIMD issues its MFMAs while this one promotes.
template <int NW, int NA>
__device__ __forceinline__ void g1f8_kblock(const unsigned char* st, int nsub_rows_bytes, int wm, int wn, int lr,
                                            int lg, int swz, v4f (&acc)[NA][2][2]) {
    if constexpr (NW > 0) {
        const unsigned char* sb = st;
        const unsigned char* sa = st + G1F8::kStageB;
        const float* sc = reinterpret_cast<const float*>(st + G1F8::kStageB + nsub_rows_bytes);
        const float swg = sc[G1F8::kScaleBlk / 4], swu = sc[G1F8::kScaleBlk / 4 + 1];
        const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
        v8i Bf[2][2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const int brow = 16 * (2 * wn + f) + lr;
            Bf[f][0] = lds_frag32(sb + brow * kRowBytes, lg, swz);
            Bf[f][1] = lds_frag32(sb + (G1F8::kBN + brow) * kRowBytes, lg, swz);
        }
        const float4 s0 = *reinterpret_cast<const float4*>(sc + 16 * lr + 8 * wm);
        const float4 s1 = *reinterpret_cast<const float4*>(sc + 16 * lr + 8 * wm + 4);
        const float sxr[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        v8i A = lds_frag32(sa + (16 * wm + lr) * kRowBytes, lg, swz);
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            v4f t[2][2];
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int g = 0; g < 2; ++g) t[f][g] = mfma_fp8(Bf[f][g], A, zero4);
            v8i An = A;
            if (i + 1 < NW) An = lds_frag32(sa + (16 * (2 * (i + 1) + wm) + lr) * kRowBytes, lg, swz);
            __builtin_amdgcn_sched_barrier(0);
            const float pg = sxr[i] * swg, pu = sxr[i] * swu;
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[i][f][0][j] += t[f][0][j] * pg;
                    acc[i][f][1][j] += t[f][1][j] * pu;
                }
            __builtin_amdgcn_sched_barrier(0);
            A = An;
        }
    }
}

// The same K block in MXFP8: the MFMA applies the E8M0 scales and
// accumulates straight into acc (no promotion).  Lane (lr, lg) supplies the
// scale byte of its fragment row for K values [32 lg, 32 lg + 32): byte lg of
// that row's 4-byte word.  With the weight fragment as the first operand, its
// scale is the first scale operand and the token row's the second.
template <int NW, int NA>
__device__ __forceinline__ void g1mx_kblock(const unsigned char* st, int nsub_rows_bytes, int wm, int wn, int lr,
                                            int lg, int swz, v4f (&acc)[NA][2][2]) {
    if constexpr (NW > 0) {
        const unsigned char* sb = st;
        const unsigned char* sa = st + G1F8::kStageB;
        const unsigned* sc = reinterpret_cast<const unsigned*>(st + G1F8::kStageB + nsub_rows_bytes);
        const unsigned* scb = sc + G1F8::kScaleBlk / 4;
        const unsigned sh = 8u * (unsigned)lg;
        v8i Bf[2][2];
        int sbw[2][2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const int brow = 16 * (2 * wn + f) + lr;
            Bf[f][0] = lds_frag32(sb + brow * kRowBytes, lg, swz);
            Bf[f][1] = lds_frag32(sb + (G1F8::kBN + brow) * kRowBytes, lg, swz);
            sbw[f][0] = (int)((scb[brow] >> sh) & 0xffu);
            sbw[f][1] = (int)((scb[G1F8::kBN + brow] >> sh) & 0xffu);
        }
        const uint4 s0 = *reinterpret_cast<const uint4*>(sc + 16 * lr + 8 * wm);
        const uint4 s1 = *reinterpret_cast<const uint4*>(sc + 16 * lr + 8 * wm + 4);
        const unsigned sxr[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        v8i A = lds_frag32(sa + (16 * wm + lr) * kRowBytes, lg, swz);
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int sa_i = (int)((sxr[i] >> sh) & 0xffu);
            v8i An = A;
            if (i + 1 < NW) An = lds_frag32(sa + (16 * (2 * (i + 1) + wm) + lr) * kRowBytes, lg, swz);
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int gu = 0; gu < 2; ++gu) acc[i][f][gu] = mfma_mx(Bf[f][gu], A, acc[i][f][gu], sbw[f][gu], sa_i);
            A = An;
        }
    }
}

// MX: MXFP8 operands (E8M0 scales per 32 values of K, applied by the MFMA,
// and the intermediate requantised per row per 32 columns); otherwise FP8
// with 128x128 block scales promoted in registers.
template <int NSUB, bool MX>
__device__ __forceinline__ void g1f8_task(const Gemm1Args& g, int e, int row0, int cb, unsigned char* smem,
                                          SchedT<kRowsLdsFp8G1>& sch, const int* rows, int par) {
    using C = G1F8;
    constexpr int S = C::stages(NSUB, MX);
    constexpr int kStage = C::stage_bytes(NSUB, MX);
    constexpr int kStageA = 16 * NSUB * kRowBytes;
    constexpr int kAInstr = 2 * NSUB;  // A loads per stage: 8 rows each
    constexpr int kRows = 16 * NSUB;
    const int K = g.d_h, N_out = g.d_e;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = w >> 2, wn = w & 3;
    const int lr = lane & 15, lg = lane >> 4;
    const int nk = K / 128;
    const unsigned smem_lds = lds_offset(smem);
    const int64_t ld_bytes = K;  // bytes per operand row
    // row scales of x: fp32 per row per 128 (FP8) or four E8M0 bytes per row
    // per 128 (MXFP8): the same 4 bytes per row and K block, at the same offsets
    const void* a_scale = g.x_scale;
    const bool loader = w < C::kLoaders;
    // vector-memory loads per stage of this wave: B instructions w, w+4, ...,
    // A instructions the same way, row-scale chunk c by wave c, and the weight
    // scales: FP8 the two block scales by wave 1, MXFP8 the scale words of
    // B rows 64 w .. 64 w + 63 by each loading wave
    const int n_b = loader ? (C::kBAll - 1 - w) / C::kLoaders + 1 : 0;
    const int n_a = loader && w < kAInstr ? (kAInstr - 1 - w) / C::kLoaders + 1 : 0;
    const int my_chunk = w < C::kLoaders ? w : -1;  // row-scale chunk of this wave, or -1
    const bool s_rows = my_chunk >= 0;  // all four chunks: the positions are permuted
    const int n_s = (s_rows ? 1 : 0) + (MX ? (loader ? 1 : 0) : (w == 1 ? 1 : 0));
    const int loads_per_stage = n_b + n_a + n_s;

    // Addresses: uniform bases (the task's weight tile or expert, x, the
    // scale arrays) plus 32-bit per-lane offsets, so each load costs one VGPR
    // (the host sends tensors whose offsets could pass 2^31 to the 4-wave
    // kernel).  Padding rows read token row 0 (their results are never used:
    // rows are independent in every step, and GEMM-2 stores no padding row).
    const unsigned char* wbase;
    unsigned b_step;
    if (g.packed) {
        const int64_t tile = (int64_t)e * (N_out / C::kBN) + cb;
        wbase = static_cast<const unsigned char*>(g.w1) + tile * nk * C::kStageB;
        b_step = C::kStageB;
    } else {
        wbase = static_cast<const unsigned char*>(g.w1) + (int64_t)e * 2 * N_out * ld_bytes;
        b_step = kRowBytes;
    }
    // B instruction b loads tile rows 8b .. 8b+7: a uniform part (b_row(b),
    // scalar arithmetic) plus one per-lane offset shared by every b, since
    // the 8 rows of an instruction sit on one side of the gate/up split and
    // the swizzle depends only on the row mod 8
    const unsigned b_lane = g.packed ? (unsigned)(lane * 16)
                                     : (unsigned)(lane >> 3) * (unsigned)ld_bytes +
                                           (unsigned)((((lane & 7) ^ ((lane >> 3) & 7))) * 16);
    auto b_row = [&](int b) -> int64_t {
        if (g.packed) return (int64_t)b * 1024;
        const int r = 8 * b;
        const int wrow = r < C::kBN ? cb * C::kBN + r : N_out + cb * C::kBN + (r - C::kBN);
        return (int64_t)wrow * ld_bytes;
    };
    const unsigned char* xbase = static_cast<const unsigned char*>(g.x);
    unsigned aoff[C::kAMax];
#pragma unroll
    for (int j = 0; j < C::kAMax; ++j) {
        const int ai = w + C::kLoaders * j;
        const int r = 8 * ai + (lane >> 3);
        const int c = (lane & 7) ^ (r & 7);
        aoff[j] = 0;
        if (loader && ai < kAInstr) {
            const int p = rows[r];
            aoff[j] = (unsigned)(p >= 0 ? p / g.k : 0) * (unsigned)ld_bytes + (unsigned)(c * 16);
        }
    }
    // row scales: stage position p = 64 * my_chunk + lane holds the scale of
    // tile row 16 (2 (p & 7) + ((p >> 3) & 1)) + (p >> 4), which is where
    // g1f8_kblock reads it (position 16 lr + 8 wm + i for row block 2 i + wm);
    // row 0's past the task's rows and on padding rows.  Or in wave 1 lanes
    // 0 and 1 the gate and up block scales of W1; byte offsets
    const int kq = K / kQ;
    unsigned soff = 0;
    if (s_rows) {
        const int pos = 64 * my_chunk + lane;
        const int srow = 16 * (2 * (pos & 7) + ((pos >> 3) & 1)) + (pos >> 4);
        const int p = srow < kRows ? rows[srow] : -1;
        soff = (unsigned)(p >= 0 ? p / g.k : 0) * (unsigned)(4 * kq);
    }
    unsigned bsoff = 0;
    const unsigned char* w_scale = static_cast<const unsigned char*>(g.w1_scale);
    if constexpr (MX) {
        // W1 scale bytes [E][2 d_e][d_h/32]: the expert's base, and for lane
        // l of loading wave w tile row r = 64 w + l (gate rows cb*128 + r,
        // then up rows d_e + cb*128 + r - 128)
        w_scale += (int64_t)e * 2 * N_out * (K / 32);
        if (loader) {
            const int r = 64 * w + lane;
            const int wrow = r < C::kBN ? cb * C::kBN + r : N_out + cb * C::kBN + (r - C::kBN);
            bsoff = (unsigned)wrow * (unsigned)(K / 32);
        }
    } else if (w == 1 && lane < 2) {
        // W1 scales [E][2 d_e/128][d_h/128]: gate block row cb, up block row d_e/128 + cb
        const int nrb = 2 * N_out / kQ;
        const int brow = lane == 0 ? cb : N_out / kQ + cb;
        bsoff = (unsigned)((e * nrb + brow) * kq) * 4u;
    }

    // routing weight of each tile row (column block 0 only; waves 0..3 hold
    // rows 64 w + lane), stored by padded row for GEMM-2
    const int w_row = 64 * w + lane;
    const bool w_owner = cb == 0 && w < 4 && w_row < kRows;
    float ep_w = 0.f;
    if (w_owner) {
        const int p = rows[w_row];
        ep_w = p >= 0 ? g.topk_w[p] : 0.f;
    }

    auto issue = [&](int kc) {
        const unsigned st = smem_lds + (unsigned)((kc % S) * kStage);
        const unsigned koff = (unsigned)kc * kRowBytes;
        const unsigned kboff = (unsigned)kc * b_step;
        if (!loader) return;
#pragma unroll
        for (int j = 0; j < C::kBMax; ++j) {
            const int b = w + C::kLoaders * j;
            if (b < C::kBAll) g2l16s(wbase + b_row(b), b_lane + kboff, st + (unsigned)(b * 1024));
        }
#pragma unroll
        for (int j = 0; j < C::kAMax; ++j) {
            const int ai = w + C::kLoaders * j;
            if (ai < kAInstr) g2l16s(xbase, aoff[j] + koff, st + (unsigned)(C::kStageB + ai * 1024));
        }
        const unsigned ss = st + (unsigned)(C::kStageB + kStageA);
        if (s_rows) g2l4s(a_scale, soff + 4u * (unsigned)kc, ss + (unsigned)(256 * my_chunk));
        if constexpr (MX)
            g2l4s(w_scale, bsoff + 4u * (unsigned)kc, ss + (unsigned)(C::kScaleBlk + 256 * w));
        else if (w == 1 && lane < 2)  // lanes 0 and 1 only: the other lanes would land past the stage
            g2l4s(w_scale, bsoff + 4u * (unsigned)kc, ss + (unsigned)C::kScaleBlk);
    };

    const int swz = lr & 7;
    const int npro = nk < S - 1 ? nk : S - 1;
    for (int kc = 0; kc < npro; ++kc) issue(kc);
    const int claim_at = nk > kClaimLead ? nk - kClaimLead : 0;
    const int settle_at = nk > kClaimLead - 2 ? nk - (kClaimLead - 2) : 0;
    const int rows_at = nk > kClaimLead - 4 ? nk - (kClaimLead - 4) : 0;
    unsigned char* stage = smem;                                               // [kRows][kEpiRow]
    float* s_amax = reinterpret_cast<float*>(smem + C::kEpiRow * C::kMaxRows);  // [4 wn][kMaxRows]

    // The K loop and the epilogue of a wave row with NW row blocks.  The two
    // wave rows run their own copy (the branch is uniform per wave), so each
    // copy keeps its accumulators in fixed registers; both execute the same
    // sequence of workgroup barriers.
    auto body = [&](auto nw_c) {
        constexpr int NW = decltype(nw_c)::value;
        constexpr int NA = NW > 0 ? NW : 1;
        v4f acc[NA][2][2];
        const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NA; ++i)
#pragma unroll
            for (int f = 0; f < 2; ++f) acc[i][f][0] = acc[i][f][1] = zero4;
        for (int kc = 0; kc < nk; ++kc) {
            if (loader) {
                const int younger = (nk - 1 - kc) < (S - 2) ? (nk - 1 - kc) : (S - 2);
                wait_vm_le(younger * loads_per_stage);
            }
            lds_barrier();
            if (kc + S - 1 < nk) issue(kc + S - 1);
            if (w == C::kSched) {
                if (kc == claim_at && lane == 0) sch.claim();
                if (kc == settle_at) sch.settle(true);
                if (kc == rows_at) sch.load_rows(par ^ 1);
            }
            if constexpr (MX)
                g1mx_kblock<NW>(smem + (kc % S) * kStage, kStageA, wm, wn, lr, lg, swz, acc);
            else
                g1f8_kblock<NW>(smem + (kc % S) * kStage, kStageA, wm, wn, lr, lg, swz, acc);
        }
        __builtin_amdgcn_s_waitcnt(VmCnt<0>::imm);

        // ---- epilogue: SwiGLU, amax per row over the task's 128 columns
        // (FP8: four waves hold 32 columns each) or over each wave's 32
        // (MXFP8), requantisation, staging, stores
        lds_barrier();
        if (w_owner) g.row_w[row0 + w_row] = ep_w;
        float hv[NA][2][4];
        const bool clamped = g.act == MOE_ACT_SWIGLU_CLAMPED;
#pragma unroll
        for (int i = 0; i < NW; ++i)
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    hv[i][f][j] = clamped ? clamped_act(acc[i][f][0][j], acc[i][f][1][j])
                                          : silu_mul(acc[i][f][0][j], acc[i][f][1][j]);
        // Row block i of this lane: tile row 32 i + 16 wm + lr, columns
        // 32 wn + 16 f + 4 lg + j.  Every address below is one per-lane base
        // plus a compile-time offset, so the loops keep no per-row addresses
        // in registers.
        const int row_l = 16 * wm + lr;
        unsigned* stage_l = reinterpret_cast<unsigned*>(stage + row_l * C::kEpiRow + 32 * wn + 4 * lg);
        if constexpr (MX) {
            // per row per 32 columns: this wave's 32 columns of a row are one
            // MX block, spread over the row's four lane groups.  Shared
            // exponent floor(log2 amax) - 8 (the e4m3 maximum is 1.75 * 2^8),
            // stored biased by 127 and clamped to [0, 254], 127 for an
            // all-zero block; elements v * 2^-exponent saturated to +-448,
            // rounded to e4m3
            int hb[NA];
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                float m = 0.f;
#pragma unroll
                for (int f = 0; f < 2; ++f)
#pragma unroll
                    for (int j = 0; j < 4; ++j) m = fmaxf(m, fabsf(hv[i][f][j]));
                m = fmaxf(m, __shfl_xor(m, 16));
                m = fmaxf(m, __shfl_xor(m, 32));
                // frexp: m = f * 2^x with f in [0.5, 1), so floor(log2 m) = x - 1
                int b = m > 0.f ? __builtin_amdgcn_frexp_expf(m) - 1 - 8 + 127 : 127;
                b = b < 0 ? 0 : (b > 254 ? 254 : b);
                hb[i] = b;
#pragma unroll
                for (int f = 0; f < 2; ++f) {
                    float v[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        v[j] = fminf(fmaxf(__builtin_amdgcn_ldexpf(hv[i][f][j], 127 - b), -448.0f), 448.0f);
                    int word = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
                    word = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], word, true);
                    stage_l[(32 * i * C::kEpiRow + 16 * f) / 4] = (unsigned)word;
                }
            }
            // h_scale bytes [n_pad][d_e/32]: byte cb*4 + wn of each of the lane's rows
            if (lg == 0) {
                uint8_t* hs_l =
                    static_cast<uint8_t*>(g.h_scale) + (int64_t)(row0 + row_l) * (N_out / 32) + cb * 4 + wn;
#pragma unroll
                for (int i = 0; i < NW; ++i) hs_l[(int64_t)(32 * i) * (N_out / 32)] = (uint8_t)hb[i];
            }
        } else {
            float* amax_w = s_amax + wn * C::kMaxRows + row_l;
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                float m = 0.f;
#pragma unroll
                for (int f = 0; f < 2; ++f)
#pragma unroll
                    for (int j = 0; j < 4; ++j) m = fmaxf(m, fabsf(hv[i][f][j]));
                // the four lane groups hold the row's other columns of this wave
                m = fmaxf(m, __shfl_xor(m, 16));
                m = fmaxf(m, __shfl_xor(m, 32));
                if (lg == 0) amax_w[32 * i] = m;
            }
            lds_barrier();
            const int nq = N_out / kQ;
            float* hs_l = static_cast<float*>(g.h_scale) + (int64_t)(row0 + row_l) * nq + cb;
            const float* amax_r = s_amax + row_l;
            float sc_keep[NA];  // row scales, stored after the loop (no store waits inside it)
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                float am = amax_r[32 * i];
#pragma unroll
                for (int ww = 1; ww < 4; ++ww) am = fmaxf(am, amax_r[ww * C::kMaxRows + 32 * i]);
                // scale amax/448; values are multiplied by its reciprocal
                sc_keep[i] = am > 0.f ? am * (1.0f / 448.0f) : 1.0f;
                const float inv = am > 0.f ? 448.0f * __builtin_amdgcn_rcpf(am) : 1.0f;
#pragma unroll
                for (int f = 0; f < 2; ++f) {
                    // four e4m3 codes, columns 4 lg .. 4 lg + 3 in byte order
                    int word = __builtin_amdgcn_cvt_pk_fp8_f32(hv[i][f][0] * inv, hv[i][f][1] * inv, 0, false);
                    word = __builtin_amdgcn_cvt_pk_fp8_f32(hv[i][f][2] * inv, hv[i][f][3] * inv, word, true);
                    stage_l[(32 * i * C::kEpiRow + 16 * f) / 4] = (unsigned)word;
                }
            }
            if (wn == 0 && lg == 0)
#pragma unroll
                for (int i = 0; i < NW; ++i) hs_l[(int64_t)(32 * i) * nq] = sc_keep[i];
        }
        lds_barrier();
        // h[row0 + r][cb*128 ...]: 128 bytes per row
        constexpr int kChunks = C::kEpiRow / 16;
        unsigned char* h = static_cast<unsigned char*>(g.h);
        if (w != C::kSched)
            for (int i = threadIdx.x; i < kRows * kChunks; i += C::kStoreThreads) {
                const int r = i / kChunks, c = i - r * kChunks;
                *reinterpret_cast<v4i*>(h + (int64_t)(row0 + r) * N_out + (int64_t)cb * C::kEpiRow + c * 16) =
                    *reinterpret_cast<const v4i*>(stage + r * C::kEpiRow + c * 16);
            }
        if (w == C::kSched) sch.publish();
        lds_barrier();  // the ring and the staging area are refilled by the next task
    };
    if (wm == 0)
        body(std::integral_constant<int, G1F8Rows<NSUB, 0>::n>{});
    else
        body(std::integral_constant<int, G1F8Rows<NSUB, 1>::n>{});
}

// The persistent 8-wave GEMM-1: scheduler set-up, then tasks until the
// queues are empty.
template <bool MX>
__device__ __forceinline__ void gemm1_wide(const Gemm1Args& a, unsigned char* smem, QueueLdsT<kRowsLdsFp8G1>& q) {
    const int xcd = my_xcd();
    if (threadIdx.x <= kXcds) q.seg[threadIdx.x] = a.ctl[kCtlSeg1 + threadIdx.x];
    if (threadIdx.x == 0) q.mask = 0;
    lds_barrier();
    if (threadIdx.x >= 64 * G1F8::kSched) {
        SchedT<kRowsLdsFp8G1> sch{a.ctl, kCtlQueue1, a.tasks, a.row_src, nullptr, &q, xcd};
        sch.first();
        sch.load_rows(0);
        sch.publish();
    }
    lds_barrier();
    for (int par = 0;; par ^= 1) {
        // readfirstlane: the task is uniform, and the compiler must know it
        // (a task loop it takes as divergent may split a one-thread region
        // next to the back-edge off the loop)
        const int t = __builtin_amdgcn_readfirstlane(q.slot);
        if (t < 0) break;
        const int e = __builtin_amdgcn_readfirstlane(q.task.x), row0 = __builtin_amdgcn_readfirstlane(q.task.y);
        const int nsub = __builtin_amdgcn_readfirstlane(q.task.z), cb = __builtin_amdgcn_readfirstlane(q.task.w);
        SchedT<kRowsLdsFp8G1> sch{a.ctl, kCtlQueue1, a.tasks, a.row_src, nullptr, &q, xcd};
#define MOE_G1F8(NS) g1f8_task<NS, MX>(a, e, row0, cb, smem, sch, q.rows[par], par)
        switch (nsub) {
            case 1: MOE_G1F8(1); break;
            case 2: MOE_G1F8(2); break;
            case 3: MOE_G1F8(3); break;
            case 4: MOE_G1F8(4); break;
            case 5: MOE_G1F8(5); break;
            case 6: MOE_G1F8(6); break;
            case 7: MOE_G1F8(7); break;
            case 8: MOE_G1F8(8); break;
            case 9: MOE_G1F8(9); break;
            case 10: MOE_G1F8(10); break;
            case 11: MOE_G1F8(11); break;
            case 12: MOE_G1F8(12); break;
            case 13: MOE_G1F8(13); break;
            case 14: MOE_G1F8(14); break;
            case 15: MOE_G1F8(15); break;
            default: MOE_G1F8(16); break;
        }
#undef MOE_G1F8
    }
}

__global__ __launch_bounds__(kGemm1Fp8Threads) void gemm1_fp8_kernel(Gemm1Args a) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[G1F8::kRing];
    __shared__ QueueLdsT<kRowsLdsFp8G1> q;
    gemm1_wide<false>(a, smem, q);
}

__global__ __launch_bounds__(kGemm1Fp8Threads) void gemm1_mxfp8_kernel(Gemm1Args a) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[G1F8::kRing];
    __shared__ QueueLdsT<kRowsLdsFp8G1> q;
    gemm1_wide<true>(a, smem, q);
}

// ---------------------------------------------- FP8 / MXFP8 GEMM-2 (8 waves)
// Block-scaled FP8 GEMM-2 for tasks of up to 16 group blocks (256 rows of h)
// by 256 output columns, on the geometry of the 8-wave GEMM-1: a stage holds
// 256 rows of W2 (32 KB), the task's h rows and their row scales; wave
// (wm, wn) owns output columns [64 wn, 64 wn + 64) (four 16-column fragments)
// of row blocks wm, wm + 2, ...; the weight fragment is the MFMA's first
// operand, so each lane promotes with one row scale of h per row block times
// the K block's W2 block scale (the 256 columns span two 128x128 scale
// blocks: waves 0, 1, 4, 5 take the first, the others the second).  The
// stage loads come from the four waves of wave row 0, one per SIMD.  Output:
// y[p] = bf16(acc * routing weight of the row), for the task's rows with a
// source assignment p (padding rows store nothing), stored from registers.
// The MXFP8 form (gemm2_mxfp8_kernel) carries the scale words of the 256 W2
// rows in each stage and accumulates through the scaled MFMA.
namespace g2w {
constexpr int kBRows = 256;          // output columns per task = W2 rows per stage
constexpr int kOutRow = 2 * kBRows;  // bytes of one task's part of an output row (bf16)
}  // namespace g2w

template <int NW, int NA>
__device__ __forceinline__ void g2f8_kblock(const unsigned char* st, int nsub_rows_bytes, int wm, int wn, int lr,
                                            int lg, int swz, v4f (&acc)[NA][4]) {
    if constexpr (NW > 0) {
        const unsigned char* sb = st;
        const unsigned char* sa = st + G1F8::kStageB;
        const float* sc = reinterpret_cast<const float*>(st + G1F8::kStageB + nsub_rows_bytes);
        const float sw = sc[G1F8::kScaleBlk / 4 + (wn >> 1)];
        const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
        v8i Bf[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) Bf[f] = lds_frag32(sb + (64 * wn + 16 * f + lr) * kRowBytes, lg, swz);
        const float4 s0 = *reinterpret_cast<const float4*>(sc + 16 * lr + 8 * wm);
        const float4 s1 = *reinterpret_cast<const float4*>(sc + 16 * lr + 8 * wm + 4);
        const float sxr[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        v8i A = lds_frag32(sa + (16 * wm + lr) * kRowBytes, lg, swz);
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            v4f t[4];
#pragma unroll
            for (int f = 0; f < 4; ++f) t[f] = mfma_fp8(Bf[f], A, zero4);
            v8i An = A;
            if (i + 1 < NW) An = lds_frag32(sa + (16 * (2 * (i + 1) + wm) + lr) * kRowBytes, lg, swz);
            __builtin_amdgcn_sched_barrier(0);
            const float pw = sxr[i] * sw;
#pragma unroll
            for (int f = 0; f < 4; ++f)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][f][j] += t[f][j] * pw;
            __builtin_amdgcn_sched_barrier(0);
            A = An;
        }
    }
}

// MXFP8 form of the K block: scales applied by the MFMA (as in g1mx_kblock);
// the weight fragments' scale words are those of W2 rows 64 wn + 16 f + lr.
template <int NW, int NA>
__device__ __forceinline__ void g2mx_kblock(const unsigned char* st, int nsub_rows_bytes, int wm, int wn, int lr,
                                            int lg, int swz, v4f (&acc)[NA][4]) {
    if constexpr (NW > 0) {
        const unsigned char* sb = st;
        const unsigned char* sa = st + G1F8::kStageB;
        const unsigned* sc = reinterpret_cast<const unsigned*>(st + G1F8::kStageB + nsub_rows_bytes);
        const unsigned* scb = sc + G1F8::kScaleBlk / 4;
        const unsigned sh = 8u * (unsigned)lg;
        v8i Bf[4];
        int sbw[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int brow = 64 * wn + 16 * f + lr;
            Bf[f] = lds_frag32(sb + brow * kRowBytes, lg, swz);
            sbw[f] = (int)((scb[brow] >> sh) & 0xffu);
        }
        const uint4 s0 = *reinterpret_cast<const uint4*>(sc + 16 * lr + 8 * wm);
        const uint4 s1 = *reinterpret_cast<const uint4*>(sc + 16 * lr + 8 * wm + 4);
        const unsigned sxr[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        v8i A = lds_frag32(sa + (16 * wm + lr) * kRowBytes, lg, swz);
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int sa_i = (int)((sxr[i] >> sh) & 0xffu);
            v8i An = A;
            if (i + 1 < NW) An = lds_frag32(sa + (16 * (2 * (i + 1) + wm) + lr) * kRowBytes, lg, swz);
#pragma unroll
            for (int f = 0; f < 4; ++f) acc[i][f] = mfma_mx(Bf[f], A, acc[i][f], sbw[f], sa_i);
            A = An;
        }
    }
}

// MX: MXFP8 operands (h and W2 with E8M0 scales per 32 values of K);
// otherwise FP8 with per-row-per-128 h scales and 128x128 W2 block scales.
template <int NSUB, bool MX>
__device__ __forceinline__ void g2f8_task(const Gemm2Args& g, int e, int row0, int cb, unsigned char* smem,
                                          SchedT<kRowsLdsFp8G1>& sch, const int* rows, const float* roww, int par) {
    using C = G1F8;
    constexpr int S = C::stages(NSUB, MX);
    constexpr int kStage = C::stage_bytes(NSUB, MX);
    constexpr int kStageA = 16 * NSUB * kRowBytes;
    constexpr int kAInstr = 2 * NSUB;  // A loads per stage: 8 rows each
    constexpr int kRows = 16 * NSUB;
    constexpr int kBAll = g2w::kBRows / 8;  // B loads per stage
    constexpr int kLoaders = 4;             // waves 0..3, one per SIMD
    constexpr int kBMax = (kBAll + kLoaders - 1) / kLoaders;
    constexpr int kAMax = (2 * kMaxRowBlocksFp8G1 + kLoaders - 1) / kLoaders;
    const int K = g.d_e, N_out = g.d_h;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = w >> 2, wn = w & 3;
    const int lr = lane & 15, lg = lane >> 4;
    const int nk = K / 128;
    const unsigned smem_lds = lds_offset(smem);
    const int64_t ld_bytes = K;  // bytes per operand row (h and W2 rows)
    const bool loader = w < kLoaders;
    // loads per stage of a loading wave: B and A instructions w, w+4, ...,
    // one 64-position chunk of row scales, and the weight scales: FP8 the two
    // block scales in wave 1, MXFP8 the scale words of W2 rows 64 w .. 64 w + 63
    const int n_b = loader ? (kBAll - 1 - w) / kLoaders + 1 : 0;
    const int n_a = loader && w < kAInstr ? (kAInstr - 1 - w) / kLoaders + 1 : 0;
    const int n_s = (loader ? 1 : 0) + (MX ? (loader ? 1 : 0) : (w == 1 ? 1 : 0));
    const int loads_per_stage = n_b + n_a + n_s;

    // Addresses: a uniform part per instruction (scalar arithmetic) plus one
    // per-lane offset shared by all instructions of an operand: the 8 rows of
    // an instruction are consecutive and the swizzle depends on the row mod 8
    // only.  h rows are the task's own padded rows (GEMM-1 wrote zeros into
    // the padding rows, with scale 1).
    const unsigned lane_rm = (unsigned)(lane >> 3) * (unsigned)ld_bytes +
                             (unsigned)((((lane & 7) ^ ((lane >> 3) & 7))) * 16);
    const unsigned b_lane = g.packed ? (unsigned)(lane * 16) : lane_rm;
    const unsigned char* w2 = static_cast<const unsigned char*>(g.w2);
    const int64_t tiles_per_expert = N_out / 128;  // packed W2: 128-row tiles, nk stages of 16 KB each
    auto b_row = [&](int b) -> int64_t {
        if (g.packed) {
            const int64_t tile = (int64_t)e * tiles_per_expert + 2 * cb + (b >> 4);
            return tile * nk * 16384 + (int64_t)(b & 15) * 1024;
        }
        return ((int64_t)e * N_out + (int64_t)cb * g2w::kBRows + 8 * b) * ld_bytes;
    };
    const unsigned b_step = g.packed ? 16384u : (unsigned)kRowBytes;
    const unsigned char* hbase = static_cast<const unsigned char*>(g.h) + (int64_t)row0 * ld_bytes;
    // h row scales: fp32 per row per 128 (FP8) or four E8M0 bytes per row per
    // 128 (MXFP8), the same 4 bytes per row and K block at the same offsets
    const void* h_scale = g.h_scale;
    const unsigned char* w_scale = static_cast<const unsigned char*>(g.w2_scale);
    // row scales: stage position p = 64 w + lane holds the scale of tile row
    // 16 (2 (p & 7) + ((p >> 3) & 1)) + (p >> 4), where g2f8_kblock reads it
    // (row 0's past the task's rows); wave 1 lanes 0 and 1: the two W2 block
    // scales of the task's columns; byte offsets
    const int kq = K / kQ;
    unsigned soff = 0;
    if (loader) {
        const int pos = 64 * w + lane;
        const int srow = 16 * (2 * (pos & 7) + ((pos >> 3) & 1)) + (pos >> 4);
        soff = (unsigned)(row0 + (srow < kRows ? srow : 0)) * (unsigned)(4 * kq);
    }
    unsigned bsoff = 0;
    if constexpr (MX) {
        // W2 scale bytes [E][d_h][d_e/32]: the expert's base, and for lane l
        // of loading wave w the task's W2 row 64 w + l
        w_scale += (int64_t)e * N_out * (K / 32);
        if (loader) bsoff = (unsigned)(cb * g2w::kBRows + 64 * w + lane) * (unsigned)(K / 32);
    } else if (w == 1 && lane < 2) {
        bsoff = (unsigned)(((int64_t)e * (N_out / kQ) + 2 * cb + lane) * kq) * 4u;
    }

    auto issue = [&](int kc) {
        const unsigned st = smem_lds + (unsigned)((kc % S) * kStage);
        const unsigned koff = (unsigned)kc * kRowBytes;
        const unsigned kboff = (unsigned)kc * b_step;
        if (!loader) return;
#pragma unroll
        for (int j = 0; j < kBMax; ++j) {
            const int b = w + kLoaders * j;
            if (b < kBAll) g2l16s(w2 + b_row(b), b_lane + kboff, st + (unsigned)(b * 1024));
        }
#pragma unroll
        for (int j = 0; j < kAMax; ++j) {
            const int ai = w + kLoaders * j;
            if (ai < kAInstr)
                g2l16s(hbase + (int64_t)(8 * ai) * ld_bytes, lane_rm + koff, st + (unsigned)(C::kStageB + ai * 1024));
        }
        const unsigned ss = st + (unsigned)(C::kStageB + kStageA);
        g2l4s(h_scale, soff + 4u * (unsigned)kc, ss + (unsigned)(256 * w));
        if constexpr (MX)
            g2l4s(w_scale, bsoff + 4u * (unsigned)kc, ss + (unsigned)(C::kScaleBlk + 256 * w));
        else if (w == 1 && lane < 2)  // lanes 0 and 1 only: the other lanes would land past the stage
            g2l4s(w_scale, bsoff + 4u * (unsigned)kc, ss + (unsigned)C::kScaleBlk);
    };

    const int swz = lr & 7;
    const int npro = nk < S - 1 ? nk : S - 1;
    for (int kc = 0; kc < npro; ++kc) issue(kc);
    const int claim_at = nk > kClaimLead ? nk - kClaimLead : 0;
    const int settle_at = nk > kClaimLead - 2 ? nk - (kClaimLead - 2) : 0;
    const int rows_at = nk > kClaimLead - 4 ? nk - (kClaimLead - 4) : 0;

    auto body = [&](auto nw_c) {
        constexpr int NW = decltype(nw_c)::value;
        constexpr int NA = NW > 0 ? NW : 1;
        v4f acc[NA][4];
        const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NA; ++i)
#pragma unroll
            for (int f = 0; f < 4; ++f) acc[i][f] = zero4;
        for (int kc = 0; kc < nk; ++kc) {
            if (loader) {
                const int younger = (nk - 1 - kc) < (S - 2) ? (nk - 1 - kc) : (S - 2);
                wait_vm_le(younger * loads_per_stage);
            }
            lds_barrier();
            if (kc + S - 1 < nk) issue(kc + S - 1);
            if (w == C::kSched) {
                if (kc == claim_at && lane == 0) sch.claim();
                if (kc == settle_at) sch.settle(true);
                if (kc == rows_at) sch.load_rows(par ^ 1);
            }
            if constexpr (MX)
                g2mx_kblock<NW>(smem + (kc % S) * kStage, kStageA, wm, wn, lr, lg, swz, acc);
            else
                g2f8_kblock<NW>(smem + (kc % S) * kStage, kStageA, wm, wn, lr, lg, swz, acc);
        }
        __builtin_amdgcn_s_waitcnt(VmCnt<0>::imm);

        // ---- epilogue: routing weight, bf16, stored from registers.  Row
        // block i of this lane: tile row 32 i + 16 wm + lr, columns
        // 64 wn + 16 f + 4 lg + j (four consecutive bf16 = 8 bytes); no
        // staging pass, no barrier before the stores.  Padding rows (no
        // source assignment) store nothing.
        // Fragments 2q and 2q + 1 (32 columns) go out as one 16-byte store
        // per lane: lane groups lg and lg ^ 1 trade halves (one lane shuffle
        // per word), so an even group holds 8 consecutive columns of fragment
        // 2q, an odd group 8 of fragment 2q + 1, and the four groups of a row
        // cover its 32 columns (64 bytes) in one instruction: half the store
        // requests of 8-byte pieces.
        const int row_l = 16 * wm + lr;
        const bool odd = lg & 1;
        const int col0 = 64 * wn + (odd ? 16 + 4 * (lg - 1) : 4 * lg);
        unsigned char* ycol = static_cast<unsigned char*>(g.y) + (int64_t)cb * g2w::kOutRow + 2 * col0;
        const int64_t yrow_bytes = (int64_t)N_out * 2;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int p = rows[row_l + 32 * i];
            const float wt = roww[row_l + 32 * i];
            uint4 v[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const unsigned a0 = pk_bf16(acc[i][2 * q][0] * wt, acc[i][2 * q][1] * wt);
                const unsigned a1 = pk_bf16(acc[i][2 * q][2] * wt, acc[i][2 * q][3] * wt);
                const unsigned b0 = pk_bf16(acc[i][2 * q + 1][0] * wt, acc[i][2 * q + 1][1] * wt);
                const unsigned b1 = pk_bf16(acc[i][2 * q + 1][2] * wt, acc[i][2 * q + 1][3] * wt);
                // an even group sends its fragment 2q + 1 words, an odd one its 2q words
                const unsigned r0 = __shfl_xor(odd ? a0 : b0, 16);
                const unsigned r1 = __shfl_xor(odd ? a1 : b1, 16);
                v[q] = odd ? make_uint4(r0, r1, b0, b1) : make_uint4(a0, a1, r0, r1);
            }
            // the partner group holds the same row, so both take this branch alike
            if (p >= 0) {
                unsigned char* dst = ycol + (int64_t)p * yrow_bytes;
                *reinterpret_cast<uint4*>(dst) = v[0];
                *reinterpret_cast<uint4*>(dst + 64) = v[1];
            }
        }
        if (w == C::kSched) sch.publish();
        lds_barrier();  // the ring is refilled by the next task
    };
    if (wm == 0)
        body(std::integral_constant<int, G1F8Rows<NSUB, 0>::n>{});
    else
        body(std::integral_constant<int, G1F8Rows<NSUB, 1>::n>{});
}

template <bool MX>
__device__ __forceinline__ void gemm2_wide(const Gemm2Args& a, unsigned char* smem, QueueLdsT<kRowsLdsFp8G1>& q) {
    const int xcd = my_xcd();
    if (threadIdx.x <= kXcds) q.seg[threadIdx.x] = a.ctl[kCtlSeg2 + threadIdx.x];
    if (threadIdx.x == 0) q.mask = 0;
    lds_barrier();
    if (threadIdx.x >= 64 * G1F8::kSched) {
        SchedT<kRowsLdsFp8G1> sch{a.ctl, kCtlQueue2, a.tasks, a.row_src, a.row_w, &q, xcd};
        sch.first();
        sch.load_rows(0);
        sch.publish();
    }
    lds_barrier();
    for (int par = 0;; par ^= 1) {
        const int t = __builtin_amdgcn_readfirstlane(q.slot);  // uniform, as in gemm1_wide
        if (t < 0) break;
        const int e = __builtin_amdgcn_readfirstlane(q.task.x), row0 = __builtin_amdgcn_readfirstlane(q.task.y);
        const int nsub = __builtin_amdgcn_readfirstlane(q.task.z), cb = __builtin_amdgcn_readfirstlane(q.task.w);
        SchedT<kRowsLdsFp8G1> sch{a.ctl, kCtlQueue2, a.tasks, a.row_src, a.row_w, &q, xcd};
#define MOE_G2F8(NS) g2f8_task<NS, MX>(a, e, row0, cb, smem, sch, q.rows[par], q.roww[par], par)
        switch (nsub) {
            case 1: MOE_G2F8(1); break;
            case 2: MOE_G2F8(2); break;
            case 3: MOE_G2F8(3); break;
            case 4: MOE_G2F8(4); break;
            case 5: MOE_G2F8(5); break;
            case 6: MOE_G2F8(6); break;
            case 7: MOE_G2F8(7); break;
            case 8: MOE_G2F8(8); break;
            case 9: MOE_G2F8(9); break;
            case 10: MOE_G2F8(10); break;
            case 11: MOE_G2F8(11); break;
            case 12: MOE_G2F8(12); break;
            case 13: MOE_G2F8(13); break;
            case 14: MOE_G2F8(14); break;
            case 15: MOE_G2F8(15); break;
            default: MOE_G2F8(16); break;
        }
#undef MOE_G2F8
    }
}

__global__ __launch_bounds__(kGemm1Fp8Threads) void gemm2_fp8_kernel(Gemm2Args a) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[G1F8::kRing];
    __shared__ QueueLdsT<kRowsLdsFp8G1> q;
    gemm2_wide<false>(a, smem, q);
}

__global__ __launch_bounds__(kGemm1Fp8Threads) void gemm2_mxfp8_kernel(Gemm2Args a) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[G1F8::kRing];
    __shared__ QueueLdsT<kRowsLdsFp8G1> q;
    gemm2_wide<true>(a, smem, q);
}

// ---------------------------------------------------------------- combine
// out[t, c..c+8) = sum_j y[t*k + j, c..c+8) in ascending j from +0.0, fp32,
// one final rounding.  Dropped assignments have no y row and are skipped.
template <bool F32>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int cpr = a.d_h / 8;
    if (gid >= (int64_t)a.T * cpr) return;
    const int t = (int)(gid / cpr);
    const int c = (int)(gid - (int64_t)t * cpr) * 8;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
    // slots in groups of up to 4: the ids and the y rows of a group are loaded
    // together (one memory round trip, not two); a dropped slot's row holds
    // no result and its values are discarded unread by the sum
    for (int j0 = 0; j0 < a.k; j0 += 4) {
        int id[4];
        uint4 raw[4][F32 ? 2 : 1];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int64_t p = (int64_t)t * a.k + j0 + jj;
            if (j0 + jj >= a.k) break;
            id[jj] = a.ids[p];
            const uint4* src = reinterpret_cast<const uint4*>(static_cast<const unsigned char*>(a.y) +
                                                              (p * a.d_h + c) * (F32 ? 4 : 2));
            raw[jj][0] = src[0];
            if (F32) raw[jj][F32 ? 1 : 0] = src[1];
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            if (j0 + jj >= a.k) break;
            if ((unsigned)id[jj] >= (unsigned)a.E) continue;
            if (F32) {
                const uint4 u = raw[jj][0], v = raw[jj][F32 ? 1 : 0];
                acc[0] += __uint_as_float(u.x); acc[1] += __uint_as_float(u.y);
                acc[2] += __uint_as_float(u.z); acc[3] += __uint_as_float(u.w);
                acc[4] += __uint_as_float(v.x); acc[5] += __uint_as_float(v.y);
                acc[6] += __uint_as_float(v.z); acc[7] += __uint_as_float(v.w);
            } else {
                const uint4 u = raw[jj][0];
                const unsigned wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] += __uint_as_float(wd[i] << 16);
                    acc[2 * i + 1] += __uint_as_float(wd[i] & 0xFFFF0000u);
                }
            }
        }
    }
    if (F32) {
        float4* dst = reinterpret_cast<float4*>(static_cast<float*>(a.out) + (int64_t)t * a.d_h + c);
        dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
        uint4 o;
        o.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
        o.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
        o.z = f32_to_bf16(acc[4]) | (f32_to_bf16(acc[5]) << 16);
        o.w = f32_to_bf16(acc[6]) | (f32_to_bf16(acc[7]) << 16);
        *reinterpret_cast<uint4*>(static_cast<unsigned short*>(a.out) + (int64_t)t * a.d_h + c) = o;
    }
}

// int8 codes -> bf16, exactly (|q| <= 128 has at most 8 significant bits):
// 16 codes per thread
__global__ __launch_bounds__(256) void i8_to_bf16_kernel(const int8_t* x, uint16_t* xb, int64_t n16) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n16) return;
    const int4 v = reinterpret_cast<const int4*>(x)[i];
    const int wd[4] = {v.x, v.y, v.z, v.w};
    unsigned o[8];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const float lo = (float)(int8_t)((wd[j] >> (16 * b)) & 0xff);
            const float hi = (float)(int8_t)((wd[j] >> (16 * b + 8)) & 0xff);
            o[2 * j + b] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
        }
    uint4* dst = reinterpret_cast<uint4*>(xb) + 2 * i;
    dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
    dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
}

__global__ __launch_bounds__(256) void x_to_bf16_kernel(const float* x, uint16_t* xb, int64_t n8) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n8) return;
    const float4 u = reinterpret_cast<const float4*>(x)[2 * i];
    const float4 v = reinterpret_cast<const float4*>(x)[2 * i + 1];
    uint4 o;
    o.x = f32_to_bf16(u.x) | (f32_to_bf16(u.y) << 16);
    o.y = f32_to_bf16(u.z) | (f32_to_bf16(u.w) << 16);
    o.z = f32_to_bf16(v.x) | (f32_to_bf16(v.y) << 16);
    o.w = f32_to_bf16(v.z) | (f32_to_bf16(v.w) << 16);
    reinterpret_cast<uint4*>(xb)[i] = o;
}

// Packed tile order: output chunk q (16 bytes) = ((tile * kb + b) * rows + r) * 8 + s
// for tile = e * (n_out / bn) + c, rows = bn (or 2 bn gated: gate rows, then
// up rows), holding 16-byte chunk s ^ (r & 7) of K block b of the tile's row
// r, i.e. exactly what the GEMM's direct-to-LDS loads place in slot s of LDS
// row r.  A grid-stride loop over output chunks; a one-time rewrite, so plain
// 64-bit index arithmetic.
__global__ __launch_bounds__(256) void pack_kernel(const uint4* w, uint4* wp, int64_t nchunks, int64_t n_out,
                                                   int64_t kb, int bn, int gated) {
    const int64_t rows = gated ? 2 * (int64_t)bn : bn;
    const int64_t ncb = n_out / bn;
    const int64_t rows_per_e = gated ? 2 * n_out : n_out;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < nchunks;
         q += (int64_t)gridDim.x * blockDim.x) {
        const int s = (int)(q & 7);
        int64_t t = q >> 3;
        const int r = (int)(t % rows);
        t /= rows;
        const int64_t b = t % kb;
        t /= kb;
        const int64_t c = t % ncb, e = t / ncb;
        const int64_t row = !gated || r < bn ? c * bn + r : n_out + c * bn + (r - bn);
        wp[q] = w[((e * rows_per_e + row) * kb + b) * 8 + (s ^ (r & 7))];
    }
}

}  // namespace

hipError_t launch_pack(const void* w, void* wp, int64_t E, int64_t n_out, int64_t k_bytes, int bn, bool gated,
                       hipStream_t s) {
    const int64_t nchunks = E * (gated ? 2 : 1) * n_out * (k_bytes / 16);
    if (nchunks == 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((nchunks + 255) / 256, 65536);
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const uint4*>(w), static_cast<uint4*>(wp), nchunks, n_out, k_bytes / 128, bn,
                       gated ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_i8_to_bf16(const int8_t* x, uint16_t* xb, int64_t n, hipStream_t s) {
    const int64_t n16 = n / 16;
    if (n16 == 0) return hipSuccess;
    hipLaunchKernelGGL(i8_to_bf16_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s, x, xb, n16);
    return hipGetLastError();
}

hipError_t launch_x_to_bf16(const float* x, uint16_t* xb, int64_t n, hipStream_t s) {
    const int64_t n8 = n / 8;
    if (n8 == 0) return hipSuccess;
    hipLaunchKernelGGL(x_to_bf16_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s, x, xb, n8);
    return hipGetLastError();
}

hipError_t launch_gemm1(int mode, bool wide, const Gemm1Args& a, int grid, hipStream_t s, hipEvent_t t0,
                        hipEvent_t t1) {
    if (mode == MOE_MODE_MXFP8 && wide)
        hipExtLaunchKernelGGL(gemm1_mxfp8_kernel, dim3(grid), dim3(kGemm1Fp8Threads), 0, s, t0, t1, 0, a);
    else if (mode == MOE_MODE_MXFP8)
        hipExtLaunchKernelGGL(gemm1_kernel<MOE_MODE_MXFP8>, dim3(grid), dim3(kGemmThreads), 0, s, t0, t1, 0, a);
    else if (mode == MOE_MODE_FP8 && wide)
        hipExtLaunchKernelGGL(gemm1_fp8_kernel, dim3(grid), dim3(kGemm1Fp8Threads), 0, s, t0, t1, 0, a);
    else if (mode == MOE_MODE_FP8)
        hipExtLaunchKernelGGL(gemm1_kernel<MOE_MODE_FP8>, dim3(grid), dim3(kGemmThreads), 0, s, t0, t1, 0, a);
    else
        hipExtLaunchKernelGGL(gemm1_kernel<MOE_MODE_BF16>, dim3(grid), dim3(kGemmThreads), 0, s, t0, t1, 0, a);
    return hipGetLastError();
}

hipError_t launch_gemm2(int mode, bool wide, const Gemm2Args& a, int grid, hipStream_t s, hipEvent_t t0,
                        hipEvent_t t1) {
    if (mode == MOE_MODE_FP8 && wide)
        hipExtLaunchKernelGGL(gemm2_fp8_kernel, dim3(grid), dim3(kGemm1Fp8Threads), 0, s, t0, t1, 0, a);
    else if (mode == MOE_MODE_MXFP8 && wide)
        hipExtLaunchKernelGGL(gemm2_mxfp8_kernel, dim3(grid), dim3(kGemm1Fp8Threads), 0, s, t0, t1, 0, a);
    else if (mode == MOE_MODE_MXFP8)
        hipExtLaunchKernelGGL(gemm2_kernel<MOE_MODE_MXFP8>, dim3(grid), dim3(kGemmThreads), 0, s, t0, t1, 0, a);
    else if (mode == MOE_MODE_FP8)
        hipExtLaunchKernelGGL(gemm2_kernel<MOE_MODE_FP8>, dim3(grid), dim3(kGemmThreads), 0, s, t0, t1, 0, a);
    else if (mode == MOE_MODE_BF16)
        hipExtLaunchKernelGGL(gemm2_kernel<MOE_MODE_BF16>, dim3(grid), dim3(kGemmThreads), 0, s, t0, t1, 0, a);
    else
        hipExtLaunchKernelGGL(gemm2_kernel<MOE_MODE_F32ACT>, dim3(grid), dim3(kGemmThreads), 0, s, t0, t1, 0, a);
    return hipGetLastError();
}

hipError_t launch_combine(int mode, const CombineArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
    const int64_t n = (int64_t)a.T * (a.d_h / 8);
    const int blocks = (int)((n + 255) / 256);
    if (blocks == 0) return hipSuccess;
    if (mode == MOE_MODE_F32ACT)
        hipExtLaunchKernelGGL(combine_kernel<true>, dim3(blocks), dim3(256), 0, s, t0, t1, 0, a);
    else
        hipExtLaunchKernelGGL(combine_kernel<false>, dim3(blocks), dim3(256), 0, s, t0, t1, 0, a);
    return hipGetLastError();
}

hipError_t gemm_occupancy(int mode, bool wide, int* g1, int* g2) {
    hipError_t e1, e2;
    if (mode == MOE_MODE_MXFP8) {
        e1 = wide ? hipOccupancyMaxActiveBlocksPerMultiprocessor(g1, gemm1_mxfp8_kernel, kGemm1Fp8Threads, 0)
                  : hipOccupancyMaxActiveBlocksPerMultiprocessor(g1, gemm1_kernel<MOE_MODE_MXFP8>, kGemmThreads, 0);
        e2 = wide ? hipOccupancyMaxActiveBlocksPerMultiprocessor(g2, gemm2_mxfp8_kernel, kGemm1Fp8Threads, 0)
                  : hipOccupancyMaxActiveBlocksPerMultiprocessor(g2, gemm2_kernel<MOE_MODE_MXFP8>, kGemmThreads, 0);
    } else if (mode == MOE_MODE_FP8) {
        e1 = wide ? hipOccupancyMaxActiveBlocksPerMultiprocessor(g1, gemm1_fp8_kernel, kGemm1Fp8Threads, 0)
                  : hipOccupancyMaxActiveBlocksPerMultiprocessor(g1, gemm1_kernel<MOE_MODE_FP8>, kGemmThreads, 0);
        e2 = wide ? hipOccupancyMaxActiveBlocksPerMultiprocessor(g2, gemm2_fp8_kernel, kGemm1Fp8Threads, 0)
                  : hipOccupancyMaxActiveBlocksPerMultiprocessor(g2, gemm2_kernel<MOE_MODE_FP8>, kGemmThreads, 0);
    } else if (mode == MOE_MODE_BF16) {
        e1 = hipOccupancyMaxActiveBlocksPerMultiprocessor(g1, gemm1_kernel<MOE_MODE_BF16>, kGemmThreads, 0);
        e2 = hipOccupancyMaxActiveBlocksPerMultiprocessor(g2, gemm2_kernel<MOE_MODE_BF16>, kGemmThreads, 0);
    } else {
        e1 = hipOccupancyMaxActiveBlocksPerMultiprocessor(g1, gemm1_kernel<MOE_MODE_BF16>, kGemmThreads, 0);
        e2 = hipOccupancyMaxActiveBlocksPerMultiprocessor(g2, gemm2_kernel<MOE_MODE_F32ACT>, kGemmThreads, 0);
    }
    return e1 != hipSuccess ? e1 : e2;
}

}  // namespace moe
