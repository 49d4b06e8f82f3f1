// Grouped expert GEMMs of the fused MoE layer on gfx950 (CDNA4).
//
// GEMM-1: for the routed rows of one expert, G = A . W1gate^T and
//   U = A . W1up^T on MFMA with fp32 accumulators; the SwiGLU epilogue
//   h = silu(G) * U runs on the unrounded accumulators in registers and the
//   result is stored once (PipeLink section 5.5 keeps the accumulator
//   unrounded through the activation; tilelang.dataflow section 3.5 step 2
//   has the GEMM-1 handler load a token chunk and a gate/up weight shard).
// GEMM-2: Y = h . W2^T per expert, scaled by the routing weight of each row in
//   the epilogue and stored to the row of its assignment (section 3.5 step 5).
//
// Both kernels are persistent: a grid sized to the resident capacity of the
// chip pulls (expert, M-tile, column block) tasks from the device-built list
// with one atomic counter, so a hot expert's many tasks spread over all CUs
// while empty experts contribute none.
//
// Data movement.  Outside the hot expert of the largest batches these GEMMs
// stream weights: every weight byte is used by at most a few dozen rows.  So
// each K block (128 bytes of every operand row: 128 FP8 or 64 bf16 values)
// moves from HBM straight into LDS with direct-to-LDS loads
// (global_load_lds_dwordx4: 64 lanes x 16 B land contiguously), in a ring of
// kStages stages per workgroup.  A wave instruction covers 8 rows x 128 B, so
// HBM sees full 128-byte lines, and tens of KB per CU stay in flight without
// costing registers.  Routed token rows are gathered the same way, each lane
// reading its row through row_src.  In LDS a row's eight 16-byte chunks are
// XOR-swizzled by (row & 7) so the operand reads below hit distinct banks.
//
// MFMA tile mapping (16x16, wave64): lane l reads A row (l % 16) and B row
// (l % 16); the K slice of a lane is chunks {g, g+4} of the 128-byte block,
// g = l / 16 (FP8: 32 of the block's 128 values; bf16: chunk g for the first
// 16x16x32 MFMA and g+4 for the second).  A and B use the same slices, so
// each MFMA sums over whole K blocks.  The accumulator element i of lane l is
// C[4*(l/16) + i][l % 16]; the gate and up accumulators of one output column
// sit in the same lane, so SwiGLU needs no data movement.
//
// FP8 (E4M3FN): one 16x16x128 MFMA covers exactly one 128-wide scale block
// of K, so it starts from zero and its result is promoted into the fp32
// accumulator with (row scale of x or h) * (block scale of W): the block
// dequantisation happens in registers.  The row and block scales of each K
// block ride in the same LDS stage as the operands.
//
// MXFP8 (E4M3 with one E8M0 scale per 32 values along K): the MFMA applies
// the scales itself and accumulates straight into the accumulator with no
// promotion.  Its operand layout (measured): lane group g = lane/16 holds K
// [16g, 16g+16) in its first 16 bytes and K [64+16g, +16) in the last 16 (the
// {g, g+4} chunks the FP8 path loads), and the lane (r, g) supplies the
// E8M0 byte of row (or column) r for K values [32g, 32g+32), whichever lanes
// hold them.  Each stage carries the 4 scale bytes of every A and B row.
#include <algorithm>
#include <type_traits>

#include "moe_internal.h"

namespace moe {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kRowBytes = 128;                  // bytes of one operand row per stage
constexpr int kAMaxRows = 16 * kMaxRowBlocks;  // rows of the A tile

// s_waitcnt immediate that waits for vmcnt <= n and nothing else (gfx9 encoding)
template <int N>
struct VmCnt {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    static constexpr int imm = (N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8);
};

// Wait until at most n (wave-uniform, 0 <= n) of this wave's vector-memory
// operations are outstanding: a binary search over the immediates, at most
// six scalar branches.
template <int LO, int HI>
__device__ __forceinline__ void wait_vm_le_tree(int n) {
    if constexpr (LO == HI) {
        __builtin_amdgcn_s_waitcnt(VmCnt<LO>::imm);
    } else {
        constexpr int MID = (LO + HI + 1) / 2;
        if (n >= MID)
            wait_vm_le_tree<MID, HI>(n);
        else
            wait_vm_le_tree<LO, MID - 1>(n);
    }
}
__device__ __forceinline__ void wait_vm_le(int n) { wait_vm_le_tree<0, 63>(n < 63 ? n : 63); }

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
    // format 0 = E4M3 for both operands; E8M0 scale 127 = 1.0 (no MX scaling)
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// scale_a / scale_b: E8M0 byte (low 8 bits) that lane (r, g) supplies for row
// r of A / column r of B and K values [32g, 32g+32); format 0 = E4M3 for both
__device__ __forceinline__ v4f mfma_mx(const v8i& a, const v8i& b, const v4f& c, int scale_a, int scale_b) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, scale_b);
}

__device__ __forceinline__ v4f mfma_bf16(const v4i& a, const v4i& b, const v4f& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0,
                                                   0, 0);
}

// binary32 -> bfloat16 bits, round to nearest even (values here are finite)
__device__ __forceinline__ unsigned f32_to_bf16(float f) {
    unsigned u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// binary32 -> E4M3FN code via the hardware converter (round to nearest even)
__device__ __forceinline__ unsigned f32_to_e4m3(float f) {
    return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(f, 0.0f, 0, false) & 0xffu;
}

// silu(g) * u, with the hardware reciprocal (v_rcp_f32, about 1 ulp) in
// place of an IEEE division: the epilogue runs with one wave per SIMD, where
// the division's long dependent sequence is not hidden
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// clamped variant: g' = min(g, 7), u' = clamp(u, -7, 7),
// g' * sigmoid(1.702 g') * (u' + 1), with the same reciprocal
__device__ __forceinline__ float clamped_act(float g, float u) {
    g = fminf(g, 7.0f);
    u = fminf(fmaxf(u, -7.0f), 7.0f);
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-1.702f * g)) * (u + 1.0f);
}

// lane permutation within rows of 16 lanes (DPP; every lane reads a lane of
// its own row, so no bound control is needed)
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
// max over the 16 lanes of a DPP row: swap neighbours, swap pairs (each lane
// then holds its quad's max), mirror the 8-lane halves, mirror the row
__device__ __forceinline__ float row16_max(float m) {
    m = fmaxf(m, dpp<0xB1>(m));   // quad_perm [1,0,3,2]
    m = fmaxf(m, dpp<0x4E>(m));   // quad_perm [2,3,0,1]
    m = fmaxf(m, dpp<0x141>(m));  // row_half_mirror
    m = fmaxf(m, dpp<0x140>(m));  // row_mirror
    return m;
}

// Direct-to-LDS loads: lane l's 16 (or 4) bytes from its own global address
// land at LDS byte offset lds + 16*l (or 4*l); lds must be wave-uniform (it
// goes to M0).  Issued from inline asm so that the compiler does not treat
// every later LDS read as possibly aliasing an in-flight load (it would wait
// for all loads, which serialises the ring); the kernel tracks completion
// itself with s_waitcnt vmcnt.  Vector-memory loads complete in issue order,
// so loads the compiler does not see can only make its own waits stricter.
__device__ __forceinline__ void g2l16(const void* g, unsigned lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ void g2l4(const void* g, unsigned lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ unsigned lds_offset(const void* p) { return (unsigned)(uintptr_t)p; }
// The same loads from a uniform (SGPR) base plus a 32-bit per-lane offset:
// one VGPR per address instead of two.
__device__ __forceinline__ void g2l16s(const void* base, unsigned off, unsigned lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(off), "s"(base)
                 : "memory", "m0");
}
__device__ __forceinline__ void g2l4s(const void* base, unsigned off, unsigned lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(off), "s"(base)
                 : "memory", "m0");
}

// Workgroup barrier for LDS hand-offs (stages of the ring, the epilogue's
// staging, the task queue state): this wave's LDS accesses are complete
// (s_waitcnt lgkmcnt(0)) but its global stores and loads may still be in
// flight, unlike __syncthreads, whose fence would wait for every store of
// the epilogue to be acknowledged.  The workgroup shares nothing through
// global memory.  The empty asm keeps the compiler from moving LDS accesses
// across the barrier.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(VmCnt<63>::imm & ~(0xF << 8));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ v4i lds16(const unsigned char* p) { return *reinterpret_cast<const v4i*>(p); }

// the 32-byte K slice {chunk g, chunk g+4} of a swizzled 128-byte row: the
// K values lane group g of the 16x16x128 8-bit MFMA takes, in its order
__device__ __forceinline__ v8i lds_frag32(const unsigned char* row, int g, int swz) {
    const v4i lo = lds16(row + ((g ^ swz) << 4));
    const v4i hi = lds16(row + (((g + 4) ^ swz) << 4));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}


// XCD of the calling wave (HW_REG_XCC_ID).  Only the task placement depends
// on it; any value in [0, 8) is correct.
__device__ __forceinline__ int my_xcd() { return __builtin_amdgcn_s_getreg((3 << 11) | 20) & (kXcds - 1); }

// Task queue of a GEMM kernel: the list is split into kXcds segments, each
// with its own counter in its own cache line; a workgroup takes tasks from
// its own XCD's segment first, then from the others in turn.
//
// The last wave of the workgroup is also its scheduler.  It issues none of
// the stage loads (the other waves share them), so its vmcnt waits cover only
// its own queue operations, and during the last K blocks of a task it claims
// the next task, then loads that task's record and source rows (row_src, and
// for GEMM-2 the routing weight of each row) into the other half of a double
// buffer in LDS.  So no queue atomic, record load or row-index load sits
// between two tasks or stalls the ring.  Record and rows go straight to LDS
// (direct-to-LDS loads); the scheduler wave issues no global stores either.
constexpr int kSchedWave = kGemmWaves - 1;
constexpr int kLoadWaves = kGemmWaves - 1;      // waves that issue the stage loads
constexpr int kStoreThreads = 64 * kSchedWave;  // threads of the epilogue's store loops
// K blocks before the end of a task at which the scheduler claims the next
// task, settles the claim and loads the record, and loads the rows: one
// step every two K blocks, about a memory round trip apart; late enough that
// tasks go to the workgroups that finish first
constexpr int kClaimLead = 6;
// rows of a task rounded up to whole 64-lane loads (the row-index loads fill
// 64 entries per instruction)
constexpr int kRowsLds = (kAMaxRows + 63) / 64 * 64;
// the FP8 GEMM-1 kernel's tasks have up to 256 rows
constexpr int kRowsLdsFp8G1 = 16 * kMaxRowBlocksFp8G1;
static_assert(kRowsLdsFp8G1 % 64 == 0, "row-index staging in whole 64-lane loads");

template <int ROWS>
struct QueueLdsT {
    int seg[kXcds + 1];  // segment starts (and the end of the last)
    unsigned mask;       // segments found exhausted (scheduler lane 0)
    int slot;            // the task of the next round, -1 when none is left
    int4 task;           // its record {expert, first padded row, row blocks, column block}
    int rec[64];         // landing area of the record load (16 copies)
    int rows[2][ROWS];    // row_src of the task's rows, by round parity
    float roww[2][ROWS];  // GEMM-2: routing weight of the task's rows
};
using QueueLds = QueueLdsT<kRowsLds>;

// Scheduler wave state of one round.  claim() runs on lane 0; the other
// steps on the whole scheduler wave, in order.
template <int ROWS>
struct SchedT {
    int32_t* ctl;
    int base;
    const int4* tasks;
    const int32_t* row_src;
    const float* row_w;  // GEMM-2 only
    QueueLdsT<ROWS>* q;
    int xcd;
    int x = -1, raw = 0;  // lane 0: segment and result of the atomic sent ahead
    int slot = -1;

    // whole scheduler wave, waiting: read every segment's counter at once
    // (lanes 0..7, one round trip), then claim from the first segment in
    // this XCD's order that still has tasks; repeat if another workgroup took
    // the last one meanwhile.  -1 once every segment is exhausted.
    __device__ __forceinline__ int claim_any() {
        const int lane = threadIdx.x & 63;
        for (int round = 0; round < kXcds; ++round) {
            const int y = (xcd + lane) & (kXcds - 1);
            bool avail = false;
            if (lane < kXcds) {
                const int c = __hip_atomic_load(&ctl[base + kQueueStride * y], __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
                avail = q->seg[y] + c < q->seg[y + 1];
            }
            const uint64_t av = __ballot(avail);
            const uint64_t gone = __ballot(lane < kXcds && !avail);
            int got = -1;
            if (lane == 0) {
                for (int l = 0; l < kXcds; ++l)
                    if ((gone >> l) & 1u) q->mask |= 1u << ((xcd + l) & (kXcds - 1));
                if (av) {
                    const int yy = (xcd + __builtin_ctzll(av)) & (kXcds - 1);
                    const int j = atomicAdd(&ctl[base + kQueueStride * yy], 1);
                    if (q->seg[yy] + j < q->seg[yy + 1])
                        got = q->seg[yy] + j;
                    else
                        q->mask |= 1u << yy;
                }
            }
            got = __shfl(got, 0, 64);
            if (got >= 0 || av == 0) return got;
        }
        return -1;
    }

    __device__ __forceinline__ void claim() {
        for (int i = 0; i < kXcds; ++i) {
            const int y = (xcd + i) & (kXcds - 1);
            if (!((q->mask >> y) & 1u)) {
                x = y;
                break;
            }
        }
        if (x >= 0) raw = atomicAdd(&ctl[base + kQueueStride * x], 1);
    }
    // the workgroup's first task: the one assigned statically to it, if its
    // segment has enough tasks, else one claimed from the queue; then start
    // loading the record
    __device__ __forceinline__ void first() {
        const int xs = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
        if (j < static_tasks(gridDim.x, xs, q->seg[xs + 1] - q->seg[xs])) {
            slot = q->seg[xs] + j;
            g2l4(reinterpret_cast<const int*>(tasks + slot) + ((threadIdx.x & 63) & 3), lds_offset(q->rec));
        } else {
            settle(false);
        }
    }
    // settle the claim (ahead: the atomic sent by claim(), and if its
    // segment ran out, claim_any; else claim_any now) and start loading the
    // record
    __device__ __forceinline__ void settle(bool ahead) {
        const int lane = threadIdx.x & 63;
        bool search = !ahead;
        int sl = -1;
        if (ahead) {
            int got = -1, ran_out = 0;
            if (lane == 0 && x >= 0) {
                if (q->seg[x] + raw < q->seg[x + 1]) {
                    got = q->seg[x] + raw;
                } else {
                    q->mask |= 1u << x;
                    ran_out = 1;
                }
            }
            sl = __shfl(got, 0, 64);
            search = __shfl(ran_out, 0, 64) != 0;
        }
        if (search) sl = claim_any();
        slot = sl;
        if (slot >= 0) g2l4(reinterpret_cast<const int*>(tasks + slot) + (lane & 3), lds_offset(q->rec));
    }
    // once the record has landed: load the task's source rows into rows[par]
    // and roww[par].  All 64 lanes take part in every direct-to-LDS load
    // (lanes past the task's rows reread its first row).
    __device__ __forceinline__ void load_rows(int par) {
        if (slot < 0) return;
        const int lane = threadIdx.x & 63;
        __builtin_amdgcn_s_waitcnt(VmCnt<0>::imm);
        asm volatile("" ::: "memory");
        const int row0 = __builtin_amdgcn_readfirstlane(q->rec[1]);
        const int n = 16 * __builtin_amdgcn_readfirstlane(q->rec[2]);
#pragma unroll
        for (int j = 0; j < ROWS / 64; ++j) {
            if (64 * j >= n) break;
            const int r = 64 * j + lane < n ? 64 * j + lane : 0;
            g2l4(row_src + row0 + r, lds_offset(&q->rows[par][64 * j]));
            if (row_w) g2l4(row_w + row0 + r, lds_offset(&q->roww[par][64 * j]));
        }
    }
    // before the round's last barrier: the rows have landed; publish the record
    __device__ __forceinline__ void publish() {
        __builtin_amdgcn_s_waitcnt(VmCnt<0>::imm);
        asm volatile("" ::: "memory");
        if ((threadIdx.x & 63) == 0) {
            q->slot = slot;
            if (slot >= 0) q->task = make_int4(q->rec[0], q->rec[1], q->rec[2], q->rec[3]);
        }
    }
};
using Sched = SchedT<kRowsLds>;

// ------------------------------------------------------------------ configs
// Stage of the ring for a task of NSUB group blocks: the K block of the
// task's weight rows (B), of its 16*NSUB operand rows (A) and, in FP8 mode,
// their scales.  The ring has a fixed byte size per kernel, so tasks with
// fewer rows get more stages in flight.
template <int MODE, bool GATED>
struct Cfg {
    static constexpr bool kBS = MODE == MOE_MODE_FP8;     // fp32 block scales, promoted per K block
    static constexpr bool kMX = MODE == MOE_MODE_MXFP8;   // E8M0 scales per 32, applied by the MFMA
    static constexpr bool kFP8 = kBS || kMX;              // one-byte e4m3 operands
    static constexpr int kNFW = (GATED && !kFP8) ? 1 : 2;  // 16-column fragments per wave
    static constexpr int kBN = 16 * kNFW * kGemmWaves;     // output columns per task
    static constexpr int kBRows = GATED ? 2 * kBN : kBN;   // weight rows per task
    static constexpr int kBAll = kBRows / 8;                            // B loads per stage (8 rows each)
    static constexpr int kBMax = (kBAll + kLoadWaves - 1) / kLoadWaves;  // per loading wave, at most
    static constexpr int kStageB = kBRows * kRowBytes;
    // FP8: up to 128 row scales (waves 0 and 2), then the block scale(s) (wave 1);
    // MXFP8: the 4 scale bytes of this K block for every A row, then every B row
    static constexpr int kStageS = kBS ? 1024 : kMX ? 4 * (kAMaxRows + kBRows) : 0;
    static constexpr int stage_bytes(int nsub) { return kStageB + 16 * nsub * kRowBytes + kStageS; }
    // ring: FP8 / MXFP8 GEMM-1 (256 weight rows per stage) takes a whole CU's LDS
    // (three stages of a 128-row task, four of a 16-row one); the others take
    // four stages of a one-block task, so two workgroups share a CU
    static constexpr int kRing = (GATED && kFP8) ? 160 * 1024 - 2560 : 4 * stage_bytes(1);
    // stages in a ring of `ring` bytes
    static constexpr int stages(int nsub, int ring) {
        return ring / stage_bytes(nsub) < 8 ? ring / stage_bytes(nsub) : 8;
    }
    static constexpr int kOutBytes = (MODE == MOE_MODE_F32ACT && !GATED) ? 4 : (GATED && kFP8 ? 1 : 2);
    static constexpr int kEpiRow = kBN * kOutBytes;  // bytes of one staged output row
    static_assert(kEpiRow * kAMaxRows + kGemmWaves * kAMaxRows * 4 <= kRing,
                  "epilogue staging must fit in the stage ring");
    static_assert(stages(kMaxRowBlocks, kRing) >= 2, "ring too small");
    static_assert(kRing <= 160 * 1024, "LDS budget");
    static_assert(GATED || kBN == 128, "GEMM-2 tasks are 128 columns wide (one W2 scale block row)");
};

// ------------------------------------------------------------------ kernel
// One task: rows [row0, row0 + 16*NSUB) of expert e, output column block cb.
//   GATED (GEMM-1): A rows are tokens x[row_src[r] / k] (zero row for padding),
//     B rows are W1[e] gate rows cb*kBN.. and up rows d_e + cb*kBN..; the
//     epilogue writes h[row0 + r][cb*kBN ..] (+ FP8 scale).
//   !GATED (GEMM-2): A rows are h[row0 + r], B rows W2[e] rows cb*kBN..; the
//     epilogue scales by topk_w[row_src[r]] and writes y[row_src[r]][cb*kBN ..].
// K is the contraction length (d_h or d_e); N_out is d_e (GATED) or d_h.
template <int MODE, bool GATED, int NSUB, int RING>
__device__ __forceinline__ void gemm_task(const void* a_base, const void* a_scale_v, const int32_t* row_src,
                                          int a_div, const void* wts, const void* w_scale_v, const unsigned char* zero,
                                          int e, int row0, int cb, int K, int N_out, bool packed,
                                          unsigned char* smem, const Gemm1Args* g1, const Gemm2Args* g2,
                                          Sched& sch, const int* rows, const float* roww, int par) {
    using C = Cfg<MODE, GATED>;
    constexpr bool kFP8 = C::kFP8, kBS = C::kBS, kMX = C::kMX;
    const float* a_scale = static_cast<const float*>(a_scale_v);  // FP8 mode
    const float* w_scale = static_cast<const float*>(w_scale_v);
    constexpr int S = C::stages(NSUB, RING);
    static_assert(RING >= C::kRing, "ring smaller than this GEMM's");
    constexpr int kStage = C::stage_bytes(NSUB);
    constexpr int kStageA = 16 * NSUB * kRowBytes;
    constexpr int kAInstr = 2 * NSUB;  // A loads per stage: 8 rows each
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, lg = lane >> 4;
    const int nk = K / (kFP8 ? 128 : 64);
    const unsigned smem_lds = lds_offset(smem);
    const int64_t ld_bytes = (int64_t)K * (kFP8 ? 1 : 2);  // bytes per operand row
    // vector-memory loads this wave issues per stage: B and A instructions
    // w, w+3, ... (8 rows each) and, in FP8 mode, the row scales (waves 0
    // and 2) or the block scales (wave 1); the scheduler wave issues none
    const bool loader = w < kLoadWaves;
    const int n_b = loader ? (C::kBAll - 1 - w) / kLoadWaves + 1 : 0;
    const int n_a = loader && w < kAInstr ? (kAInstr - 1 - w) / kLoadWaves + 1 : 0;
    int n_s = 0;
    if constexpr (kBS) n_s = (w < 2 || (w == 2 && NSUB > 4)) ? 1 : 0;
    if constexpr (kMX) n_s = w == 0 ? 2 : w == 1 ? (GATED ? 2 : 1) : w == 2 ? (NSUB > 4) + (GATED ? 1 : 0) : 0;
    const int loads_per_stage = n_b + n_a + n_s;

    // ---- per-lane load sources (stage 0); a K block advances the A sources by
    // 128 bytes and the B sources by b_step: 128 bytes in row-major weights,
    // a whole stage in packed ones, where the stages of task (e, cb) follow
    // each other and each holds its rows already in the swizzled LDS order
    const unsigned char* bsrc[C::kBMax];
    const int64_t b_step = packed ? C::kStageB : kRowBytes;
#pragma unroll
    for (int j = 0; j < C::kBMax; ++j) {
        const int b = w + kLoadWaves * j;  // B instruction: tile rows 8*b .. 8*b+7
        if (packed) {
            const int64_t tile = (int64_t)e * (N_out / C::kBN) + cb;
            bsrc[j] = static_cast<const unsigned char*>(wts) + tile * nk * C::kStageB + (b * 64 + lane) * 16;
            continue;
        }
        const int r = 8 * b + (lane >> 3);  // tile row (past the tile for unused b: never loaded)
        const int c = (lane & 7) ^ (r & 7);
        int64_t wrow;
        if constexpr (GATED)
            wrow = r < C::kBN ? (int64_t)cb * C::kBN + r : (int64_t)N_out + (int64_t)cb * C::kBN + (r - C::kBN);
        else
            wrow = (int64_t)cb * C::kBN + r;
        const int64_t rows_per_expert = GATED ? 2 * (int64_t)N_out : (int64_t)N_out;
        bsrc[j] = static_cast<const unsigned char*>(wts) + ((int64_t)e * rows_per_expert + wrow) * ld_bytes + c * 16;
    }
    constexpr int kAMaxPerWave = (kAInstr + kLoadWaves - 1) / kLoadWaves;
    const unsigned char* asrc[kAMaxPerWave];
    bool apad[kAMaxPerWave];
#pragma unroll
    for (int j = 0; j < kAMaxPerWave; ++j) {
        const int ai = w + kLoadWaves * j;  // A instruction: rows 8*ai .. 8*ai+7
        const int r = 8 * ai + (lane >> 3);
        const int c = (lane & 7) ^ (r & 7);
        apad[j] = false;
        asrc[j] = zero;
        if (loader && ai < kAInstr) {
            if constexpr (GATED) {
                const int p = rows[r];
                apad[j] = p < 0;
                asrc[j] = apad[j] ? zero + c * 16
                                  : static_cast<const unsigned char*>(a_base) + (int64_t)(p / a_div) * ld_bytes + c * 16;
            } else {
                // GEMM-2 reads its own padded rows (GEMM-1 wrote zeros there)
                asrc[j] = static_cast<const unsigned char*>(a_base) + (int64_t)(row0 + r) * ld_bytes + c * 16;
            }
        }
    }
    // scale sources: wave 0 lane r -> row scale of tile row r, wave 2 lane r
    // -> row 64 + r; wave 1 lane 0 (and 1) -> block scale(s) of W for this K block
    const float* ssrc = nullptr;
    bool son = false, spad = false;
    if constexpr (kBS) {
        const int kq = K / kQ;
        const int srow = (w == 2 ? 64 : 0) + lane;
        if ((w == 0 || w == 2) && srow < 16 * NSUB) {
            son = true;
            const int p = rows[srow];
            if (GATED) {
                spad = p < 0;
                ssrc = spad ? reinterpret_cast<const float*>(zero) : a_scale + (int64_t)(p / a_div) * kq;
            } else {
                ssrc = a_scale + (int64_t)(row0 + srow) * kq;
            }
        } else if (w == 1 && lane < (GATED ? 2 : 1)) {
            son = true;
            // W1 scales [E][2 d_e/128][d_h/128]: gate block row cb, up block row d_e/128 + cb
            // W2 scales [E][d_h/128][d_e/128]: block row cb (128-column tasks)
            const int64_t nrb = GATED ? 2 * (int64_t)N_out / kQ : (int64_t)N_out / kQ;
            const int64_t brow = GATED ? (lane == 0 ? cb : N_out / kQ + cb) : (int64_t)cb;
            ssrc = w_scale + ((int64_t)e * nrb + brow) * kq;
        }
    }
    // MXFP8 scale sources: lane l of a slot reads the 4 bytes (K block kc's
    // four E8M0 scales) of one row, rows stored [rows][K/32]:
    //   wave 0: A rows 0..63 and B rows 0..63; wave 1: B rows 64..127 (and
    //   128..191 in GEMM-1); wave 2: A rows 64..127 (more than 4 row blocks)
    //   and, in GEMM-1, B rows 192..255.  LDS: A row r at 4*r, B row r at
    //   4*(128 + r); mdst is the wave's base (lane l writes mdst + 4*l).
    const unsigned char* msrc[2] = {zero, zero};
    bool mon[2] = {false, false}, mfix[2] = {true, true};  // mfix: padding row, source not advanced
    unsigned mdst[2] = {0u, 0u};
    if constexpr (kMX) {
        const unsigned char* as8 = static_cast<const unsigned char*>(a_scale_v);
        const unsigned char* ws8 = static_cast<const unsigned char*>(w_scale_v);
        const int64_t kq = K / 32;  // scale bytes per row
        auto a_row = [&](int slot, int r) {
            mon[slot] = true;
            mdst[slot] = 4u * (r - lane);
            if (r >= 16 * NSUB) return;  // past the task's rows: zeros, never read
            if constexpr (GATED) {
                const int p = rows[r];
                if (p < 0) return;  // padding row: zero codes, zero scale bytes
                msrc[slot] = as8 + (int64_t)(p / a_div) * kq;
            } else {
                msrc[slot] = as8 + (int64_t)(row0 + r) * kq;
            }
            mfix[slot] = false;
        };
        auto b_row = [&](int slot, int r) {
            mon[slot] = true;
            mdst[slot] = 4u * (kAMaxRows + r - lane);
            int64_t wrow;
            if constexpr (GATED)
                wrow = r < C::kBN ? (int64_t)cb * C::kBN + r : (int64_t)N_out + (int64_t)cb * C::kBN + (r - C::kBN);
            else
                wrow = (int64_t)cb * C::kBN + r;
            msrc[slot] = ws8 + ((int64_t)e * (GATED ? 2 : 1) * N_out + wrow) * kq;
            mfix[slot] = false;
        };
        if (w == 0) {
            a_row(0, lane);
            b_row(1, lane);
        } else if (w == 1) {
            b_row(0, 64 + lane);
            if (GATED) b_row(1, 128 + lane);
        } else if (w == 2) {
            if (NSUB > 4) a_row(0, 64 + lane);
            if (GATED) b_row(NSUB > 4 ? 1 : 0, 192 + lane);
        }
    }

    // Routing weight of each tile row: GEMM-1 tasks of column block 0 look it
    // up (topk_w[row_src]) and store it by padded row for GEMM-2, whose
    // scheduler wave loads it with the rows of its next task.  Row
    // 64 * w + lane in waves 0 and 1; the load is issued ahead of the stage
    // loads.
    constexpr int kRows = 16 * NSUB;
    const int w_row = 64 * w + lane;
    const bool w_owner = GATED && cb == 0 && w < 2 && w_row < kRows;
    float ep_w = 0.f;
    if constexpr (GATED) {
        if (w_owner) {
            const int p = rows[w_row];
            ep_w = p >= 0 ? g1->topk_w[p] : 0.f;
        }
    }
    // INT8 tokens (bf16 GEMM on the widened codes): each row's token scale,
    // loaded ahead like the routing weight (waves 0 and 1, one row per lane)
    // and applied to the gate and up accumulators before the activation
    float ep_xs = 0.f;
    bool xs_owner = false;
    if constexpr (GATED && !kFP8) {
        xs_owner = g1->x_row_scale && w < 2 && w_row < kRows;
        if (xs_owner) {
            const int p = rows[w_row];
            ep_xs = p >= 0 ? g1->x_row_scale[p / a_div] : 0.f;
        }
    }

    auto issue = [&](int kc) {
        const unsigned st = smem_lds + (unsigned)((kc % S) * kStage);
        const int64_t koff = (int64_t)kc * kRowBytes;
        const int64_t boff = (int64_t)kc * b_step;
        if (!loader) return;
#pragma unroll
        for (int j = 0; j < C::kBMax; ++j) {
            const int b = w + kLoadWaves * j;
            if (b < C::kBAll) g2l16(bsrc[j] + boff, st + (unsigned)(b * 1024));
        }
#pragma unroll
        for (int j = 0; j < kAMaxPerWave; ++j) {
            const int ai = w + kLoadWaves * j;
            if (ai < kAInstr) g2l16(apad[j] ? asrc[j] : asrc[j] + koff, st + (unsigned)(C::kStageB + ai * 1024));
        }
        if constexpr (kBS) {
            // wave 0 reads the row scales, wave 1 the weights' block scales
            const unsigned ss = st + (unsigned)(C::kStageB + kStageA);
            if (son) g2l4(spad ? ssrc : ssrc + kc, ss + (unsigned)(w == 1 ? 512 : w * 128));
        }
        if constexpr (kMX) {
            const unsigned ss = st + (unsigned)(C::kStageB + kStageA);
#pragma unroll
            for (int m = 0; m < 2; ++m)
                if (mon[m]) g2l4(mfix[m] ? msrc[m] : msrc[m] + 4 * kc, ss + mdst[m]);
        }
    };

    v4f acc[NSUB][C::kNFW][GATED ? 2 : 1];
    const v4f zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int f = 0; f < C::kNFW; ++f)
#pragma unroll
            for (int q = 0; q < (GATED ? 2 : 1); ++q) acc[s][f][q] = zero4;

    const int swz = lr & 7;
    const int npro = nk < S - 1 ? nk : S - 1;
    for (int kc = 0; kc < npro; ++kc) issue(kc);
    const int claim_at = nk > kClaimLead ? nk - kClaimLead : 0;
    const int settle_at = nk > kClaimLead - 2 ? nk - (kClaimLead - 2) : 0;
    const int rows_at = nk > kClaimLead - 4 ? nk - (kClaimLead - 4) : 0;
    for (int kc = 0; kc < nk; ++kc) {
        // stage kc is complete once at most the younger stages' loads remain
        // (each loading wave waits for its own; the barrier covers the rest)
        if (loader) {
            const int younger = (nk - 1 - kc) < (S - 2) ? (nk - 1 - kc) : (S - 2);
            wait_vm_le(younger * loads_per_stage);
        }
        lds_barrier();
        if (kc + S - 1 < nk) issue(kc + S - 1);
        if (w == kSchedWave) {
            if (kc == claim_at && lane == 0) sch.claim();
            if (kc == settle_at) sch.settle(true);
            if (kc == rows_at) sch.load_rows(par ^ 1);
        }
        const unsigned char* st = smem + (kc % S) * kStage;
        const unsigned char* sb = st;
        const unsigned char* sa = st + C::kStageB;
        if constexpr (kMX) {
            // lane (lr, lg): chunks lg and lg + 4 of row lr of each fragment, and
            // the scale byte of row lr for K values [32 lg, 32 lg + 32) (row r's
            // four bytes at 4 r + 0..3)
            const unsigned char* sc = st + C::kStageB + kStageA;
            v8i A[NSUB];
            int sxa[NSUB];
#pragma unroll
            for (int s = 0; s < NSUB; ++s) {
                A[s] = lds_frag32(sa + (16 * s + lr) * kRowBytes, lg, swz);
                sxa[s] = sc[4 * (16 * s + lr) + lg];
            }
            const unsigned char* scb = sc + 4 * kAMaxRows;
#pragma unroll
            for (int f = 0; f < C::kNFW; ++f) {
                const int brow = 16 * (C::kNFW * w + f) + lr;
                const v8i Bg = lds_frag32(sb + brow * kRowBytes, lg, swz);
                const int sbg = scb[4 * brow + lg];
#pragma unroll
                for (int s = 0; s < NSUB; ++s) acc[s][f][0] = mfma_mx(A[s], Bg, acc[s][f][0], sxa[s], sbg);
                if constexpr (GATED) {
                    const v8i Bu = lds_frag32(sb + (C::kBN + brow) * kRowBytes, lg, swz);
                    const int sbu = scb[4 * (C::kBN + brow) + lg];
#pragma unroll
                    for (int s = 0; s < NSUB; ++s)
                        acc[s][f][GATED ? 1 : 0] = mfma_mx(A[s], Bu, acc[s][f][GATED ? 1 : 0], sxa[s], sbu);
                }
            }
        } else if constexpr (kBS) {
            // software-pipelined by one row block: the MFMAs of row block s
            // are issued, and the LDS reads of row block s + 1 started, before
            // the promotion of row block s - 1 reads its results, so neither
            // an MFMA result nor an LDS read is waited for right after issue
            const float* sc = reinterpret_cast<const float*>(st + C::kStageB + kStageA);
            const float swg = sc[128];  // written by lane 0 (and 1) of wave 1
            const float swu = GATED ? sc[129] : 0.f;
            constexpr int kG = GATED ? 2 : 1;
            constexpr int kT = C::kNFW * kG;  // MFMAs per row block
            v8i Bf[C::kNFW][kG];
#pragma unroll
            for (int f = 0; f < C::kNFW; ++f) {
                const int brow = 16 * (C::kNFW * w + f) + lr;
                Bf[f][0] = lds_frag32(sb + brow * kRowBytes, lg, swz);
                if constexpr (GATED) Bf[f][kG - 1] = lds_frag32(sb + (C::kBN + brow) * kRowBytes, lg, swz);
            }
            v4f tp[kT];
            float pp[kG][4];
            auto promote = [&](int s) {
#pragma unroll
                for (int f = 0; f < C::kNFW; ++f)
#pragma unroll
                    for (int g = 0; g < kG; ++g)
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc[s][f][g][i] += tp[f * kG + g][i] * pp[g][i];
            };
            v8i A = lds_frag32(sa + lr * kRowBytes, lg, swz);
#pragma unroll
            for (int s = 0; s < NSUB; ++s) {
                v4f tq[kT];
#pragma unroll
                for (int f = 0; f < C::kNFW; ++f)
#pragma unroll
                    for (int g = 0; g < kG; ++g) tq[f * kG + g] = mfma_fp8(A, Bf[f][g], zero4);
                v8i An = A;
                if (s + 1 < NSUB) An = lds_frag32(sa + (16 * (s + 1) + lr) * kRowBytes, lg, swz);
                float sx[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) sx[i] = sc[16 * s + 4 * lg + i];
                __builtin_amdgcn_sched_barrier(0);
                if (s > 0) promote(s - 1);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < kT; ++j) tp[j] = tq[j];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pp[0][i] = sx[i] * swg;
                    if constexpr (GATED) pp[kG - 1][i] = sx[i] * swu;
                }
                A = An;
            }
            promote(NSUB - 1);
        } else {
            // two 16x16x32 bf16 MFMAs per K block: chunk g, then chunk g+4
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int ch = ((lg + 4 * half) ^ swz) << 4;
                v4i A[NSUB];
#pragma unroll
                for (int s = 0; s < NSUB; ++s) A[s] = lds16(sa + (16 * s + lr) * kRowBytes + ch);
#pragma unroll
                for (int f = 0; f < C::kNFW; ++f) {
                    const int brow = 16 * (C::kNFW * w + f) + lr;
                    const v4i Bg = lds16(sb + brow * kRowBytes + ch);
#pragma unroll
                    for (int s = 0; s < NSUB; ++s) acc[s][f][0] = mfma_bf16(A[s], Bg, acc[s][f][0]);
                    if constexpr (GATED) {
                        const v4i Bu = lds16(sb + (C::kBN + brow) * kRowBytes + ch);
#pragma unroll
                        for (int s = 0; s < NSUB; ++s)
                            acc[s][f][GATED ? 1 : 0] = mfma_bf16(A[s], Bu, acc[s][f][GATED ? 1 : 0]);
                    }
                }
            }
        }
    }

    // every wave: the stage loads are complete (and the scheduler's queue
    // loads, issued two K blocks ago); this also settles, for the compiler's
    // own bookkeeping, every load it saw (no store of the previous task is
    // still young)
    __builtin_amdgcn_s_waitcnt(VmCnt<0>::imm);

    // ---- epilogue: stage the output tile in LDS, then 16-byte row stores
    lds_barrier();  // every wave is done with the ring
    unsigned char* stage = smem;                                              // [16*NSUB][kEpiRow]
    float* s_amax = reinterpret_cast<float*>(smem + C::kEpiRow * kAMaxRows);  // [waves][kAMaxRows]
    if constexpr (GATED && !kFP8) {
        if (g1->x_row_scale) {  // uniform: INT8 mode
            // dequantisation: the GEMM ran on the integer codes, so each row's
            // accumulators take its token's scale (one fp32 multiply each)
            float* s_xs = s_amax;  // [kAMaxRows], past the staging rows
            if (xs_owner) s_xs[w_row] = ep_xs;
            lds_barrier();
#pragma unroll
            for (int s = 0; s < NSUB; ++s)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float sc = s_xs[16 * s + 4 * lg + i];
#pragma unroll
                    for (int f = 0; f < C::kNFW; ++f) {
                        acc[s][f][0][i] *= sc;
                        acc[s][f][1][i] *= sc;
                    }
                }
        }
    }
    if constexpr (GATED) {
        if (w_owner) g1->row_w[row0 + w_row] = ep_w;
        float hv[NSUB][C::kNFW][4];
        if (g1->act == MOE_ACT_SWIGLU_CLAMPED) {
#pragma unroll
            for (int s = 0; s < NSUB; ++s)
#pragma unroll
                for (int f = 0; f < C::kNFW; ++f)
#pragma unroll
                    for (int i = 0; i < 4; ++i) hv[s][f][i] = clamped_act(acc[s][f][0][i], acc[s][f][1][i]);
        } else {
#pragma unroll
            for (int s = 0; s < NSUB; ++s)
#pragma unroll
                for (int f = 0; f < C::kNFW; ++f)
#pragma unroll
                    for (int i = 0; i < 4; ++i) hv[s][f][i] = silu_mul(acc[s][f][0][i], acc[s][f][1][i]);
        }
        if constexpr (kMX) {
            // per-row-per-32 requantisation: this wave's two fragments are
            // columns [32 w, 32 w + 32) of the task, one MX block.  Shared
            // exponent: floor(log2 amax) - 8 (the e4m3 maximum is 1.75 * 2^8),
            // stored biased by 127 and clamped to [0, 254]; an all-zero block
            // stores 127.  Elements: v * 2^-exponent, saturated to +-448.
            uint8_t* hs = static_cast<uint8_t*>(g1->h_scale);
#pragma unroll
            for (int s = 0; s < NSUB; ++s)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = 16 * s + 4 * lg + i;
                    float m = 0.f;
#pragma unroll
                    for (int f = 0; f < C::kNFW; ++f) m = fmaxf(m, fabsf(hv[s][f][i]));
                    m = row16_max(m);
                    // frexp: m = f * 2^x with f in [0.5, 1), so floor(log2 m) = x - 1
                    int b = m > 0.f ? __builtin_amdgcn_frexp_expf(m) - 1 - 8 + 127 : 127;
                    b = b < 0 ? 0 : (b > 254 ? 254 : b);
#pragma unroll
                    for (int f = 0; f < C::kNFW; ++f) {
                        float v = __builtin_amdgcn_ldexpf(hv[s][f][i], 127 - b);
                        v = fminf(fmaxf(v, -448.0f), 448.0f);
                        stage[rr * C::kEpiRow + 16 * (C::kNFW * w + f) + lr] = (unsigned char)f32_to_e4m3(v);
                    }
                    if (lr == 0) hs[(int64_t)(row0 + rr) * (N_out / 32) + cb * kGemmWaves + w] = (uint8_t)b;
                }
        } else if constexpr (kBS) {
            // per-row-per-128 requantisation: amax over the task's 128 columns
#pragma unroll
            for (int s = 0; s < NSUB; ++s)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float m = 0.f;
#pragma unroll
                    for (int f = 0; f < C::kNFW; ++f) m = fmaxf(m, fabsf(hv[s][f][i]));
                    m = row16_max(m);  // the 16 lanes of a row group hold one tile row
                    if (lr == 0) s_amax[w * kAMaxRows + 16 * s + 4 * lg + i] = m;
                }
            lds_barrier();
            // every partial amax of this lane's rows (rows 16 s + 4 lg + i,
            // i = 0..3, are four consecutive floats per wave) is read before
            // the first staging write, so the reads go out back to back and
            // are waited for once
            static_assert(C::kNFW == 2, "two 16-column fragments per wave");
            float amax[NSUB][4];
#pragma unroll
            for (int s = 0; s < NSUB; ++s) {
                float4 m = *reinterpret_cast<const float4*>(&s_amax[16 * s + 4 * lg]);
#pragma unroll
                for (int ww = 1; ww < kGemmWaves; ++ww) {
                    const float4 o = *reinterpret_cast<const float4*>(&s_amax[ww * kAMaxRows + 16 * s + 4 * lg]);
                    m = make_float4(fmaxf(m.x, o.x), fmaxf(m.y, o.y), fmaxf(m.z, o.z), fmaxf(m.w, o.w));
                }
                amax[s][0] = m.x;
                amax[s][1] = m.y;
                amax[s][2] = m.z;
                amax[s][3] = m.w;
            }
#pragma unroll
            for (int s = 0; s < NSUB; ++s)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rr = 16 * s + 4 * lg + i;
                    const float am = amax[s][i];
                    // scale amax/448; values are multiplied by its reciprocal
                    // (|v| * 448/amax stays within rounding of 448, the e4m3 maximum)
                    const float sc = am > 0.f ? am * (1.0f / 448.0f) : 1.0f;
                    const float inv = am > 0.f ? 448.0f * __builtin_amdgcn_rcpf(am) : 1.0f;
                    // both fragments' codes from one converter instruction
                    const unsigned q2 = (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(hv[s][0][i] * inv, hv[s][1][i] * inv, 0, false);
                    stage[rr * C::kEpiRow + 16 * (C::kNFW * w) + lr] = (unsigned char)(q2 & 0xffu);
                    stage[rr * C::kEpiRow + 16 * (C::kNFW * w + 1) + lr] = (unsigned char)((q2 >> 8) & 0xffu);
                    if (w == 0 && lr == 0) static_cast<float*>(g1->h_scale)[(int64_t)(row0 + rr) * (N_out / kQ) + cb] = sc;
                }
        } else {
#pragma unroll
            for (int s = 0; s < NSUB; ++s)
#pragma unroll
                for (int f = 0; f < C::kNFW; ++f)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int rr = 16 * s + 4 * lg + i;
                        reinterpret_cast<unsigned short*>(stage + rr * C::kEpiRow)[16 * (C::kNFW * w + f) + lr] =
                            (unsigned short)f32_to_bf16(hv[s][f][i]);
                    }
        }
        lds_barrier();
        // h[row0 + r][cb*kBN ...]: kEpiRow bytes per row
        constexpr int kChunks = C::kEpiRow / 16;
        unsigned char* h = static_cast<unsigned char*>(g1->h);
        const int64_t hrow_bytes = (int64_t)N_out * (kFP8 ? 1 : 2);
        if (w != kSchedWave)
            for (int i = threadIdx.x; i < 16 * NSUB * kChunks; i += kStoreThreads) {
                const int r = i / kChunks, c = i - r * kChunks;
                *reinterpret_cast<v4i*>(h + (int64_t)(row0 + r) * hrow_bytes + (int64_t)cb * C::kEpiRow + c * 16) =
                    *reinterpret_cast<const v4i*>(stage + r * C::kEpiRow + c * 16);
            }
    } else {
        constexpr bool kF32 = MODE == MOE_MODE_F32ACT;
#pragma unroll
        for (int s = 0; s < NSUB; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int rr = 16 * s + 4 * lg + i;
                const float wt = roww[rr];  // 0 on padding rows
#pragma unroll
                for (int f = 0; f < C::kNFW; ++f) {
                    const float v = acc[s][f][0][i] * wt;
                    const int col = 16 * (C::kNFW * w + f) + lr;
                    if constexpr (kF32)
                        reinterpret_cast<float*>(stage + rr * C::kEpiRow)[col] = v;
                    else
                        reinterpret_cast<unsigned short*>(stage + rr * C::kEpiRow)[col] = (unsigned short)f32_to_bf16(v);
                }
            }
        lds_barrier();
        constexpr int kChunks = C::kEpiRow / 16;
        unsigned char* y = static_cast<unsigned char*>(g2->y);
        const int64_t yrow_bytes = (int64_t)N_out * C::kOutBytes;
        if (w != kSchedWave)
            for (int i = threadIdx.x; i < 16 * NSUB * kChunks; i += kStoreThreads) {
                const int r = i / kChunks, c = i - r * kChunks;
                const int p = rows[r];
                if (p < 0) continue;
                *reinterpret_cast<v4i*>(y + (int64_t)p * yrow_bytes + (int64_t)cb * C::kEpiRow + c * 16) =
                    *reinterpret_cast<const v4i*>(stage + r * C::kEpiRow + c * 16);
            }
    }
    if (w == kSchedWave) sch.publish();
    lds_barrier();  // the ring and the staging area are refilled by the next task
}

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

// ------------------------------------------------------- FP8 GEMM-1 (8 waves)
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
// bounds this kernel before HBM or the MFMAs do.  Seven waves issue the
// stage loads; the last one is the scheduler (as in gemm_task) and computes.
struct G1F8 {
    static constexpr int kWaves = kGemm1Fp8Waves;
    static constexpr int kSched = kWaves - 1;
    static constexpr int kLoaders = kWaves - 1;
    static constexpr int kStoreThreads = 64 * kSched;
    static constexpr int kMaxRows = 16 * kMaxRowBlocksFp8G1;
    static constexpr int kBN = 128;
    static constexpr int kBRows = 2 * kBN;
    static constexpr int kBAll = kBRows / 8;                         // B loads per stage
    static constexpr int kBMax = (kBAll + kLoaders - 1) / kLoaders;  // per loading wave, at most
    static constexpr int kAMax = (2 * kMaxRowBlocksFp8G1 + kLoaders - 1) / kLoaders;
    static constexpr int kStageB = kBRows * kRowBytes;
    // row scales of up to 256 rows (4 B each), then the gate and up block scales
    static constexpr int kScaleBlk = 4 * kMaxRows;
    static constexpr int kStageS = kScaleBlk + 16;
    static constexpr int stage_bytes(int nsub) { return kStageB + 16 * nsub * kRowBytes + kStageS; }
    static constexpr int kRing = 160 * 1024 - 5 * 1024;
    static constexpr int stages(int nsub) { return kRing / stage_bytes(nsub) < 8 ? kRing / stage_bytes(nsub) : 8; }
    static constexpr int kEpiRow = kBN;  // one e4m3 byte per column
};
static_assert(G1F8::kEpiRow * G1F8::kMaxRows + 4 * G1F8::kMaxRows * 4 <= G1F8::kRing,
              "epilogue staging must fit in the ring");
static_assert(G1F8::stages(kMaxRowBlocksFp8G1) >= 2, "ring too small");
static_assert(G1F8::stage_bytes(1) % 16 == 0, "stages 16-byte aligned");

// Row blocks of the task that wave row wm computes: wm, wm + 2, ...
template <int NSUB, int WM>
struct G1F8Rows {
    static constexpr int n = WM == 0 ? (NSUB + 1) / 2 : NSUB / 2;
};

// One K block of the FP8 GEMM-1 for a wave owning NW row blocks
// (2 i + wm, i < NW): MFMAs of each row block against the wave's four B
// fragments (two columns x gate/up), each promoted into acc[i].  The A
// fragment and row scales of block i + 1 are read from LDS while block i's
// MFMAs run; the promotion then waits for block i's results, during which
// the other wave on the SIMD issues its MFMAs (registers do not allow a
// second set of MFMA results in flight).
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
        v8i A = lds_frag32(sa + (16 * wm + lr) * kRowBytes, lg, swz);
        float4 sx = *reinterpret_cast<const float4*>(sc + 16 * wm + 4 * lg);
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            v4f t[2][2];
#pragma unroll
            for (int f = 0; f < 2; ++f)
#pragma unroll
                for (int g = 0; g < 2; ++g) t[f][g] = mfma_fp8(A, Bf[f][g], zero4);
            v8i An = A;
            float4 sxn = sx;
            if (i + 1 < NW) {
                const int s = 2 * (i + 1) + wm;
                An = lds_frag32(sa + (16 * s + lr) * kRowBytes, lg, swz);
                sxn = *reinterpret_cast<const float4*>(sc + 16 * s + 4 * lg);
            }
            __builtin_amdgcn_sched_barrier(0);
            const float sxa[4] = {sx.x, sx.y, sx.z, sx.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float pg = sxa[j] * swg, pu = sxa[j] * swu;
#pragma unroll
                for (int f = 0; f < 2; ++f) {
                    acc[i][f][0][j] += t[f][0][j] * pg;
                    acc[i][f][1][j] += t[f][1][j] * pu;
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            A = An;
            sx = sxn;
        }
    }
}

template <int NSUB>
__device__ __forceinline__ void g1f8_task(const Gemm1Args& g, int e, int row0, int cb, unsigned char* smem,
                                          SchedT<kRowsLdsFp8G1>& sch, const int* rows, int par) {
    using C = G1F8;
    constexpr int S = C::stages(NSUB);
    constexpr int kStage = C::stage_bytes(NSUB);
    constexpr int kStageA = 16 * NSUB * kRowBytes;
    constexpr int kAInstr = 2 * NSUB;  // A loads per stage: 8 rows each
    constexpr int kRows = 16 * NSUB;
    constexpr int kScaleChunks = (kRows + 63) / 64;  // row-scale loads: 64 rows each
    const int K = g.d_h, N_out = g.d_e;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = w >> 2, wn = w & 3;
    const int lr = lane & 15, lg = lane >> 4;
    const int nk = K / 128;
    const unsigned smem_lds = lds_offset(smem);
    const int64_t ld_bytes = K;  // bytes per operand row
    const float* a_scale = static_cast<const float*>(g.x_scale);
    const float* w_scale = static_cast<const float*>(g.w1_scale);
    const bool loader = w < C::kLoaders;
    // vector-memory loads per stage of this wave: B instructions w, w+7, ...,
    // A instructions the same way, row-scale chunk c by wave (c == 0 ? 0 : c + 1),
    // the block scales by wave 1
    const int n_b = loader ? (C::kBAll - 1 - w) / C::kLoaders + 1 : 0;
    const int n_a = loader && w < kAInstr ? (kAInstr - 1 - w) / C::kLoaders + 1 : 0;
    const int my_chunk = w == 0 ? 0 : (w >= 2 ? w - 1 : -1);  // row-scale chunk of this wave, or -1
    const bool s_rows = my_chunk >= 0 && my_chunk < kScaleChunks;
    const int n_s = (s_rows ? 1 : 0) + (w == 1 ? 1 : 0);
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
    unsigned boff[C::kBMax];
#pragma unroll
    for (int j = 0; j < C::kBMax; ++j) {
        const int b = w + C::kLoaders * j;  // B instruction: tile rows 8*b .. 8*b+7
        if (g.packed) {
            boff[j] = (unsigned)((b * 64 + lane) * 16);
        } else {
            const int r = 8 * b + (lane >> 3);
            const int c = (lane & 7) ^ (r & 7);
            const int wrow = r < C::kBN ? cb * C::kBN + r : N_out + cb * C::kBN + (r - C::kBN);
            boff[j] = (unsigned)wrow * (unsigned)ld_bytes + (unsigned)(c * 16);
        }
    }
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
    // row scale of tile row 64 * my_chunk + lane (row 0's past the task's rows
    // and on padding rows), or in wave 1 lanes 0 and 1 the gate and up block
    // scales of W1; byte offsets
    const int kq = K / kQ;
    unsigned soff = 0;
    if (s_rows) {
        const int srow = 64 * my_chunk + lane;
        const int p = srow < kRows ? rows[srow] : -1;
        soff = (unsigned)(p >= 0 ? p / g.k : 0) * (unsigned)(4 * kq);
    }
    unsigned bsoff = 0;
    if (w == 1 && lane < 2) {
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
            if (b < C::kBAll) g2l16s(wbase, boff[j] + kboff, st + (unsigned)(b * 1024));
        }
#pragma unroll
        for (int j = 0; j < C::kAMax; ++j) {
            const int ai = w + C::kLoaders * j;
            if (ai < kAInstr) g2l16s(xbase, aoff[j] + koff, st + (unsigned)(C::kStageB + ai * 1024));
        }
        const unsigned ss = st + (unsigned)(C::kStageB + kStageA);
        if (s_rows) g2l4s(a_scale, soff + 4u * (unsigned)kc, ss + (unsigned)(256 * my_chunk));
        // lanes 0 and 1 only: the other lanes would land past the stage
        if (w == 1 && lane < 2) g2l4s(w_scale, bsoff + 4u * (unsigned)kc, ss + (unsigned)C::kScaleBlk);
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
            g1f8_kblock<NW>(smem + (kc % S) * kStage, kStageA, wm, wn, lr, lg, swz, acc);
        }
        __builtin_amdgcn_s_waitcnt(VmCnt<0>::imm);

        // ---- epilogue: SwiGLU, amax per row over the task's 128 columns
        // (four waves hold 32 columns each), requantisation, staging, stores
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
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int s = 2 * i + wm;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float m = fmaxf(fabsf(hv[i][0][j]), fabsf(hv[i][1][j]));
                m = row16_max(m);  // the 16 lanes of a row group hold one tile row
                if (lr == 0) s_amax[wn * C::kMaxRows + 16 * s + 4 * lg + j] = m;
            }
        }
        lds_barrier();
        float* hs = static_cast<float*>(g.h_scale);
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int s = 2 * i + wm;
            float4 m = *reinterpret_cast<const float4*>(&s_amax[16 * s + 4 * lg]);
#pragma unroll
            for (int ww = 1; ww < 4; ++ww) {
                const float4 o = *reinterpret_cast<const float4*>(&s_amax[ww * C::kMaxRows + 16 * s + 4 * lg]);
                m = make_float4(fmaxf(m.x, o.x), fmaxf(m.y, o.y), fmaxf(m.z, o.z), fmaxf(m.w, o.w));
            }
            const float am4[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int rr = 16 * s + 4 * lg + j;
                const float am = am4[j];
                // scale amax/448; values are multiplied by its reciprocal
                const float sc = am > 0.f ? am * (1.0f / 448.0f) : 1.0f;
                const float inv = am > 0.f ? 448.0f * __builtin_amdgcn_rcpf(am) : 1.0f;
                const unsigned q2 =
                    (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(hv[i][0][j] * inv, hv[i][1][j] * inv, 0, false);
                stage[rr * C::kEpiRow + 32 * wn + lr] = (unsigned char)(q2 & 0xffu);
                stage[rr * C::kEpiRow + 32 * wn + 16 + lr] = (unsigned char)((q2 >> 8) & 0xffu);
                if (wn == 0 && lr == 0) hs[(int64_t)(row0 + rr) * (N_out / kQ) + cb] = sc;
            }
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

__global__ __launch_bounds__(kGemm1Fp8Threads) void gemm1_fp8_kernel(Gemm1Args a) {
    __shared__ __attribute__((aligned(16))) unsigned char smem[G1F8::kRing];
    __shared__ QueueLdsT<kRowsLdsFp8G1> q;
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
#define MOE_G1F8(NS) g1f8_task<NS>(a, e, row0, cb, smem, sch, q.rows[par], par)
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
    if (mode == MOE_MODE_MXFP8)
        hipExtLaunchKernelGGL(gemm1_kernel<MOE_MODE_MXFP8>, dim3(grid), dim3(kGemmThreads), 0, s, t0, t1, 0, a);
    else if (mode == MOE_MODE_FP8 && wide)
        hipExtLaunchKernelGGL(gemm1_fp8_kernel, dim3(grid), dim3(kGemm1Fp8Threads), 0, s, t0, t1, 0, a);
    else if (mode == MOE_MODE_FP8)
        hipExtLaunchKernelGGL(gemm1_kernel<MOE_MODE_FP8>, dim3(grid), dim3(kGemmThreads), 0, s, t0, t1, 0, a);
    else
        hipExtLaunchKernelGGL(gemm1_kernel<MOE_MODE_BF16>, dim3(grid), dim3(kGemmThreads), 0, s, t0, t1, 0, a);
    return hipGetLastError();
}

hipError_t launch_gemm2(int mode, const Gemm2Args& a, int grid, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
    if (mode == MOE_MODE_MXFP8)
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
        e1 = hipOccupancyMaxActiveBlocksPerMultiprocessor(g1, gemm1_kernel<MOE_MODE_MXFP8>, kGemmThreads, 0);
        e2 = hipOccupancyMaxActiveBlocksPerMultiprocessor(g2, gemm2_kernel<MOE_MODE_MXFP8>, kGemmThreads, 0);
    } else if (mode == MOE_MODE_FP8) {
        e1 = wide ? hipOccupancyMaxActiveBlocksPerMultiprocessor(g1, gemm1_fp8_kernel, kGemm1Fp8Threads, 0)
                  : hipOccupancyMaxActiveBlocksPerMultiprocessor(g1, gemm1_kernel<MOE_MODE_FP8>, kGemmThreads, 0);
        e2 = hipOccupancyMaxActiveBlocksPerMultiprocessor(g2, gemm2_kernel<MOE_MODE_FP8>, kGemmThreads, 0);
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
