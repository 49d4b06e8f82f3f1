// Device building blocks of the grouped expert GEMMs (internal header of the
// fused MoE library, included by the kernel translation units; not installed).
//
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
#pragma once

#include <algorithm>
#include <type_traits>

#include "moe_internal.h"

namespace moe {
// Each including translation unit gets its own copy of these device helpers.
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
    // format 0 = E4M3 for both operands, no MX scaling.  With zero scale
    // operands clang lowers this builtin to the unscaled
    // v_mfma_f32_16x16x128_f8f6f4 (it has no builtin of its own), which is
    // about a tenth faster on gfx950 than the scaled form with unit (127)
    // scales and gives bit-identical results; the FP8 parity tests against
    // the oracle pin that lowering
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
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

// two binary32 -> bf16 in one v_cvt_pk_bf16_f32 (round to nearest even, as
// f32_to_bf16 for every finite value): a in the low half, b in the high half
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned pk_bf16(float a, float b) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
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
// Device-scope (sc1) forms, for data that another workgroup of the same launch
// wrote, possibly on another XCD: an sc1 access is coherent across the XCDs'
// L2 caches by itself (the compiler's own lowering of a relaxed agent-scope
// atomic load or store is exactly this bit), so neither a writeback of the
// producer's L2 nor an invalidation of the consumer's is needed.
__device__ __forceinline__ void g2l16c(const void* g, unsigned lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off sc1" ::"s"(lds), "v"(g)
                 : "memory", "m0");
}
__device__ __forceinline__ void g2l4c(const void* g, unsigned lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off sc1" ::"s"(lds), "v"(g)
                 : "memory", "m0");
}
// 16-byte vector store, device scope (written through to where every XCD reads it)
template <typename V>
__device__ __forceinline__ void st16c(void* g, const V& v) {
    static_assert(sizeof(V) == 16, "16-byte store");
    asm volatile("global_store_dwordx4 %0, %1, off sc1" ::"v"(g), "v"(v) : "memory");
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
template <int MODE, bool GATED, bool Y32 = false>
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
    // y rows: fp32 with fp32 activations or Y32 (the single launch keeps y in fp32), else bf16
    static constexpr int kOutBytes = ((MODE == MOE_MODE_F32ACT || Y32) && !GATED) ? 4 : (GATED && kFP8 ? 1 : 2);
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
// Single-launch form (FUSED): the task runs inside the one persistent grid of
// the layer (tilelang.dataflow README section 3.5: GEMM-1 and GEMM-2 under one
// wrapper launch, the dependency resolved without a kernel boundary).  GEMM-1
// stores h (and its scales) with device-scope stores, waits for them, then adds
// 1 to the counter of the GEMM-2 M-tile its rows belong to.  GEMM-2 first
// requests its weight stages, waits (bounded) until that counter reaches every
// column block of every GEMM-1 M-tile in it, then loads h with device-scope
// loads; it keeps y in fp32 and, once its y stores are complete, adds 1 per
// row to the arrival counter of the row's (token, column block), which the
// layer kernel's combine waits on.
struct FusedCtx {
    int32_t* done;      // this task's GEMM-2 M-tile counter: GEMM-1 column blocks that stored their h rows
    int32_t target;     // GEMM-2: the count that means all of its h rows are stored
    int32_t* timeouts;  // waits that ran out (diagnostic; each such task went on)
    int32_t* arrive;    // [token * nb2 + column block]: y rows stored
    int32_t k, nb2;
};
// polls of a bounded wait (each a device-scope load and a short sleep):
// far longer than any GEMM-1 task, so only a broken schedule reaches it
constexpr int kSpinLimit = 1 << 18;

template <int MODE, bool GATED, int NSUB, int RING, bool FUSED = false, class SCH = Sched>
__device__ __forceinline__ void gemm_task(const void* a_base, const void* a_scale_v, const int32_t* row_src,
                                          int a_div, const void* wts, const void* w_scale_v, const unsigned char* zero,
                                          int e, int row0, int cb, int K, int N_out, bool packed,
                                          unsigned char* smem, const Gemm1Args* g1, const Gemm2Args* g2,
                                          SCH& sch, const int* rows, const float* roww, int par,
                                          const FusedCtx* fx = nullptr, bool h_ready = false) {
    using C = Cfg<MODE, GATED, FUSED && !GATED>;
    constexpr bool kFP8 = C::kFP8, kBS = C::kBS, kMX = C::kMX;
    // single-launch GEMM-2: h is read at device scope, and unless it was
    // already complete when the task was claimed, the weight loads go first
    // and the h loads after the wait
    constexpr bool kSplit = FUSED && !GATED;
    const bool split = kSplit && !h_ready;
    const float* a_scale = static_cast<const float*>(a_scale_v);  // FP8 mode
    const float* w_scale = static_cast<const float*>(w_scale_v);
    constexpr int S = C::stages(NSUB, RING);
    static_assert(C::stages(NSUB, RING) >= 2, "ring too small for two stages of this task");
    static_assert(C::kEpiRow * kAMaxRows + kGemmWaves * kAMaxRows * 4 <= RING, "epilogue staging must fit in the ring");
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
    const int loads_a = n_a + n_s;  // the part of a stage that reads the A operand and the scales

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
    const bool w_owner = GATED && !FUSED && cb == 0 && w < 2 && w_row < kRows;
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

    // a stage's loads: the weight rows (issue_b), then the A rows and the
    // scales (issue_a); a single-launch GEMM-2 reads the latter at device scope
    auto issue_b = [&](int kc) {
        const unsigned st = smem_lds + (unsigned)((kc % S) * kStage);
        const int64_t boff = (int64_t)kc * b_step;
        if (!loader) return;
#pragma unroll
        for (int j = 0; j < C::kBMax; ++j) {
            const int b = w + kLoadWaves * j;
            if (b < C::kBAll) g2l16(bsrc[j] + boff, st + (unsigned)(b * 1024));
        }
    };
    auto issue_a = [&](int kc) {
        const unsigned st = smem_lds + (unsigned)((kc % S) * kStage);
        const int64_t koff = (int64_t)kc * kRowBytes;
        if (!loader) return;
        auto ld16 = [&](const void* g, unsigned l) {
            if constexpr (kSplit) g2l16c(g, l); else g2l16(g, l);
        };
        auto ld4 = [&](const void* g, unsigned l) {
            if constexpr (kSplit) g2l4c(g, l); else g2l4(g, l);
        };
#pragma unroll
        for (int j = 0; j < kAMaxPerWave; ++j) {
            const int ai = w + kLoadWaves * j;
            if (ai < kAInstr) ld16(apad[j] ? asrc[j] : asrc[j] + koff, st + (unsigned)(C::kStageB + ai * 1024));
        }
        if constexpr (kBS) {
            // wave 0 reads the row scales, wave 1 the weights' block scales
            const unsigned ss = st + (unsigned)(C::kStageB + kStageA);
            if (son) ld4(spad ? ssrc : ssrc + kc, ss + (unsigned)(w == 1 ? 512 : w * 128));
        }
        if constexpr (kMX) {
            const unsigned ss = st + (unsigned)(C::kStageB + kStageA);
#pragma unroll
            for (int m = 0; m < 2; ++m)
                if (mon[m]) ld4(mfix[m] ? msrc[m] : msrc[m] + 4 * kc, ss + mdst[m]);
        }
    };
    auto issue = [&](int kc) {
        issue_b(kc);
        issue_a(kc);
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
    if (split) {
        for (int kc = 0; kc < npro; ++kc) issue_b(kc);
        // the scheduler wave (no stage loads of its own) waits until every
        // GEMM-1 column block of this M-tile has stored its h rows
        if (w == kSchedWave) {
            for (int it = 0;; ++it) {
                const int v = __builtin_amdgcn_readfirstlane(
                    __hip_atomic_load(fx->done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
                if (v >= fx->target) break;
                if (it >= kSpinLimit) {
                    if (lane == 0) __hip_atomic_fetch_add(fx->timeouts, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        lds_barrier();
        for (int kc = 0; kc < npro; ++kc) issue_a(kc);
    } else {
        for (int kc = 0; kc < npro; ++kc) issue(kc);
    }
    const int claim_at = nk > kClaimLead ? nk - kClaimLead : 0;
    const int settle_at = nk > kClaimLead - 2 ? nk - (kClaimLead - 2) : 0;
    const int rows_at = nk > kClaimLead - 4 ? nk - (kClaimLead - 4) : 0;
    for (int kc = 0; kc < nk; ++kc) {
        // stage kc is complete once at most the younger stages' loads remain
        // (each loading wave waits for its own; the barrier covers the rest)
        if (loader) {
            int younger;
            if (split && kc < npro) {
                // the prologue's A parts went out after all its weight parts:
                // younger than stage kc are the A parts of the later prologue
                // stages and the whole stages issued since
                const int whole = kc < nk - npro ? kc : nk - npro;
                younger = (npro - 1 - kc) * loads_a + whole * loads_per_stage;
            } else {
                younger = ((nk - 1 - kc) < (S - 2) ? (nk - 1 - kc) : (S - 2)) * loads_per_stage;
            }
            wait_vm_le(younger);
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
                    if (lr == 0) {
                        uint8_t* dst = hs + (int64_t)(row0 + rr) * (N_out / 32) + cb * kGemmWaves + w;
                        if constexpr (FUSED)
                            __hip_atomic_store(dst, (uint8_t)b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        else
                            *dst = (uint8_t)b;
                    }
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
                    if (w == 0 && lr == 0) {
                        float* dst = static_cast<float*>(g1->h_scale) + (int64_t)(row0 + rr) * (N_out / kQ) + cb;
                        if constexpr (FUSED)
                            __hip_atomic_store(dst, sc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        else
                            *dst = sc;
                    }
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
                unsigned char* dst = h + (int64_t)(row0 + r) * hrow_bytes + (int64_t)cb * C::kEpiRow + c * 16;
                const v4i v = *reinterpret_cast<const v4i*>(stage + r * C::kEpiRow + c * 16);
                if constexpr (FUSED)
                    st16c(dst, v);
                else
                    *reinterpret_cast<v4i*>(dst) = v;
            }
    } else {
        constexpr bool kF32 = MODE == MOE_MODE_F32ACT || FUSED;
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
                unsigned char* dst = y + (int64_t)p * yrow_bytes + (int64_t)cb * C::kEpiRow + c * 16;
                const v4i v = *reinterpret_cast<const v4i*>(stage + r * C::kEpiRow + c * 16);
                if constexpr (FUSED)
                    st16c(dst, v);
                else
                    *reinterpret_cast<v4i*>(dst) = v;
            }
    }
    // single launch: this task's stores of h (and its scales) or y are complete
    // before it is counted
    if constexpr (FUSED) __builtin_amdgcn_s_waitcnt(VmCnt<0>::imm);
    if (w == kSchedWave) sch.publish();
    lds_barrier();  // the ring and the staging area are refilled by the next task
    if constexpr (FUSED) {
        if constexpr (GATED) {
            if (threadIdx.x == 0) __hip_atomic_fetch_add(fx->done, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else if (threadIdx.x < 16 * NSUB) {
            const int p = rows[threadIdx.x];
            if (p >= 0)
                __hip_atomic_fetch_add(fx->arrive + (int64_t)(p / fx->k) * fx->nb2 + cb, 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace
}  // namespace moe
