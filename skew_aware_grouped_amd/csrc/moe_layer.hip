// The fused MoE layer in one persistent launch (moe_dims.launch =
// MOE_LAUNCH_SINGLE): routing, GEMM-1 with the activation, GEMM-2 with the
// routing weights and the top-k combine, with no kernel boundary between them
// (tilelang.dataflow README, section 3.5: GEMM-1 and GEMM-2 execute under one
// wrapper launch, so their dependency needs no kernel barrier; section 1 names
// what kernel boundaries cost: idle SMs, tails and launch overhead).
//
// Every workgroup first derives the routing plan itself, in LDS, from the ids
// (section 3.5 step 1: group sizes, padded offsets, the expert of each group
// block): the batches this form serves have at most kLayerMaxN assignments, so
// reading them all per workgroup costs less than any grid-wide step.  The plan:
//   counts per expert, 16-row group blocks, padded offsets in expert order (h
//   rows live there, as in the four-launch layout), M-tiles of MT group blocks,
//   experts ranked by descending count (ties by id), and one task list: every
//   GEMM-1 task (rank, column block, M-tile), then every GEMM-2 task in the same
//   order.
// Tasks are claimed in list order from one queue counter (the claim for a
// workgroup's next task goes out during its current task's last K blocks).
// GEMM-1 tasks never wait; a GEMM-2 task waits only on the GEMM-1 tasks of its
// M-tile, all of lower index.  So the lowest unfinished claimed task can
// always proceed, whether or not every workgroup of the grid is resident, and
// each wait is bounded anyway.  The protocol (with the combine and the exit
// reset described at FusedCtx and in the kernel) is modelled on the CPU and
// checked there for coverage, dependency order and termination.
//
// The rows of a task are found by the scheduler wave: a ballot scan of the ids
// kept in LDS (rank of each assignment within its expert, ascending p).
#include "moe_gemm_task.h"

namespace moe {
namespace {

// routing plan of the call, the same in every workgroup
struct FusedPlan {
    uint64_t bad[kLayerMaxN / 64];    // bit p: assignment p's id is outside [0, E) (or p >= N)
    unsigned char id8[kLayerMaxN];    // low 8 bits of each id (E <= 256)
    short cnt[kMaxExperts];           // rows routed to each expert
    short poff[kMaxExperts + 2];      // padded offsets, expert order
    short moff[kMaxExperts + 2];      // M-tiles of the ranks before each rank
    unsigned char order[kMaxExperts]; // expert of each rank
};

// the workgroup's current task and the rows of the current and next task
struct FusedQ {
    int slot;
    int list;  // 0: GEMM-1, 1: GEMM-2
    int pad[2];
    int4 task;  // {expert, first padded row, row blocks, column block}
    int rows[2][kRowsLds];
    float roww[2][kRowsLds];
};

// ring of the layer kernel: the larger of its two GEMMs' rings, less what the
// plan and the queue state take (two workgroups per CU in the bf16 modes, one
// in the FP8 ones)
template <int MODE>
struct LayerCfg {
    static constexpr int kMT = mode_fp8(MODE) ? kSmallRowBlocks : kMaxRowBlocks1;
    static constexpr int kRing = mode_fp8(MODE) ? 153 * 1024 : Cfg<MODE, true>::kRing;
    static_assert(kRing + (int)sizeof(FusedPlan) + (int)sizeof(FusedQ) <= (mode_fp8(MODE) ? 160 : 80) * 1024,
                  "LDS budget");
};

// Largest r in [0, n) with off[r] <= v (off non-decreasing, v < off[n]):
// never an entry without tasks
__device__ __forceinline__ int upper_rank(const short* off, int n, int v) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= v)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Scheduler of the single launch; the interface gemm_task drives (claim on
// lane 0, then settle, load_rows and publish on the scheduler wave).
struct FusedSched {
    int32_t* queue;
    const FusedPlan* pl;
    FusedQ* q;
    const float* topk_w;
    int total, n1, nb1, nb2, mtb, E, Np;
    int raw = -1;  // lane 0: the claimed index
    int slot = -1;
    int e = 0, row0 = 0, nsub = 0, cb = 0, m = 0, list = 0;

    __device__ __forceinline__ void claim() {
        raw = __hip_atomic_fetch_add(queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __device__ __forceinline__ void settle(bool) {
        int s = __builtin_amdgcn_readfirstlane(raw);
        slot = (s >= 0 && s < total) ? s : -1;
        if (slot < 0) return;
        list = slot < n1 ? 0 : 1;
        const int j = list ? slot - n1 : slot;
        const int nb = list ? nb2 : nb1;
        const int r = upper_rank(pl->moff, E, j / nb);
        const int mt = pl->moff[r + 1] - pl->moff[r];
        const int local = j - pl->moff[r] * nb;
        cb = local / mt;
        m = local - cb * mt;
        e = pl->order[r];
        const int tiles = (pl->cnt[e] + kBlockM - 1) / kBlockM;
        row0 = pl->poff[e] + kBlockM * mtb * m;
        nsub = min(mtb, tiles - mtb * m);
    }
    // rows of the task: ranks [lo, lo + 16 nsub) of expert e's assignments
    // (ascending p), -1 past its count; GEMM-2 also its routing weights
    __device__ __forceinline__ void load_rows(int par) {
        if (slot < 0) return;
        const int lane = threadIdx.x & 63;
        int* rows = q->rows[par];
        const int lo = kBlockM * mtb * m, n = kBlockM * nsub;
        const int cnt = pl->cnt[e];
        const int hi = min(lo + n, cnt);
        const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
        int base = 0;
        for (int p0 = 0; p0 < Np && base < hi; p0 += 256) {
            const int p = p0 + 4 * lane;
            const unsigned w4 = *reinterpret_cast<const unsigned*>(&pl->id8[p]);
            const unsigned b4 = (unsigned)(pl->bad[p >> 6] >> (p & 63)) & 0xFu;
            unsigned mine = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                mine |= ((((w4 >> (8 * i)) & 0xFFu) == (unsigned)e) && !((b4 >> i) & 1u)) ? (1u << i) : 0u;
            int below = 0, all = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint64_t bal = __ballot((mine >> i) & 1u);
                below += __popcll(bal & lt);
                all += __popcll(bal);
            }
            int r = base + below;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if ((mine >> i) & 1u) {
                    if (r >= lo && r < hi) rows[r - lo] = p + i;
                    ++r;
                }
            base += all;
        }
        for (int r = lane; r < n; r += 64)
            if (lo + r >= cnt) rows[r] = -1;
        if (list == 1) {
            // routing weight of each row (direct-to-LDS; padding rows read entry 0, never used)
            for (int j = 0; j < n; j += 64) {
                const int p = j + lane < n ? rows[j + lane] : -1;
                g2l4(topk_w + (p > 0 ? p : 0), lds_offset(&q->roww[par][j]));
            }
        }
    }
    __device__ __forceinline__ void publish() {
        __builtin_amdgcn_s_waitcnt(VmCnt<0>::imm);
        asm volatile("" ::: "memory");
        if ((threadIdx.x & 63) == 0) {
            q->slot = slot;
            q->list = list;
            if (slot >= 0) q->task = make_int4(e, row0, nsub, cb);
        }
    }
};

template <int MODE>
__global__ __launch_bounds__(kGemmThreads) void layer_kernel(LayerArgs a) {
    using L = LayerCfg<MODE>;
    constexpr int RING = L::kRing;
    constexpr int MT = L::kMT;
    __shared__ __attribute__((aligned(16))) unsigned char smem[RING];
    __shared__ FusedQ q;
    __shared__ FusedPlan pl;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int N = a.N, E = a.E, k = a.k;
    const int Np = (N + 255) / 256 * 256;
    int32_t* sync = a.sync;
    const unsigned char* zero = reinterpret_cast<const unsigned char*>(sync + kSyncZero);

    FusedSched sch0{sync + kSyncQueue, &pl, &q, a.g1.topk_w, 0, 0, a.nb1, a.nb2, MT, E, Np};
    // the first claim goes out before the plan is built
    if (w == kSchedWave && lane == 0) sch0.claim();

    // ---- plan: ids into LDS, histogram (in the ring, free until the first task)
    int* hist = reinterpret_cast<int*>(smem);
    for (int i = tid; i < E; i += kGemmThreads) hist[i] = 0;
    lds_barrier();
    for (int p0 = 64 * w; p0 < Np; p0 += 64 * kGemmWaves) {
        const int p = p0 + lane;
        const int id = p < N ? a.ids[p] : -1;
        const bool ok = (unsigned)id < (unsigned)E;
        pl.id8[p] = (unsigned char)(ok ? id : 0);
        const uint64_t badm = __ballot(!ok);
        if (lane == 0) pl.bad[p0 >> 6] = badm;
        if (ok) atomicAdd(&hist[id], 1);
    }
    lds_barrier();
    // counts, then each expert's rank (descending count, ties by id)
    for (int e = tid; e < E; e += kGemmThreads) {
        const int c = hist[e];
        pl.cnt[e] = (short)c;
        int r = 0;
        for (int f = 0; f < E; ++f) {
            const int cf = hist[f];
            r += (cf > c) || (cf == c && f < e);
        }
        pl.order[r] = (unsigned char)e;
    }
    lds_barrier();
    // padded offsets (expert order) and M-tile offsets (rank order): one wave each
    if (w < 2) {
        int run = 0;
        for (int i0 = 0; i0 < E; i0 += 64) {
            const int i = i0 + lane;
            int v = 0;
            if (i < E) {
                const int tiles = (hist[w == 0 ? i : pl.order[i]] + kBlockM - 1) / kBlockM;
                v = w == 0 ? kBlockM * tiles : (tiles + MT - 1) / MT;
            }
            int incl = v;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int o = __shfl_up(incl, d, 64);
                if (lane >= d) incl += o;
            }
            if (i < E) (w == 0 ? pl.poff : pl.moff)[i] = (short)(run + incl - v);
            run += __shfl(incl, 63, 64);
        }
        if (lane == 0) (w == 0 ? pl.poff : pl.moff)[E] = (short)run;
    }
    lds_barrier();
    const int n_mt = pl.moff[E];
    const int n1 = n_mt * a.nb1, total = n1 + n_mt * a.nb2;

    // tokens without a valid slot: zero output rows (token t by workgroup t mod grid)
    for (int t = blockIdx.x; t < a.T; t += gridDim.x) {
        bool none = true;
        for (int j = 0; j < k; ++j) {
            const int p = t * k + j;
            none = none && ((pl.bad[p >> 6] >> (p & 63)) & 1ull);
        }
        if (none) {
            uint4* dst = reinterpret_cast<uint4*>(static_cast<unsigned short*>(a.out) + (int64_t)t * a.g1.d_h);
            for (int c = tid; c < a.g1.d_h / 8; c += kGemmThreads) dst[c] = make_uint4(0u, 0u, 0u, 0u);
        }
    }

    // ---- the first task
    if (w == kSchedWave) {
        sch0.total = total;
        sch0.n1 = n1;
        sch0.settle(true);
        sch0.load_rows(0);
        sch0.publish();
    }
    lds_barrier();

    FusedCtx fx{sync + kSyncDone, sync + kSyncArrive, sync + kSyncTimeouts, pl.bad, a.out, a.nb1, a.nb2, k,
                a.g1.d_h};
    for (int par = 0;; par ^= 1) {
        // uniform task fields (readfirstlane: see gemm1_kernel)
        const int t = __builtin_amdgcn_readfirstlane(q.slot);
        if (t < 0) break;
        const int list = __builtin_amdgcn_readfirstlane(q.list);
        const int e = __builtin_amdgcn_readfirstlane(q.task.x), row0 = __builtin_amdgcn_readfirstlane(q.task.y);
        const int nsub = __builtin_amdgcn_readfirstlane(q.task.z), cb = __builtin_amdgcn_readfirstlane(q.task.w);
        FusedSched sch{sync + kSyncQueue, &pl, &q, a.g1.topk_w, total, n1, a.nb1, a.nb2, MT, E, Np};
        const int* rows = q.rows[par];
        const float* roww = q.roww[par];
#define MOE_L1(NS)                                                                                                 \
    gemm_task<MODE, true, NS, RING, true, FusedSched>(a.g1.x, a.g1.x_scale, nullptr, k, a.g1.w1, a.g1.w1_scale,     \
                                                      zero, e, row0, cb, a.g1.d_h, a.g1.d_e, a.g1.packed != 0,     \
                                                      smem, &a.g1, nullptr, sch, rows, roww, par, &fx)
#define MOE_L2(NS)                                                                                                 \
    gemm_task<MODE, false, NS, RING, true, FusedSched>(a.g2.h, a.g2.h_scale, nullptr, 1, a.g2.w2, a.g2.w2_scale,   \
                                                       zero, e, row0, cb, a.g2.d_e, a.g2.d_h, a.g2.packed != 0,    \
                                                       smem, nullptr, &a.g2, sch, rows, roww, par, &fx)
        // one body per row-block count (M-tiles of MT blocks: nsub in [1, MT])
        if (list == 0) {
            if constexpr (MT == 8) {
                switch (nsub) {
                    case 1: MOE_L1(1); break;
                    case 2: MOE_L1(2); break;
                    case 3: MOE_L1(3); break;
                    case 4: MOE_L1(4); break;
                    case 5: MOE_L1(5); break;
                    case 6: MOE_L1(6); break;
                    case 7: MOE_L1(7); break;
                    default: MOE_L1(8); break;
                }
            } else {
                switch (nsub) {
                    case 1: MOE_L1(1); break;
                    case 2: MOE_L1(2); break;
                    case 3: MOE_L1(3); break;
                    default: MOE_L1(4); break;
                }
            }
        } else {
            if constexpr (MT == 8) {
                switch (nsub) {
                    case 1: MOE_L2(1); break;
                    case 2: MOE_L2(2); break;
                    case 3: MOE_L2(3); break;
                    case 4: MOE_L2(4); break;
                    case 5: MOE_L2(5); break;
                    case 6: MOE_L2(6); break;
                    case 7: MOE_L2(7); break;
                    default: MOE_L2(8); break;
                }
            } else {
                switch (nsub) {
                    case 1: MOE_L2(1); break;
                    case 2: MOE_L2(2); break;
                    case 3: MOE_L2(3); break;
                    default: MOE_L2(4); break;
                }
            }
        }
#undef MOE_L1
#undef MOE_L2
    }

    // ---- exit: every memory operation of this workgroup is complete, then
    // it is counted; the last one resets the queue, the exit counter and the
    // M-tile counters for the next call
    __builtin_amdgcn_s_waitcnt(VmCnt<0>::imm);
    int* s_last = reinterpret_cast<int*>(smem);
    lds_barrier();
    if (tid == 0) {
        const int old = __hip_atomic_fetch_add(sync + kSyncExit, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_last = old == (int)gridDim.x - 1;
    }
    lds_barrier();
    if (*s_last) {
        const int n_blocks = pl.poff[E] / kBlockM;
        for (int i = tid; i < n_blocks; i += kGemmThreads)
            __hip_atomic_store(sync + kSyncDone + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (tid == 0) {
            __hip_atomic_store(sync + kSyncQueue, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(sync + kSyncExit, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

__global__ __launch_bounds__(256) void sync_clear_kernel(int32_t* sync) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < kSyncWords; i += gridDim.x * blockDim.x) sync[i] = 0;
}

}  // namespace

hipError_t launch_layer(int mode, const LayerArgs& a, int grid, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
    if (mode == MOE_MODE_FP8)
        hipExtLaunchKernelGGL(layer_kernel<MOE_MODE_FP8>, dim3(grid), dim3(kGemmThreads), 0, s, t0, t1, 0, a);
    else if (mode == MOE_MODE_MXFP8)
        hipExtLaunchKernelGGL(layer_kernel<MOE_MODE_MXFP8>, dim3(grid), dim3(kGemmThreads), 0, s, t0, t1, 0, a);
    else
        hipExtLaunchKernelGGL(layer_kernel<MOE_MODE_BF16>, dim3(grid), dim3(kGemmThreads), 0, s, t0, t1, 0, a);
    return hipGetLastError();
}

hipError_t layer_occupancy(int mode, int* blocks) {
    if (mode == MOE_MODE_FP8)
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, layer_kernel<MOE_MODE_FP8>, kGemmThreads, 0);
    if (mode == MOE_MODE_MXFP8)
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, layer_kernel<MOE_MODE_MXFP8>, kGemmThreads, 0);
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, layer_kernel<MOE_MODE_BF16>, kGemmThreads, 0);
}

hipError_t launch_sync_clear(int32_t* sync, hipStream_t s) {
    hipLaunchKernelGGL(sync_clear_kernel, dim3(64), dim3(256), 0, s, sync);
    return hipGetLastError();
}

}  // namespace moe
