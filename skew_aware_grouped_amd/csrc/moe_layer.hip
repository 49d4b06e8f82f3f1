// The fused MoE layer in one persistent launch (moe_dims.launch =
// MOE_LAUNCH_SINGLE): routing, GEMM-1 with the activation, GEMM-2 with the
// routing weights and the top-k combine, with no kernel boundary between them
// (tilelang.dataflow README, section 3.5: GEMM-1 and GEMM-2 execute under one
// wrapper launch, so their dependency needs no kernel barrier; section 1 names
// what kernel boundaries cost: idle SMs, tails and launch overhead).
//
// Every workgroup first derives the routing plan itself, in LDS, from the ids
// (section 3.5 step 1: group sizes, padded offsets, the expert of each group
// block, and the stable scatter): the batches this form serves have at most
// kLayerMaxN assignments, so reading them all per workgroup costs less than
// any grid-wide step.  The plan: counts per expert, 16-row group blocks,
// padded offsets in expert order (h rows live there, as in the four-launch
// layout), the assignment of every padded row, M-tiles of group blocks,
// experts ranked by descending count (ties by id: the longest work first),
// and one task list: every GEMM-1 task, then every GEMM-2 task, each by
// rank, then column block, then M-tile.
// Tasks are claimed in list order from one queue counter (the claim for a
// workgroup's next task goes out during its current task's last K blocks).
// GEMM-1 tasks never wait; a GEMM-2 task waits only on the GEMM-1 tasks of its
// M-tile, all of lower index.  So the lowest unfinished claimed task can
// always proceed, whether or not every workgroup of the grid is resident, and
// each wait is bounded anyway.  After its y stores, a GEMM-2 task counts each
// row's arrival at (token, column block).  The combine comes last: once its
// queue is empty, workgroup b sums the (token, column block) outputs b, b +
// grid, ..., waiting (bounded) until each has all its arrivals; those come
// from GEMM-2 tasks, every one of them already claimed.  The protocol is
// modelled on the CPU and checked there for coverage, dependency order and
// termination.
#include "moe_gemm_task.h"
#include "moe_wave.h"

namespace moe {
namespace {

// routing plan of the call, the same in every workgroup
struct FusedPlan {
    uint64_t bad[kLayerMaxN / 64];                          // bit p: id of p outside [0, E) (or p >= N)
    int row_src[kLayerMaxN + kMaxExperts * (kBlockM - 1)];  // padded rows: assignment p, -1 on padding
    int poff[kMaxExperts + 2];                              // padded offsets, expert order
    int moff[2][kMaxExperts + 2];                           // per GEMM: M-tiles of the ranks before each rank
    short cnt[kMaxExperts];                                 // rows routed to each expert
    unsigned char order[kMaxExperts];                       // expert of each rank
};

// the workgroup's current task and the routing weights of the current and next task's rows
struct FusedQ {
    int slot;
    int list;   // 0: GEMM-1, 1: GEMM-2
    int ready;  // GEMM-2: its h was complete when the task was claimed
    int pad;
    int4 task;  // {expert, first padded row, row blocks, column block}
    float roww[2][kRowsLds];
};

// One workgroup per CU in every mode: the ring takes what the plan and the
// queue state leave of the CU's LDS (up to eight stages of a one-block bf16
// task, three of a 64-row FP8 GEMM-1 task): the loads a workgroup keeps in
// flight are what bounds its streaming rate.
//
// M-tiles in group blocks: GEMM-1 128 rows in the bf16 modes, 64 in the FP8
// ones (their requantising epilogue costs more per row at 128); GEMM-2 always
// 128 rows, so a GEMM-2 M-tile holds one or two GEMM-1 M-tiles, aligned.
template <int MODE>
struct LayerCfg {
    static constexpr int kMT1 = mode_fp8(MODE) ? kSmallRowBlocks : kMaxRowBlocks1;
    static constexpr int kMT2 = kMaxRowBlocks2;
    static_assert(kMT2 % kMT1 == 0, "GEMM-1 M-tiles nest in GEMM-2 M-tiles");
    static constexpr int kRing = 131 * 1024;
    static_assert(kRing + (int)sizeof(FusedPlan) + (int)sizeof(FusedQ) <= 160 * 1024, "LDS budget");
};

// Largest r in [0, n) with off[r] <= v (off non-decreasing, v < off[n]):
// never an entry without tasks
__device__ __forceinline__ int upper_rank(const int* off, int n, int v) {
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
    const int32_t* done1;
    const FusedPlan* pl;
    FusedQ* q;
    const float* topk_w;
    int n1, total, nb1, nb2, mt1, mt2, E;
    int raw = -1;  // lane 0: the claimed index
    int slot = -1;
    int e = 0, row0 = 0, nsub = 0, cb = 0, list = 0, done = 0, need = 0;

    __device__ __forceinline__ void claim() {
        raw = __hip_atomic_fetch_add(queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // GEMM-1 column blocks that store the h rows of a GEMM-2 M-tile of ns
    // group blocks: every column block of each GEMM-1 M-tile in it
    __device__ __forceinline__ int done_target(int ns) const { return nb1 * ((ns + mt1 - 1) / mt1); }
    __device__ __forceinline__ void settle(bool) {
        const int s = __builtin_amdgcn_readfirstlane(raw);
        slot = (s >= 0 && s < total) ? s : -1;
        if (slot < 0) return;
        // list 0 (GEMM-1) or 1 (GEMM-2); rank r owns the list's tasks
        // [moff[r] * nb, moff[r + 1] * nb): column blocks, each with its
        // M-tiles next to each other
        list = slot < n1 ? 0 : 1;
        const int j = list ? slot - n1 : slot;
        const int nb = list ? nb2 : nb1;
        const int* moff = pl->moff[list];
        const int r = upper_rank(moff, E, j / nb);
        const int mt = moff[r + 1] - moff[r];
        const int local = j - moff[r] * nb;
        cb = local / mt;
        const int m = local - cb * mt;
        e = pl->order[r];
        const int mtb = list ? mt2 : mt1;
        const int tiles = (pl->cnt[e] + kBlockM - 1) / kBlockM;
        row0 = pl->poff[e] + kBlockM * mtb * m;
        nsub = min(mtb, tiles - mtb * m);
        if (list == 1) {
            need = done_target(nsub);
            done = __hip_atomic_load(done1 + row0 / kBlockM, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    // the task's rows are the plan's padded rows [row0, row0 + 16 nsub); a
    // GEMM-2 task also needs their routing weights (direct-to-LDS; padding
    // rows read entry 0, never used)
    __device__ __forceinline__ void load_rows(int par) {
        if (slot < 0 || list != 1) return;
        const int lane = threadIdx.x & 63;
        const int n = kBlockM * nsub;
        for (int j = 0; j < n; j += 64) {
            const int p = j + lane < n ? pl->row_src[row0 + j + lane] : -1;
            g2l4(topk_w + (p > 0 ? p : 0), lds_offset(&q->roww[par][j]));
        }
    }
    __device__ __forceinline__ void publish() {
        __builtin_amdgcn_s_waitcnt(VmCnt<0>::imm);
        asm volatile("" ::: "memory");
        if ((threadIdx.x & 63) == 0) {
            q->slot = slot;
            q->list = list;
            q->ready = list == 1 && done >= need;
            if (slot >= 0) q->task = make_int4(e, row0, nsub, cb);
        }
    }
};

// The combine (tilelang.dataflow README section 3.5 step 5), once this
// workgroup's queue is empty: outputs i = blockIdx + grid * j of the T * nb2
// (token t, 128-column block cb) pieces, i = t nb2 + cb.  A batch of them
// waits (bounded, on the scheduler wave) until each has an arrival from every
// valid slot of its token, then their fp32 y rows come into LDS with
// device-scope direct-to-LDS loads (a lane per 16-byte piece, 32 pieces per
// row), and each (token, 4 columns) is summed in ascending slot order from +0.0
// and rounded once to bf16; a token without a valid slot gets zeros.  Each
// arrival counter goes back to 0.
template <int RING>
__device__ __forceinline__ void combine_share(const FusedPlan* pl, int32_t* arrive, int32_t* timeouts, int T, int nb2,
                                              int k, int d_h, const float* y, void* out, const unsigned char* zero,
                                              unsigned char* smem) {
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int items = T * nb2, G = gridDim.x;
    const int mine = items > (int)blockIdx.x ? (items - 1 - (int)blockIdx.x) / G + 1 : 0;
    // pieces a batch takes in LDS: item u, slot j, 16-byte piece c -> (u k + j) 32 + c;
    // a wave's load fills 64 pieces, so a batch keeps 64 pieces of room past its last one
    const int per_batch = min((RING - 64 * 16) / (k * 512), 64);
    auto valid = [&](int q) { return !((pl->bad[q >> 6] >> (q & 63)) & 1ull); };
    auto nvalid = [&](int t) {
        int nv = 0;
        for (int j = 0; j < k; ++j) nv += valid(t * k + j);
        return nv;
    };
    for (int u0 = 0; u0 < mine; u0 += per_batch) {
        const int nu = min(mine - u0, per_batch);
        if (w == kSchedWave) {
            // lane u: item u0 + u of the batch
            const int i = blockIdx.x + G * (u0 + lane);
            const int need = lane < nu ? nvalid(i / nb2) : 0;
            for (int it = 0;; ++it) {
                const int got = lane < nu ? __hip_atomic_load(arrive + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                          : 0;
                if (__ballot(got < need) == 0) break;
                if (it >= kSpinLimit) {
                    if (lane == 0)
                        __hip_atomic_fetch_add(timeouts, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        lds_barrier();
        const int pieces = nu * k * 32;
        for (int s0 = 64 * w; s0 < pieces; s0 += 64 * kGemmWaves) {
            const int sl = s0 + lane;
            const void* src = zero;
            if (sl < pieces) {
                const int uj = sl >> 5, c = sl & 31;
                const int u = uj / k, j = uj - u * k;
                const int i = blockIdx.x + G * (u0 + u);
                const int t = i / nb2, cb = i - t * nb2;
                const int q = t * k + j;
                if (valid(q)) src = y + (int64_t)q * d_h + cb * 128 + 4 * c;
            }
            g2l16c(src, lds_offset(smem + 16 * s0));
        }
        __builtin_amdgcn_s_waitcnt(VmCnt<0>::imm);
        lds_barrier();
        for (int x = tid; x < nu * 32; x += kGemmThreads) {
            const int u = x >> 5, c = x & 31;
            const int i = blockIdx.x + G * (u0 + u);
            const int t = i / nb2, cb = i - t * nb2;
            float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
            for (int j = 0; j < k; ++j) {
                if (!valid(t * k + j)) continue;
                const float4 v = *reinterpret_cast<const float4*>(smem + 16 * ((u * k + j) * 32 + c));
                a0 += v.x;
                a1 += v.y;
                a2 += v.z;
                a3 += v.w;
            }
            uint2 o;
            o.x = f32_to_bf16(a0) | (f32_to_bf16(a1) << 16);
            o.y = f32_to_bf16(a2) | (f32_to_bf16(a3) << 16);
            *reinterpret_cast<uint2*>(static_cast<unsigned short*>(out) + (int64_t)t * d_h + cb * 128 + 4 * c) = o;
        }
        for (int u = tid; u < nu; u += kGemmThreads)
            __hip_atomic_store(arrive + blockIdx.x + G * (u0 + u), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lds_barrier();  // the batch is read before the next one lands
    }
}

template <int MODE>
__global__ __launch_bounds__(kGemmThreads) void layer_kernel(LayerArgs a) {
    using L = LayerCfg<MODE>;
    constexpr int RING = L::kRing;
    constexpr int MT1 = L::kMT1, MT2 = L::kMT2;
    __shared__ __attribute__((aligned(16))) unsigned char smem[RING];
    __shared__ FusedQ q;
    __shared__ FusedPlan pl;
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int N = a.N, E = a.E, k = a.k;
    int32_t* sync = a.sync;
    const unsigned char* zero = reinterpret_cast<const unsigned char*>(sync + kSyncZero);

    FusedSched sch0{sync + kSyncQueue, sync + kSyncDone, &pl, &q, a.g1.topk_w, 0, 0, a.nb1, a.nb2, MT1, MT2, E};
    // the first claim goes out before the plan is built
    if (w == kSchedWave && lane == 0) sch0.claim();

    // ---- plan (tilelang.dataflow README section 3.5 step 1), in LDS.  Wave w
    // owns the contiguous chunk [w C, w C + C) of the assignments (C a multiple
    // of 64, 4 C = N rounded up to 256): ranks follow ascending p across waves,
    // then across the wave's 64-wide steps, then across lanes.
    constexpr int kSteps = kLayerMaxN / (64 * kGemmWaves);  // 64-wide steps of a chunk, at most
    const int C = ((N + kGemmWaves - 1) / kGemmWaves + 63) / 64 * 64;
    const int c_lo = w * C;
    int* wcnt = reinterpret_cast<int*>(smem);  // [waves][E]: per-wave counts, then bases (ring free until the first task)
    for (int i = tid; i < kGemmWaves * E; i += kGemmThreads) wcnt[i] = 0;
    // every id load goes out before the first is used (one memory round trip)
    int idv[kSteps];
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
        const int p = c_lo + 64 * u + lane;
        idv[u] = (64 * u < C && p < N) ? a.ids[p] : -1;
    }
    lds_barrier();
#pragma unroll
    for (int u = 0; u < kSteps; ++u) {
        if (64 * u >= C) break;
        const int p = c_lo + 64 * u + lane;
        const bool ok = (unsigned)idv[u] < (unsigned)E;
        const uint64_t badm = __ballot(!ok);
        if (lane == 0) pl.bad[p >> 6] = badm;
        if (ok) atomicAdd(&wcnt[w * E + idv[u]], 1);
    }
    lds_barrier();
    // Every wave reads all the per-wave counts at once and keeps, in lane l,
    // those of experts l, l + 64, ...: the expert counts, this wave's rank base
    // within each expert, and (a DPP scan) the padded offsets.  It writes
    // padded offset + base into its own row of wcnt, which only it reads: the
    // scatter below then needs no further barrier.  Wave 0 also publishes the
    // counts and padded offsets; every wave ranks a share of the experts (the
    // experts before e, with more rows or as many and a lower id, are a
    // popcount of ballots).
    constexpr int kJ = kMaxExperts / 64;
    int cj[kJ], bj[kJ];
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
        const int e = lane + 64 * j;
        int c = 0, base = 0;
        if (64 * j < E) {
#pragma unroll
            for (int ww = 0; ww < kGemmWaves; ++ww) {
                const int v = e < E ? wcnt[ww * E + e] : 0;
                if (ww < w) base += v;
                c += v;
            }
        }
        cj[j] = e < E ? c : -1;
        bj[j] = base;
    }
    lds_barrier();  // every wave has read the counts before any row is overwritten
    {
        int run = 0;
#pragma unroll
        for (int j = 0; j < kJ; ++j) {
            if (64 * j >= E) break;
            const int e = lane + 64 * j;
            const int padded = e < E ? kBlockM * ((cj[j] + kBlockM - 1) / kBlockM) : 0;
            const int incl = wave_inclusive_scan(padded, lane);
            const int off = run + incl - padded;
            if (e < E) {
                wcnt[w * E + e] = off + bj[j];
                if (w == 0) {
                    pl.poff[e] = off;
                    pl.cnt[e] = (short)cj[j];
                }
            }
            run += __builtin_amdgcn_readlane(incl, 63);
        }
        if (w == 0 && lane == 0) pl.poff[E] = run;
        for (int e = w; e < E; e += kGemmWaves) {
            int c = 0;
#pragma unroll
            for (int j = 0; j < kJ; ++j)
                if (j == (e >> 6)) c = __builtin_amdgcn_readlane(cj[j], e & 63);
            int r = 0;
#pragma unroll
            for (int j = 0; j < kJ; ++j) {
                if (64 * j >= E) break;
                const int e2 = lane + 64 * j;
                r += __popcll(__ballot(e2 < E && (cj[j] > c || (cj[j] == c && e2 < e))));
            }
            if (lane == 0) pl.order[r] = (unsigned char)e;
        }
    }
    // the stable scatter (no LDS atomics: the plan must come out the same in
    // every workgroup, since a GEMM-2 task reads the h rows that another
    // workgroup's GEMM-1 task placed by its own copy): each wave walks its chunk; lanes with the same expert
    // find each other with one ballot per bit of the key (the id, or 256 for an
    // invalid one: 9 bits); a lane's padded row is its wave's running position
    // for the expert plus the lanes before it in the group, and the group's
    // first lane advances that position (read once per step: a wave's LDS
    // accesses stay in order)
    {
        const uint64_t lt = lane ? (~0ull >> (64 - lane)) : 0ull;
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            if (64 * u >= C) break;
            const int p = c_lo + 64 * u + lane;
            const int id = idv[u];
            const bool valid = (unsigned)id < (unsigned)E;
            const int key = valid ? id : 256;
            uint64_t m = ~0ull;
#pragma unroll
            for (int b = 0; b < 9; ++b) {
                const bool bit = (key >> b) & 1;
                const uint64_t bal = __ballot(bit);
                m &= bit ? bal : ~bal;
            }
            const int wrank = __popcll(m & lt);
            if (valid) {
                const int pos = wcnt[w * E + id];
                pl.row_src[pos + wrank] = p;
                if (wrank == 0) wcnt[w * E + id] = pos + __popcll(m);
            }
        }
    }
    lds_barrier();
    // the M-tile offsets of both GEMMs in rank order (waves 1, 2) and the
    // padding rows of each expert's group
    auto tiles_of = [&](int e) { return (pl.cnt[e] + kBlockM - 1) / kBlockM; };
    if (w == 1)
        wave_exclusive_scan256([&](int r) { return (tiles_of(pl.order[r]) + MT1 - 1) / MT1; }, pl.moff[0], E, lane);
    if (w == 2)
        wave_exclusive_scan256([&](int r) { return (tiles_of(pl.order[r]) + MT2 - 1) / MT2; }, pl.moff[1], E, lane);
    for (int e = tid; e < E; e += kGemmThreads) {
        const int r1 = pl.poff[e + 1];
        for (int r = pl.poff[e] + pl.cnt[e]; r < r1; ++r) pl.row_src[r] = -1;
    }
    lds_barrier();
    const int n1 = pl.moff[0][E] * a.nb1, total = n1 + pl.moff[1][E] * a.nb2;

    // ---- the first task
    if (w == kSchedWave) {
        sch0.n1 = n1;
        sch0.total = total;
        sch0.settle(true);
        sch0.load_rows(0);
        sch0.publish();
    }
    lds_barrier();

    FusedCtx fx{nullptr, 0, sync + kSyncTimeouts, sync + kSyncArrive, k, a.nb2};
    for (int par = 0;; par ^= 1) {
        // uniform task fields (readfirstlane: see gemm1_kernel)
        const int t = __builtin_amdgcn_readfirstlane(q.slot);
        if (t < 0) break;
        const int list = __builtin_amdgcn_readfirstlane(q.list);
        const int e = __builtin_amdgcn_readfirstlane(q.task.x), row0 = __builtin_amdgcn_readfirstlane(q.task.y);
        const int nsub = __builtin_amdgcn_readfirstlane(q.task.z), cb = __builtin_amdgcn_readfirstlane(q.task.w);
        const bool ready = __builtin_amdgcn_readfirstlane(q.ready) != 0;
        FusedSched sch{sync + kSyncQueue, sync + kSyncDone, &pl, &q, a.g1.topk_w, n1, total, a.nb1, a.nb2, MT1, MT2, E};
        const int* rows = pl.row_src + row0;
        const float* roww = q.roww[par];
        // the completion counter of a task's GEMM-2 M-tile, at its first group
        // block: GEMM-1 adds to it, GEMM-2 waits for done_target
        const int g2_tile = (pl.poff[e] + (row0 - pl.poff[e]) / (kBlockM * MT2) * (kBlockM * MT2)) / kBlockM;
        fx.done = sync + kSyncDone + g2_tile;
        fx.target = sch.done_target(nsub);
#define MOE_L1(NS)                                                                                                 \
    gemm_task<MODE, true, NS, RING, true, FusedSched>(a.g1.x, a.g1.x_scale, nullptr, k, a.g1.w1, a.g1.w1_scale,     \
                                                      zero, e, row0, cb, a.g1.d_h, a.g1.d_e, a.g1.packed != 0,     \
                                                      smem, &a.g1, nullptr, sch, rows, roww, par, &fx)
#define MOE_L2(NS)                                                                                                 \
    gemm_task<MODE, false, NS, RING, true, FusedSched>(a.g2.h, a.g2.h_scale, nullptr, 1, a.g2.w2, a.g2.w2_scale,   \
                                                       zero, e, row0, cb, a.g2.d_e, a.g2.d_h, a.g2.packed != 0,    \
                                                       smem, nullptr, &a.g2, sch, rows, roww, par, &fx, ready)
        // one body per row-block count (nsub in [1, MT1] or [1, MT2])
        if (list == 0) {
            if constexpr (MT1 == 8) {
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
            static_assert(MT2 == 8, "GEMM-2 bodies for 1..8 row blocks");
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
        }
#undef MOE_L1
#undef MOE_L2
    }

    combine_share<RING>(&pl, sync + kSyncArrive, sync + kSyncTimeouts, a.T, a.nb2, k, a.g1.d_h,
                        static_cast<const float*>(a.g2.y), a.out, zero, smem);

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
        const int n_blocks = pl.poff[E] / kBlockM;  // every counter this call may have raised
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
