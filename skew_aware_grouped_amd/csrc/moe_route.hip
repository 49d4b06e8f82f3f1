// Routing metadata of the fused MoE layer on gfx950: per-expert histogram,
// prefix scan, stable scatter into the grouped-by-expert (padded) layout, the
// block map, and the device-built GEMM task lists.
//
// The metadata is the one the tilelang.dataflow README lists as the input of
// its fused MoE (section 3.5, step 1: group sizes, offsets, padded offsets and
// the expert of each group block).  Here it is produced on the device so that
// no host round trip of the routing is needed.
//
// 1 + 16 workgroups of 16 wave64s, with no communication between them.
// Every workgroup counts the whole batch per chunk (wave w of each counts
// chunk w, so all hold the same numbers): up to kLdsIds ids are read once
// into LDS, larger N reads them from memory again in the scatter.
// Workgroup 0 writes the counts, offsets and padding rows and builds the task
// lists; workgroup 1 + c scatters chunk c with its 16 waves (sub-chunk counts,
// then a ballot ranking within each sub-chunk).  The scatter is bound by a
// workgroup's VALU issue, so it runs on 16 CUs while workgroup 0 plans.
#include "moe_internal.h"
#include "moe_wave.h"

namespace moe {
namespace {

constexpr int kLdsIds = 16384;
// M-tiles per list that the rank-lookup table (kept in the ids' LDS, which
// workgroup 0 no longer needs when it builds the lists) can hold
constexpr int kRankTable = kLdsIds / 2;

// Largest e in [0,n) with off[e] <= r, for a non-decreasing off[0..n]
// and r < off[n].  Empty entries (off[e] == off[e+1]) are never returned.
__device__ __forceinline__ int upper_index(const int* off, int n, int r) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= r)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Column blocks cb in [0, nb) of expert rank r that go to XCD x: the task
// group (r, cb) has global index r*nb + cb and XCD (r*nb + cb) mod 8.
__device__ __forceinline__ int first_cb_on(int r, int nb, int x) { return (x - r * nb) & (kXcds - 1); }
__device__ __forceinline__ int cbs_on(int r, int nb, int x) {
    const int c0 = first_cb_on(r, nb, x);
    return c0 < nb ? (nb - 1 - c0) / kXcds + 1 : 0;
}

__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs a) {
    __shared__ short s_ids[kLdsIds];   // valid ids, -1 for the others; later the rank tables
    __shared__ int s_sub[kRouteWaves * kMaxExperts];  // [wave][E]: sub-chunk counts of the scattered chunk
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int s_tiles[kMaxExperts];
    __shared__ int s_off[kMaxExperts + 1];
    __shared__ int s_poff[kMaxExperts + 1];
    __shared__ int s_wcnt[kRouteWaves][kMaxExperts];
    __shared__ int s_order[kMaxExperts];
    __shared__ int s_rtiles[kMaxExperts];        // group blocks of the expert of each rank
    __shared__ int s_mt[2][kMaxExperts];         // M-tiles per expert rank, per list
    __shared__ int s_mtoff[2][kMaxExperts + 1];
    __shared__ int s_xpre[2][kXcds][kMaxExperts + 1];  // per list and XCD: tasks of lower ranks
    __shared__ int s_seg[2][kXcds + 1];
    __shared__ int s_dropped, s_mb1, s_mb2;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int E = a.E;
    const int N = a.N;
    const int g = blockIdx.x;  // 0: counts, offsets, task lists; 1 + c: scatter of chunk c
    const bool in_lds = N <= kLdsIds;

    for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) {
        s_wcnt[i / E][i % E] = 0;
        s_sub[i] = 0;
    }
    if (tid == 0) s_dropped = 0;
    if (a.zero && g == 0)
        for (int i = tid; i < kZeroBytes / 4; i += kRouteThreads) reinterpret_cast<int*>(a.zero)[i] = 0;
    __syncthreads();

    // Wave w owns the contiguous chunk [w*chunk, (w+1)*chunk) of the flat
    // assignments (chunk a multiple of 64), so ranks follow ascending p
    // across waves, then across the wave's 64-wide steps, then across lanes.
    const int chunk = ((N + kRouteWaves - 1) / kRouteWaves + 63) / 64 * 64;
    const int c_lo = wave * chunk;
    const int c_hi = min(N, c_lo + chunk);

    // 1. per-wave histograms (LDS atomics on the wave's own row); the ids
    // stay in LDS for the scatter when they fit
    int my_drop = 0;
    if (in_lds) {
        // the wave's whole chunk (at most kLdsIds / kRouteWaves ids) as one
        // batch of independent loads: one memory round trip, where a loop
        // whose every step ends in an LDS atomic on the loaded id waits for
        // each load in turn
        constexpr int kPer = kLdsIds / kRouteWaves / 64;
        int idv[kPer];
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int p = c_lo + lane + 64 * u;
            idv[u] = p < c_hi ? a.ids[p] : 0;
        }
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
            const int p = c_lo + lane + 64 * u;
            if (p < c_hi) {
                const bool ok = (unsigned)idv[u] < (unsigned)E;
                s_ids[p] = ok ? (short)idv[u] : (short)-1;
                if (ok)
                    atomicAdd(&s_wcnt[wave][idv[u]], 1);
                else
                    ++my_drop;
            }
        }
    } else {
        for (int p = c_lo + lane; p < c_hi; p += 64) {
            const int id = a.ids[p];
            if ((unsigned)id < (unsigned)E)
                atomicAdd(&s_wcnt[wave][id], 1);
            else
                ++my_drop;
        }
    }
    if (my_drop) atomicAdd(&s_dropped, my_drop);
    __syncthreads();

    // 2. counts, then each wave's rank base per expert (earlier waves' counts),
    // then the prefix scans of the counts and of the padded counts
    for (int e = tid; e < E; e += kRouteThreads) {
        int c[kRouteWaves];
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w) c[w] = s_wcnt[w][e];  // independent reads first
        int run = 0;
#pragma unroll
        for (int w = 0; w < kRouteWaves; ++w) {
            s_wcnt[w][e] = run;
            run += c[w];
        }
        s_cnt[e] = run;
        s_tiles[e] = (run + kBlockM - 1) / kBlockM;
    }
    __syncthreads();
    if (wave == 0) wave_exclusive_scan256([&](int e) { return s_cnt[e]; }, s_off, E, lane);
    if (wave == 1) wave_exclusive_scan256([&](int e) { return kBlockM * s_tiles[e]; }, s_poff, E, lane);
    __syncthreads();
    const int n_valid = s_off[E];
    const int n_pad = s_poff[E];
    if (g == 0) {
        for (int e = tid; e < E; e += kRouteThreads) a.counts[e] = s_cnt[e];
        for (int e = tid; e <= E; e += kRouteThreads) {
            a.offsets[e] = s_off[e];
            a.padded_offsets[e] = s_poff[e];
        }
    }
    // padding rows of each group and the unused tail of the padded space
    if (g == 0) {
        for (int e = wave; e < E; e += kRouteWaves)
            for (int r = s_poff[e] + s_cnt[e] + lane; r < s_poff[e + 1]; r += 64) a.row_src[r] = -1;
        for (int64_t i = n_pad + tid; i < a.n_pad_cap; i += kRouteThreads) a.row_src[i] = -1;
        if (a.full)
            for (int i = n_valid + tid; i < N; i += kRouteThreads) a.sorted_p[i] = -1;
    }

    if (g > 0) {
        // 3. stable scatter of chunk c = g - 1 (workgroup 0 goes on to the
        // task lists): wave v takes the v-th sub-chunk and counts it; then it
        // walks the sub-chunk 64 assignments at a time.  Lanes with the same
        // expert find each other with one ballot per bit of the key (the
        // expert id, or E for an invalid id: as many bits as E has, at most
        // 9).  The rank of p: chunk base (earlier chunks' counts, s_wcnt[c])
        // + earlier sub-chunks' counts + the wave's running count for the
        // expert + the number of lower lanes with the same expert; the lowest
        // such lane then advances the running count.  Ranks follow ascending p.
        {
            const int c = g - 1;
            const int q_lo = c * chunk, q_hi = min(N, q_lo + chunk);
            const int sub = ((chunk + kRouteWaves - 1) / kRouteWaves + 63) / 64 * 64;
            const int s_lo = q_lo + wave * sub;
            const int s_hi = min(q_hi, s_lo + sub);
            for (int p = s_lo + lane; p < s_hi; p += 64) {
                const int id = in_lds ? s_ids[p] : a.ids[p];
                if ((unsigned)id < (unsigned)E) atomicAdd(&s_sub[wave * E + id], 1);
            }
            __syncthreads();
            for (int e = tid; e < E; e += kRouteThreads) {
                int run = 0;
                for (int v = 0; v < kRouteWaves; ++v) {
                    const int n = s_sub[v * E + e];
                    s_sub[v * E + e] = run;
                    run += n;
                }
            }
            __syncthreads();
            const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
            const int kb = 32 - __clz(E);
            for (int base = s_lo; base < s_hi; base += 64) {
                const int p = base + lane;
                const int id = p < s_hi ? (in_lds ? s_ids[p] : a.ids[p]) : -1;
                const bool valid = (unsigned)id < (unsigned)E;
                const int key = valid ? id : E;
                uint64_t m = ~0ull;
#pragma unroll
                for (int b = 0; b < 9; ++b) {
                    if (b >= kb) break;
                    const bool bit = (key >> b) & 1;
                    const uint64_t bal = __ballot(bit);
                    m &= bit ? bal : ~bal;
                }
                const int wrank = __popcll(m & lt);
                if (valid) {
                    const int r = s_wcnt[c][id] + s_sub[wave * E + id] + wrank;
                    if (a.full) {
                        a.pos[p] = s_off[id] + r;
                        a.ppos[p] = s_poff[id] + r;
                        a.sorted_p[s_off[id] + r] = p;
                    }
                    a.row_src[s_poff[id] + r] = p;
                } else if (p < s_hi && a.full) {
                    a.pos[p] = -1;
                    a.ppos[p] = -1;
                }
                // every lane has read its base above; the first lane of each
                // expert group advances it
                if (valid && wrank == 0) s_sub[wave * E + id] += __popcll(m);
            }
        }
        return;
    }

    // (workgroup 0 from here on)
    if (a.nb1 > 0) {
        // 5. task lists.  Experts are ranked by descending row count (ties by id):
        // longest work first.  An expert's tasks are its M-tiles (up to
        // kMaxRowBlocks1 / kMaxRowBlocks2 group blocks) times the column blocks.  The task group
        // (rank r, column block cb) -- every M-tile of one weight block -- goes to
        // XCD (r*nb + cb) mod 8, so the M-tiles that read the same weights run
        // side by side on one L2; each XCD's segment of the list keeps rank order.
        {
            // lane l of every wave holds the counts of experts l, l + 64, ...;
            // wave w ranks experts w, w + 16, ...: the number of experts ranked
            // before e is a popcount of ballots over the lanes, with no LDS
            // round trip per comparison
            constexpr int kJ = kMaxExperts / 64;
            int cj[kJ];
#pragma unroll
            for (int j = 0; j < kJ; ++j) cj[j] = lane + 64 * j < E ? s_cnt[lane + 64 * j] : -1;
            for (int e = wave; e < E; e += kRouteWaves) {
                const int je = e >> 6;  // wave-uniform
                int c = 0;
#pragma unroll
                for (int j = 0; j < kJ; ++j)
                    if (j == je) c = __builtin_amdgcn_readlane(cj[j], e & 63);
                int r = 0;
#pragma unroll
                for (int j = 0; j < kJ; ++j) {
                    if (64 * j >= E) break;
                    const int e2 = lane + 64 * j;
                    const bool before = e2 < E && ((cj[j] > c) || (cj[j] == c && e2 < e));
                    r += __popcll(__ballot(before));
                }
                if (lane == 0) {
                    s_order[r] = e;
                    s_rtiles[r] = s_tiles[e];
                }
            }
        }
        // M-tiles of 8 group blocks (fewer weight re-reads) when that still leaves
        // min_tasks1 (min_tasks2) tasks, otherwise kSmallRowBlocks (more tasks to
        // spread over the CUs); the 8-wave FP8 GEMMs (mb1_max 16, mb2 16) take
        // 16-block M-tiles when those still leave min_tasks1 (min_tasks2) tasks.
        // The last wave decides for both lists after its share of the ranking
        if (wave == kRouteWaves - 1) {
            int big = 0, big16 = 0;
            for (int e = lane; e < E; e += 64) {
                big += (s_tiles[e] + 7) >> 3;
                big16 += (s_tiles[e] + 15) >> 4;
            }
            big = __builtin_amdgcn_readlane(wave_inclusive_scan(big, lane), 63);
            big16 = __builtin_amdgcn_readlane(wave_inclusive_scan(big16, lane), 63);
            if (lane == 0) {
                s_mb1 = a.mb1_max == 16 && big16 * a.nb1 >= a.min_tasks1 ? 16
                        : big * a.nb1 >= a.min_tasks1                   ? kMaxRowBlocks1
                                                                        : kSmallRowBlocks;
                s_mb2 = a.mb2 == 16 && big16 * a.nb2 >= a.min_tasks2  ? 16
                        : a.mb2 >= 8 && big * a.nb2 >= a.min_tasks2 ? 8
                                                                     : kSmallRowBlocks;
            }
        }
    }
    __syncthreads();

    // 4. block map: expert and first padded row of each group block (the
    // layer's GEMMs take the task lists instead, so only for moe_route)
    const int ntiles = n_pad / kBlockM;
    for (int64_t i = tid; a.full && i < a.tile_cap; i += kRouteThreads) {
        if (i < ntiles) {
            const int r = (int)i * kBlockM;
            a.tile_expert[i] = upper_index(s_poff, E, r);
            a.tile_row0[i] = r;
        } else {
            a.tile_expert[i] = -1;
            a.tile_row0[i] = -1;
        }
    }
    if (tid == 0) {
        a.ctl[kStatDropped] = s_dropped;
        a.ctl[kStatTiles] = ntiles;
        a.ctl[kStatPadRows] = n_pad;
        a.ctl[kStatTasks1] = 0;
    }
    if (a.nb1 <= 0) return;

    const int mb1 = s_mb1, mb2 = s_mb2;
    // M-tiles of the expert of rank r in list 0 (GEMM-1) or 1 (GEMM-2); the
    // M-tile sizes are powers of two
    static_assert(kMaxRowBlocks1 == 8 && kMaxRowBlocks2 == 8 && kSmallRowBlocks == 4 && kMaxRowBlocksFp8G1 == 16,
                  "M-tile sizes 16, 8 and 4 group blocks");
    // When 8-block GEMM-1 tiles leave workgroup slots idle but 4-block tiles
    // make more tasks than slots (a second, partial round), the hottest ranks
    // [0, r8) keep 8-block tiles: the fewest that bring the task count down to
    // min_tasks1.  Every wave works r8 out itself (no barrier).  Not in FP8
    // mode (mix1 = 0), where a 128-row task's epilogue costs more than the
    // partial round it saves.
    int r8 = mb1 == 8 ? E : 0;
    if (mb1 == kSmallRowBlocks && a.mix1) {
        int t4 = 0, d8[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * lane + i;
            const int t = r < E ? s_rtiles[r] : 0;
            t4 += (t + 3) >> 2;
            d8[i] = ((t + 3) >> 2) - ((t + 7) >> 3);  // M-tiles saved by 8-block tiles
        }
        const int total4 = __builtin_amdgcn_readlane(wave_inclusive_scan(t4, lane), 63);
        const int need = total4 * a.nb1 - a.min_tasks1;  // tasks to remove
        if (need > 0) {
            const int dl = d8[0] + d8[1] + d8[2] + d8[3];
            int run = wave_inclusive_scan(dl, lane) - dl;  // saved by the ranks before this lane's
            int first = kMaxExperts;                        // first rank whose prefix covers need
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                run += d8[i];
                if (first == kMaxExperts && run * a.nb1 >= need && 4 * lane + i < E) first = 4 * lane + i;
            }
            const uint64_t hit = __ballot(first < kMaxExperts);
            r8 = hit ? __builtin_amdgcn_readlane(first, __builtin_ctzll(hit)) + 1 : E;
        }
    }
    // group blocks per GEMM-1 M-tile of rank r
    auto lg1 = [&](int r) { return mb1 == 16 ? 4 : r < r8 ? 3 : 2; };
    auto mb1_of = [&](int r) { return 1 << lg1(r); };
    const int lg_mb2 = mb2 == 16 ? 4 : mb2 == 8 ? 3 : 2;
    auto mtiles = [&](int list, int r) {
        const int lg = list == 0 ? lg1(r) : lg_mb2;
        return (s_rtiles[r] + (1 << lg) - 1) >> lg;
    };
    {
        // waves 0..7: GEMM-1 list, XCD = wave; waves 8..15: GEMM-2 list
        const int list = wave / kXcds, x = wave % kXcds;
        const int nb = list == 0 ? a.nb1 : a.nb2;
        wave_exclusive_scan256([&](int r) { return cbs_on(r, nb, x) * mtiles(list, r); }, s_xpre[list][x], E,
                               lane);
    }
    if (wave < 2) {
        wave_exclusive_scan256([&](int r) { return mtiles(wave, r); }, s_mtoff[wave], E, lane);
        for (int r = lane; r < E; r += 64) s_mt[wave][r] = mtiles(wave, r);
    }
    __syncthreads();
    if (tid < 2) {
        int run = 0;
        for (int x = 0; x < kXcds; ++x) {
            s_seg[tid][x] = run;
            run += s_xpre[tid][x][E];
        }
        s_seg[tid][kXcds] = run;
    }
    // with more tasks than threads: the rank of every M-tile of each list, so
    // that a task finds its expert rank with one LDS read instead of a binary
    // search (the ids in LDS are no longer needed)
    short* s_rank_of = s_ids;  // [2][kRankTable]
    const bool rank_table = s_mtoff[0][E] * a.nb1 + s_mtoff[1][E] * a.nb2 > kRouteThreads &&
                            s_mtoff[0][E] <= kRankTable && s_mtoff[1][E] <= kRankTable;
    if (rank_table) {
        const int mt0 = s_mtoff[0][E];
        for (int g = tid; g < mt0 + s_mtoff[1][E]; g += kRouteThreads) {
            const int list = g < mt0 ? 0 : 1;
            const int m = list == 0 ? g : g - mt0;
            s_rank_of[list * kRankTable + m] = (short)upper_index(s_mtoff[list], E, m);
        }
    }
    __syncthreads();
    {
        // both lists in one pass over their concatenated task indices
        const int total0 = s_mtoff[0][E] * a.nb1;
        const int total = total0 + s_mtoff[1][E] * a.nb2;
        for (int g = tid; g < total; g += kRouteThreads) {
            const int list = g < total0 ? 0 : 1;
            const int i = list == 0 ? g : g - total0;
            const int nb = list == 0 ? a.nb1 : a.nb2;
            int4* tasks = list == 0 ? a.tasks1 : a.tasks2;
            // rank r owns tasks [s_mtoff[r]*nb, s_mtoff[r+1]*nb), column-major
            const int r = rank_table ? s_rank_of[list * kRankTable + i / nb] : upper_index(s_mtoff[list], E, i / nb);
            const int mb = list == 0 ? mb1_of(r) : mb2;
            const int mt = s_mt[list][r];
            const int local = i - s_mtoff[list][r] * nb;
            const int cb = local / mt;
            const int m = local - cb * mt;
            const int e = s_order[r];
            const int x = (r * nb + cb) & (kXcds - 1);
            const int q = (cb - first_cb_on(r, nb, x)) / kXcds;
            const int nsub = min(mb, s_rtiles[r] - m * mb);
            tasks[s_seg[list][x] + s_xpre[list][x][r] + q * mt + m] =
                make_int4(e, s_poff[e] + m * mb * kBlockM, nsub, cb);
        }
    }
    if (tid < 2) a.ctl[tid == 0 ? kStatTasks1 : kStatTasks2] = s_seg[tid][kXcds];
    // queue counters start past the tasks the workgroups take statically
    if (tid < 2 * kXcds) {
        const int list = tid / kXcds, x = tid % kXcds;
        a.ctl[(list == 0 ? kCtlQueue1 : kCtlQueue2) + kQueueStride * x] =
            static_tasks(list == 0 ? a.grid1 : a.grid2, x, s_seg[list][x + 1] - s_seg[list][x]);
    }
    if (tid < 2 * (kXcds + 1)) {
        const int list = tid / (kXcds + 1), x = tid % (kXcds + 1);
        a.ctl[(list == 0 ? kCtlSeg1 : kCtlSeg2) + x] = s_seg[list][x];
    }
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
    hipExtLaunchKernelGGL(route_kernel, dim3(1 + kRouteWaves), dim3(kRouteThreads), 0, s, t0, t1, 0, a);
    return hipGetLastError();
}

}  // namespace moe
