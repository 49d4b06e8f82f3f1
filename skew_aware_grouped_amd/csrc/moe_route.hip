// Routing metadata of the fused MoE layer on gfx950: per-expert histogram,
// prefix scan, stable scatter into the grouped-by-expert (padded) layout, the
// block map, and the device-built GEMM task lists.
//
// The metadata is the one the tilelang.dataflow README lists as the input of
// its fused MoE (section 3.5, step 1: group sizes, offsets, padded offsets and
// the expert of each group block).  Here it is produced on the device so that
// no host round trip of the routing is needed.
//
// One workgroup of 16 wave64s does everything in LDS: N = T*k is at most a few
// ten thousand assignments on the paths this serves, so a single workgroup
// finishes in a few microseconds and avoids any cross-workgroup protocol.
#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int t = __shfl_up(v, d, 64);
        if (lane >= d) v += t;
    }
    return v;
}

// Exclusive scan of src[0..n) into dst[0..n], dst[n] = total; n <= 256; run by
// one full wave.  Each lane owns four consecutive entries.
__device__ __forceinline__ void wave_exclusive_scan256(const int* src, int* dst, int n, int lane) {
    int v[4];
    int local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int e = 4 * lane + i;
        v[i] = e < n ? src[e] : 0;
        local += v[i];
    }
    int incl = wave_inclusive_scan(local, lane);
    int run = incl - local;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int e = 4 * lane + i;
        if (e < n) dst[e] = run;
        run += v[i];
    }
    if (lane == 63) dst[n] = incl;
}

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

__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs a) {
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int s_tiles[kMaxExperts];
    __shared__ int s_off[kMaxExperts + 1];
    __shared__ int s_poff[kMaxExperts + 1];
    __shared__ int s_base[kMaxExperts];
    __shared__ int s_wcnt[kRouteWaves][kMaxExperts];
    __shared__ int s_order[kMaxExperts];
    __shared__ int s_mt[kMaxExperts];
    __shared__ int s_mtoff[kMaxExperts + 1];
    __shared__ int s_dropped;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int E = a.E;
    const int N = a.N;

    for (int e = tid; e < kMaxExperts; e += kRouteThreads) {
        s_cnt[e] = 0;
        s_base[e] = 0;
    }
    for (int i = tid; i < kRouteWaves * kMaxExperts; i += kRouteThreads) (&s_wcnt[0][0])[i] = 0;
    if (tid == 0) s_dropped = 0;
    if (a.zero)
        for (int i = tid; i < kZeroBytes / 4; i += kRouteThreads) reinterpret_cast<int*>(a.zero)[i] = 0;
    __syncthreads();

    // 1. histogram (LDS atomics: the counts do not depend on their order)
    int my_drop = 0;
    for (int p = tid; p < N; p += kRouteThreads) {
        int id = a.ids[p];
        if ((unsigned)id < (unsigned)E)
            atomicAdd(&s_cnt[id], 1);
        else
            ++my_drop;
    }
    if (my_drop) atomicAdd(&s_dropped, my_drop);
    __syncthreads();

    // 2. prefix scans of the counts and of the padded counts
    for (int e = tid; e < E; e += kRouteThreads) s_tiles[e] = (s_cnt[e] + kBlockM - 1) / kBlockM;
    __syncthreads();
    if (wave == 0) wave_exclusive_scan256(s_cnt, s_off, E, lane);
    if (wave == 1) {
        wave_exclusive_scan256(s_tiles, s_poff, E, lane);
    }
    __syncthreads();
    for (int e = tid; e <= E; e += kRouteThreads) s_poff[e] *= kBlockM;
    __syncthreads();
    const int n_valid = s_off[E];
    const int n_pad = s_poff[E];
    for (int e = tid; e < E; e += kRouteThreads) a.counts[e] = s_cnt[e];
    for (int e = tid; e <= E; e += kRouteThreads) {
        a.offsets[e] = s_off[e];
        a.padded_offsets[e] = s_poff[e];
    }
    for (int64_t i = tid; i < a.n_pad_cap; i += kRouteThreads) a.row_src[i] = -1;
    for (int i = n_valid + tid; i < N; i += kRouteThreads) a.sorted_p[i] = -1;
    __syncthreads();

    // 3. stable scatter, 1024 assignments per round.  Inside a wave, lanes with
    // the same expert find each other with 9 ballots over the id bits; the rank
    // of an assignment is the count of earlier rounds, of lower waves in this
    // round, and of lower lanes in its own wave.
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = 0; base < N; base += kRouteThreads) {
        const int p = base + tid;
        const int id = p < N ? a.ids[p] : -1;
        const bool valid = (unsigned)id < (unsigned)E;
        const int key = valid ? id : 511;
        uint64_t m = ~0ull;
#pragma unroll
        for (int b = 0; b < 9; ++b) {
            const bool bit = (key >> b) & 1;
            const uint64_t bal = __ballot(bit);
            m &= bit ? bal : ~bal;
        }
        const int wrank = __popcll(m & lt_mask);
        if (valid && wrank == 0) s_wcnt[wave][id] = __popcll(m);
        __syncthreads();
        if (valid) {
            int r = s_base[id] + wrank;
            for (int w = 0; w < wave; ++w) r += s_wcnt[w][id];
            a.pos[p] = s_off[id] + r;
            a.ppos[p] = s_poff[id] + r;
            a.sorted_p[s_off[id] + r] = p;
            a.row_src[s_poff[id] + r] = p;
        } else if (p < N) {
            a.pos[p] = -1;
            a.ppos[p] = -1;
        }
        __syncthreads();
        for (int e = tid; e < E; e += kRouteThreads) {
            int s = 0;
            for (int w = 0; w < kRouteWaves; ++w) {
                s += s_wcnt[w][e];
                s_wcnt[w][e] = 0;
            }
            s_base[e] += s;
        }
        __syncthreads();
    }

    // 4. block map: expert and first padded row of each group block
    const int ntiles = n_pad / kBlockM;
    for (int64_t i = tid; i < a.tile_cap; i += kRouteThreads) {
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
        a.stats[kStatDropped] = s_dropped;
        a.stats[kStatTiles] = ntiles;
        a.stats[kStatPadRows] = n_pad;
        a.stats[kStatTasks1] = 0;
    }
    if (a.nb1 <= 0) return;

    // 5. task lists.  Experts are ordered by descending row count (ties by id):
    // longest work first.  An expert's tasks are its M-tiles (up to
    // kMaxRowBlocks group blocks) times the column blocks, M-tile fastest, so
    // the tasks that read the same weight block are pulled back to back.
    for (int e = tid; e < E; e += kRouteThreads) {
        const int c = s_cnt[e];
        int r = 0;
        for (int e2 = 0; e2 < E; ++e2) {
            const int c2 = s_cnt[e2];
            r += (c2 > c) || (c2 == c && e2 < e);
        }
        s_order[r] = e;
    }
    __syncthreads();
    for (int r = tid; r < E; r += kRouteThreads)
        s_mt[r] = (s_tiles[s_order[r]] + kMaxRowBlocks - 1) / kMaxRowBlocks;
    __syncthreads();
    if (wave == 0) wave_exclusive_scan256(s_mt, s_mtoff, E, lane);
    __syncthreads();
    const int n_mtiles = s_mtoff[E];
    for (int list = 0; list < 2; ++list) {
        const int nb = list == 0 ? a.nb1 : a.nb2;
        int4* tasks = list == 0 ? a.tasks1 : a.tasks2;
        const int total = n_mtiles * nb;
        for (int i = tid; i < total; i += kRouteThreads) {
            // rank r owns tasks [s_mtoff[r]*nb, s_mtoff[r+1]*nb)
            const int r = upper_index(s_mtoff, E, i / nb);
            const int mt = s_mt[r];
            const int local = i - s_mtoff[r] * nb;
            const int col = local / mt;
            const int m = local - col * mt;
            const int e = s_order[r];
            const int nsub = min(kMaxRowBlocks, s_tiles[e] - m * kMaxRowBlocks);
            tasks[i] = make_int4(e, s_poff[e] + m * kMaxRowBlocks * kBlockM, nsub, col);
        }
        if (tid == 0) a.stats[list == 0 ? kStatTasks1 : kStatTasks2] = total;
    }
    if (tid == 0) {
        a.stats[kStatCounter1] = 0;
        a.stats[kStatCounter2] = 0;
    }
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(route_kernel, dim3(1), dim3(kRouteThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
