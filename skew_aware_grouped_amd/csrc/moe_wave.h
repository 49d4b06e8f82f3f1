// Wave-level scans (DPP, register to register) shared by the routing kernel
// and the single-launch layer kernel.  Internal header, not installed.
#pragma once

#include "moe_internal.h"

namespace moe {
namespace {

// v + (the value of lane - k in the same row of 16 lanes, 0 where that lane
// is outside the row), or with row_bcast the last lane of the previous row(s)
// for the rows ROW_MASK selects (DPP: register-to-register, no LDS traffic)
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_add(int v) {
    return v + __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive sum over lanes 0..lane of a wave64: shifts by 1, 2, 4 and 8
// within each row of 16 lanes, then the row totals carried into rows 1 and 3
// (row_bcast:15) and into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ int wave_inclusive_scan(int v, int) {
    v = dpp_add<0x111>(v);  // row_shr:1
    v = dpp_add<0x112>(v);  // row_shr:2
    v = dpp_add<0x114>(v);  // row_shr:4
    v = dpp_add<0x118>(v);  // row_shr:8
    v = dpp_add<0x142, 0xA>(v);  // row_bcast:15
    v = dpp_add<0x143, 0xC>(v);  // row_bcast:31
    return v;
}

// Exclusive scan of src[0..n) into dst[0..n], dst[n] = total; n <= 256; run by
// one full wave.  Each lane owns four consecutive entries.
template <typename F>
__device__ __forceinline__ void wave_exclusive_scan256(F src, int* dst, int n, int lane) {
    int v[4];
    int local = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int e = 4 * lane + i;
        v[i] = e < n ? src(e) : 0;
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

}  // namespace
}  // namespace moe
