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
// Tile mapping (16x16 MFMA, wave64): lane l holds A row (l % 16) and B row
// (l % 16) with a K slice chosen by (l / 16); the accumulator element i of
// lane l is C[4*(l/16) + i][l % 16].  A and B use the same K slice per lane,
// so any per-lane K assignment is a valid split of the reduction.  The gate
// and up accumulators of one output column sit in the same lane, so SwiGLU
// needs no data movement.
//
// FP8 (E4M3FN): one 16x16x128 MFMA covers exactly one 128-wide scale block
// of K, so each MFMA starts from zero and its result is promoted into the fp32
// accumulator with (row scale of x or h) * (block scale of W) -- the block
// dequantisation happens in registers.  bf16: 16x16x32 MFMA, accumulating
// directly.
#include "moe_internal.h"

namespace moe {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef unsigned short v8u16 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v4f mfma_fp8(const v8i& a, const v8i& b, const v4f& c) {
    // format 0 = E4M3 for both operands; E8M0 scale 127 = 1.0 (no MX scaling)
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ v4f mfma_bf16(const v8bf& a, const v8bf& b, const v4f& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// binary32 -> bfloat16 bits, round to nearest even (values here are finite)
__device__ __forceinline__ unsigned short f32_to_bf16(float f) {
    unsigned u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (unsigned short)(u >> 16);
}

// binary32 -> E4M3FN code via the hardware converter (round to nearest even)
__device__ __forceinline__ unsigned char f32_to_e4m3(float f) {
    return (unsigned char)(__builtin_amdgcn_cvt_pk_fp8_f32(f, 0.0f, 0, false) & 0xff);
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

__device__ __forceinline__ v8i ld32(const unsigned char* p) { return *reinterpret_cast<const v8i*>(p); }

// 16 bf16 values (32 bytes) split in two MFMA operands
struct Bf16x16 {
    v8bf lo, hi;
};

__device__ __forceinline__ Bf16x16 ld_bf16x16(const unsigned short* p) {
    const v8i raw = *reinterpret_cast<const v8i*>(p);
    Bf16x16 r;
    __builtin_memcpy(&r, &raw, 32);
    return r;
}

__device__ __forceinline__ Bf16x16 ld_f32x16_as_bf16(const float* p) {
    const float4* q = reinterpret_cast<const float4*>(p);
    unsigned short b[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float4 v = q[i];
        b[4 * i + 0] = f32_to_bf16(v.x);
        b[4 * i + 1] = f32_to_bf16(v.y);
        b[4 * i + 2] = f32_to_bf16(v.z);
        b[4 * i + 3] = f32_to_bf16(v.w);
    }
    Bf16x16 r;
    __builtin_memcpy(&r, b, 32);
    return r;
}

__device__ __forceinline__ Bf16x16 zero_bf16x16() {
    const v8i z = {0, 0, 0, 0, 0, 0, 0, 0};
    Bf16x16 r;
    __builtin_memcpy(&r, &z, 32);
    return r;
}

__device__ __forceinline__ int pull_task(int32_t* counter, int* s_slot) {
    if (threadIdx.x == 0) *s_slot = atomicAdd(counter, 1);
    __syncthreads();
    const int t = *s_slot;
    __syncthreads();
    return t;
}

// ---------------------------------------------------------------- GEMM-1 FP8
// Task: 16*NSUB rows x 128 intermediate columns; wave w owns columns
// [32w, 32w+32) as two 16-column fragments, for both gate and up.
template <int NSUB>
__device__ __forceinline__ void gemm1_fp8_task(const Gemm1Args& a, int e, int row0, int cb, float* s_amax) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int d_h = a.d_h, d_e = a.d_e, kq = d_h / kQ;
    const unsigned char* x = static_cast<const unsigned char*>(a.x);
    const unsigned char* w1 = static_cast<const unsigned char*>(a.w1);

    const unsigned char* pa[NSUB];
    bool va[NSUB];
    const float* psx[NSUB][4];
    bool vc[NSUB][4];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
        const int p = a.row_src[row0 + 16 * s + lr];
        va[s] = p >= 0;
        pa[s] = x + (int64_t)(p >= 0 ? p / a.k : 0) * d_h + lg * 32;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pc = a.row_src[row0 + 16 * s + 4 * lg + i];
            vc[s][i] = pc >= 0;
            psx[s][i] = a.x_scale + (int64_t)(pc >= 0 ? pc / a.k : 0) * kq;
        }
    }
    const unsigned char* pg[2];
    const unsigned char* pu[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        const int row = cb * 128 + w * 32 + 16 * f + lr;
        pg[f] = w1 + ((int64_t)e * 2 * d_e + row) * d_h + lg * 32;
        pu[f] = pg[f] + (int64_t)d_e * d_h;
    }
    const float* psg = a.w1_scale + ((int64_t)e * (2 * d_e / kQ) + cb) * kq;
    const float* psu = psg + (int64_t)(d_e / kQ) * kq;

    v4f accg[NSUB][2], accu[NSUB][2];
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int f = 0; f < 2; ++f) accg[s][f] = accu[s][f] = zero;

    const v8i vz = {0, 0, 0, 0, 0, 0, 0, 0};
    v8i A[NSUB], BG[2], BU[2];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) A[s] = va[s] ? ld32(pa[s]) : vz;
#pragma unroll
    for (int f = 0; f < 2; ++f) {
        BG[f] = ld32(pg[f]);
        BU[f] = ld32(pu[f]);
    }
    for (int kb = 0; kb < kq; ++kb) {
        // prefetch the next K block (clamped on the last iteration)
        const int kn = (kb + 1 < kq ? kb + 1 : kb) * kQ;
        v8i An[NSUB], BGn[2], BUn[2];
#pragma unroll
        for (int s = 0; s < NSUB; ++s) An[s] = va[s] ? ld32(pa[s] + kn) : vz;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            BGn[f] = ld32(pg[f] + kn);
            BUn[f] = ld32(pu[f] + kn);
        }
        const float sg = psg[kb], su = psu[kb];
        float sx[NSUB][4];
#pragma unroll
        for (int s = 0; s < NSUB; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) sx[s][i] = vc[s][i] ? psx[s][i][kb] : 0.f;
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                const v4f tg = mfma_fp8(A[s], BG[f], zero);
                const v4f tu = mfma_fp8(A[s], BU[f], zero);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    accg[s][f][i] += tg[i] * (sx[s][i] * sg);
                    accu[s][f][i] += tu[i] * (sx[s][i] * su);
                }
            }
        }
#pragma unroll
        for (int s = 0; s < NSUB; ++s) A[s] = An[s];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            BG[f] = BGn[f];
            BU[f] = BUn[f];
        }
    }

    // SwiGLU on the fp32 accumulators, then per-row-per-128 requantisation:
    // amax over the task's 128 columns (2 fragments x 16 lanes x 4 waves).
    float hv[NSUB][2][4];
    float rmax[NSUB][4];
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float m = 0.f;
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                hv[s][f][i] = silu_mul(accg[s][f][i], accu[s][f][i]);
                m = fmaxf(m, fabsf(hv[s][f][i]));
            }
#pragma unroll
            for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
            rmax[s][i] = m;
        }
    if (lr == 0) {
#pragma unroll
        for (int s = 0; s < NSUB; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_amax[w * 64 + s * 16 + 4 * lg + i] = rmax[s][i];
    }
    __syncthreads();
    unsigned char* h = static_cast<unsigned char*>(a.h);
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rr = s * 16 + 4 * lg + i;
            float amax = fmaxf(fmaxf(s_amax[rr], s_amax[64 + rr]), fmaxf(s_amax[128 + rr], s_amax[192 + rr]));
            const float sc = amax > 0.f ? amax / 448.0f : 1.0f;
            const int64_t prow = row0 + rr;
#pragma unroll
            for (int f = 0; f < 2; ++f)
                h[prow * d_e + cb * 128 + w * 32 + 16 * f + lr] = f32_to_e4m3(hv[s][f][i] / sc);
            if (w == 0 && lr == 0) a.h_scale[prow * (d_e / kQ) + cb] = sc;
        }
    __syncthreads();
}

// --------------------------------------------------------------- GEMM-1 bf16
// Task: 16*NSUB rows x 64 intermediate columns; wave w owns columns [16w, 16w+16).
template <int NSUB, bool F32X>
__device__ __forceinline__ void gemm1_bf16_task(const Gemm1Args& a, int e, int row0, int cb) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int d_h = a.d_h, d_e = a.d_e;
    const unsigned short* w1 = static_cast<const unsigned short*>(a.w1);

    int64_t ao[NSUB];
    bool va[NSUB];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
        const int p = a.row_src[row0 + 16 * s + lr];
        va[s] = p >= 0;
        ao[s] = (int64_t)(p >= 0 ? p / a.k : 0) * d_h + lg * 16;
    }
    const int row = cb * 64 + w * 16 + lr;
    const unsigned short* pg = w1 + ((int64_t)e * 2 * d_e + row) * d_h + lg * 16;
    const unsigned short* pu = pg + (int64_t)d_e * d_h;

    auto load_a = [&](int s, int k0) -> Bf16x16 {
        if (!va[s]) return zero_bf16x16();
        if (F32X) return ld_f32x16_as_bf16(static_cast<const float*>(a.x) + ao[s] + k0);
        return ld_bf16x16(static_cast<const unsigned short*>(a.x) + ao[s] + k0);
    };

    v4f accg[NSUB], accu[NSUB];
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NSUB; ++s) accg[s] = accu[s] = zero;

    const int nk = d_h / 64;
    Bf16x16 A[NSUB], BG, BU;
#pragma unroll
    for (int s = 0; s < NSUB; ++s) A[s] = load_a(s, 0);
    BG = ld_bf16x16(pg);
    BU = ld_bf16x16(pu);
    for (int kc = 0; kc < nk; ++kc) {
        const int kn = (kc + 1 < nk ? kc + 1 : kc) * 64;
        Bf16x16 An[NSUB];
#pragma unroll
        for (int s = 0; s < NSUB; ++s) An[s] = load_a(s, kn);
        const Bf16x16 BGn = ld_bf16x16(pg + kn);
        const Bf16x16 BUn = ld_bf16x16(pu + kn);
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
            accg[s] = mfma_bf16(A[s].lo, BG.lo, accg[s]);
            accg[s] = mfma_bf16(A[s].hi, BG.hi, accg[s]);
            accu[s] = mfma_bf16(A[s].lo, BU.lo, accu[s]);
            accu[s] = mfma_bf16(A[s].hi, BU.hi, accu[s]);
        }
#pragma unroll
        for (int s = 0; s < NSUB; ++s) A[s] = An[s];
        BG = BGn;
        BU = BUn;
    }
    unsigned short* h = static_cast<unsigned short*>(a.h);
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t prow = row0 + s * 16 + 4 * lg + i;
            h[prow * d_e + cb * 64 + w * 16 + lr] = f32_to_bf16(silu_mul(accg[s][i], accu[s][i]));
        }
}

template <int MODE>
__global__ __launch_bounds__(kGemmThreads) void gemm1_kernel(Gemm1Args a) {
    __shared__ float s_amax[kGemmWaves * 64];
    __shared__ int s_slot;
    const int ntasks = a.stats[kStatTasks1];
    for (;;) {
        const int t = pull_task(&a.stats[kStatCounter1], &s_slot);
        if (t >= ntasks) break;
        const int4 task = a.tasks[t];
        const int e = task.x, row0 = task.y, nsub = task.z, cb = task.w;
        if constexpr (MODE == MOE_MODE_FP8) {
            switch (nsub) {
                case 1: gemm1_fp8_task<1>(a, e, row0, cb, s_amax); break;
                case 2: gemm1_fp8_task<2>(a, e, row0, cb, s_amax); break;
                case 3: gemm1_fp8_task<3>(a, e, row0, cb, s_amax); break;
                default: gemm1_fp8_task<4>(a, e, row0, cb, s_amax); break;
            }
        } else {
            constexpr bool F32X = MODE == MOE_MODE_F32ACT;
            switch (nsub) {
                case 1: gemm1_bf16_task<1, F32X>(a, e, row0, cb); break;
                case 2: gemm1_bf16_task<2, F32X>(a, e, row0, cb); break;
                case 3: gemm1_bf16_task<3, F32X>(a, e, row0, cb); break;
                default: gemm1_bf16_task<4, F32X>(a, e, row0, cb); break;
            }
        }
    }
}

// ---------------------------------------------------------------- GEMM-2 FP8
// Task: 16*NSUB rows x 128 output columns; wave w owns [32w, 32w+32).
template <int NSUB, int NF, bool F32OUT>
__device__ __forceinline__ void store_y(const Gemm2Args& a, const v4f (&acc)[NSUB][2], int row0, int col0, int lg,
                                        int lr) {
    const int d_h = a.d_h;
#pragma unroll
    for (int s = 0; s < NSUB; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = a.row_src[row0 + 16 * s + 4 * lg + i];
            if (p < 0) continue;
            const float wt = a.topk_w[p];
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const float v = acc[s][f][i] * wt;
                const int64_t off = (int64_t)p * d_h + col0 + 16 * f + lr;
                if (F32OUT)
                    static_cast<float*>(a.y)[off] = v;
                else
                    static_cast<unsigned short*>(a.y)[off] = f32_to_bf16(v);
            }
        }
}

template <int NSUB>
__device__ __forceinline__ void gemm2_fp8_task(const Gemm2Args& a, int e, int row0, int cb) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int d_h = a.d_h, d_e = a.d_e, kq = d_e / kQ;
    const unsigned char* h = static_cast<const unsigned char*>(a.h);
    const unsigned char* w2 = static_cast<const unsigned char*>(a.w2);

    const unsigned char* pa[NSUB];
    const float* psh[NSUB][4];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
        pa[s] = h + (int64_t)(row0 + 16 * s + lr) * d_e + lg * 32;
#pragma unroll
        for (int i = 0; i < 4; ++i) psh[s][i] = a.h_scale + (int64_t)(row0 + 16 * s + 4 * lg + i) * kq;
    }
    const unsigned char* pb[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) pb[f] = w2 + ((int64_t)e * d_h + cb * 128 + w * 32 + 16 * f + lr) * d_e + lg * 32;
    const float* psw = a.w2_scale + ((int64_t)e * (d_h / kQ) + cb) * kq;

    v4f acc[NSUB][2];
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NSUB; ++s) acc[s][0] = acc[s][1] = zero;
    v8i A[NSUB], B[2];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) A[s] = ld32(pa[s]);
#pragma unroll
    for (int f = 0; f < 2; ++f) B[f] = ld32(pb[f]);
    for (int kb = 0; kb < kq; ++kb) {
        const int kn = (kb + 1 < kq ? kb + 1 : kb) * kQ;
        v8i An[NSUB], Bn[2];
#pragma unroll
        for (int s = 0; s < NSUB; ++s) An[s] = ld32(pa[s] + kn);
#pragma unroll
        for (int f = 0; f < 2; ++f) Bn[f] = ld32(pb[f] + kn);
        const float sw = psw[kb];
        float sh[NSUB][4];
#pragma unroll
        for (int s = 0; s < NSUB; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) sh[s][i] = psh[s][i][kb] * sw;
#pragma unroll
        for (int s = 0; s < NSUB; ++s)
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                const v4f t = mfma_fp8(A[s], B[f], zero);
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[s][f][i] += t[i] * sh[s][i];
            }
#pragma unroll
        for (int s = 0; s < NSUB; ++s) A[s] = An[s];
#pragma unroll
        for (int f = 0; f < 2; ++f) B[f] = Bn[f];
    }
    store_y<NSUB, 2, false>(a, acc, row0, cb * 128 + w * 32, lg, lr);
}

// --------------------------------------------------------------- GEMM-2 bf16
// Task: 16*NSUB rows x 64 output columns; wave w owns [16w, 16w+16).
template <int NSUB, bool F32OUT>
__device__ __forceinline__ void gemm2_bf16_task(const Gemm2Args& a, int e, int row0, int cb) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    const int d_h = a.d_h, d_e = a.d_e;
    const unsigned short* h = static_cast<const unsigned short*>(a.h);
    const unsigned short* w2 = static_cast<const unsigned short*>(a.w2);
    const unsigned short* pa[NSUB];
#pragma unroll
    for (int s = 0; s < NSUB; ++s) pa[s] = h + (int64_t)(row0 + 16 * s + lr) * d_e + lg * 16;
    const unsigned short* pb = w2 + ((int64_t)e * d_h + cb * 64 + w * 16 + lr) * d_e + lg * 16;

    v4f acc[NSUB][2];
    const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NSUB; ++s) acc[s][0] = acc[s][1] = zero;
    const int nk = d_e / 64;
    Bf16x16 A[NSUB], B;
#pragma unroll
    for (int s = 0; s < NSUB; ++s) A[s] = ld_bf16x16(pa[s]);
    B = ld_bf16x16(pb);
    for (int kc = 0; kc < nk; ++kc) {
        const int kn = (kc + 1 < nk ? kc + 1 : kc) * 64;
        Bf16x16 An[NSUB];
#pragma unroll
        for (int s = 0; s < NSUB; ++s) An[s] = ld_bf16x16(pa[s] + kn);
        const Bf16x16 Bn = ld_bf16x16(pb + kn);
#pragma unroll
        for (int s = 0; s < NSUB; ++s) {
            acc[s][0] = mfma_bf16(A[s].lo, B.lo, acc[s][0]);
            acc[s][0] = mfma_bf16(A[s].hi, B.hi, acc[s][0]);
        }
#pragma unroll
        for (int s = 0; s < NSUB; ++s) A[s] = An[s];
        B = Bn;
    }
    store_y<NSUB, 1, F32OUT>(a, acc, row0, cb * 64 + w * 16, lg, lr);
}

template <int MODE>
__global__ __launch_bounds__(kGemmThreads) void gemm2_kernel(Gemm2Args a) {
    __shared__ int s_slot;
    const int ntasks = a.stats[kStatTasks2];
    for (;;) {
        const int t = pull_task(&a.stats[kStatCounter2], &s_slot);
        if (t >= ntasks) break;
        const int4 task = a.tasks[t];
        const int e = task.x, row0 = task.y, nsub = task.z, cb = task.w;
        if constexpr (MODE == MOE_MODE_FP8) {
            switch (nsub) {
                case 1: gemm2_fp8_task<1>(a, e, row0, cb); break;
                case 2: gemm2_fp8_task<2>(a, e, row0, cb); break;
                case 3: gemm2_fp8_task<3>(a, e, row0, cb); break;
                default: gemm2_fp8_task<4>(a, e, row0, cb); break;
            }
        } else {
            constexpr bool F32OUT = MODE == MOE_MODE_F32ACT;
            switch (nsub) {
                case 1: gemm2_bf16_task<1, F32OUT>(a, e, row0, cb); break;
                case 2: gemm2_bf16_task<2, F32OUT>(a, e, row0, cb); break;
                case 3: gemm2_bf16_task<3, F32OUT>(a, e, row0, cb); break;
                default: gemm2_bf16_task<4, F32OUT>(a, e, row0, cb); break;
            }
        }
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
    for (int j = 0; j < a.k; ++j) {
        const int64_t p = (int64_t)t * a.k + j;
        const int id = a.ids[p];
        if ((unsigned)id >= (unsigned)a.E) continue;
        if (F32) {
            const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(a.y) + p * a.d_h + c);
            const float4 u = src[0], v = src[1];
            acc[0] += u.x; acc[1] += u.y; acc[2] += u.z; acc[3] += u.w;
            acc[4] += v.x; acc[5] += v.y; acc[6] += v.z; acc[7] += v.w;
        } else {
            const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const unsigned short*>(a.y) + p * a.d_h + c);
            const unsigned wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] += __uint_as_float(wd[i] << 16);
                acc[2 * i + 1] += __uint_as_float(wd[i] & 0xFFFF0000u);
            }
        }
    }
    if (F32) {
        float4* dst = reinterpret_cast<float4*>(static_cast<float*>(a.out) + (int64_t)t * a.d_h + c);
        dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
        dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
    } else {
        uint4 o;
        o.x = f32_to_bf16(acc[0]) | ((unsigned)f32_to_bf16(acc[1]) << 16);
        o.y = f32_to_bf16(acc[2]) | ((unsigned)f32_to_bf16(acc[3]) << 16);
        o.z = f32_to_bf16(acc[4]) | ((unsigned)f32_to_bf16(acc[5]) << 16);
        o.w = f32_to_bf16(acc[6]) | ((unsigned)f32_to_bf16(acc[7]) << 16);
        *reinterpret_cast<uint4*>(static_cast<unsigned short*>(a.out) + (int64_t)t * a.d_h + c) = o;
    }
}

}  // namespace

hipError_t launch_gemm1(int mode, const Gemm1Args& a, int grid, hipStream_t s) {
    if (mode == MOE_MODE_FP8)
        hipLaunchKernelGGL(gemm1_kernel<MOE_MODE_FP8>, dim3(grid), dim3(kGemmThreads), 0, s, a);
    else if (mode == MOE_MODE_BF16)
        hipLaunchKernelGGL(gemm1_kernel<MOE_MODE_BF16>, dim3(grid), dim3(kGemmThreads), 0, s, a);
    else
        hipLaunchKernelGGL(gemm1_kernel<MOE_MODE_F32ACT>, dim3(grid), dim3(kGemmThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_gemm2(int mode, const Gemm2Args& a, int grid, hipStream_t s) {
    if (mode == MOE_MODE_FP8)
        hipLaunchKernelGGL(gemm2_kernel<MOE_MODE_FP8>, dim3(grid), dim3(kGemmThreads), 0, s, a);
    else if (mode == MOE_MODE_BF16)
        hipLaunchKernelGGL(gemm2_kernel<MOE_MODE_BF16>, dim3(grid), dim3(kGemmThreads), 0, s, a);
    else
        hipLaunchKernelGGL(gemm2_kernel<MOE_MODE_F32ACT>, dim3(grid), dim3(kGemmThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_combine(int mode, const CombineArgs& a, hipStream_t s) {
    const int64_t n = (int64_t)a.T * (a.d_h / 8);
    const int blocks = (int)((n + 255) / 256);
    if (blocks == 0) return hipSuccess;
    if (mode == MOE_MODE_F32ACT)
        hipLaunchKernelGGL(combine_kernel<true>, dim3(blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(combine_kernel<false>, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t gemm_occupancy(int mode, int* g1, int* g2) {
    hipError_t e1, e2;
    if (mode == MOE_MODE_FP8) {
        e1 = hipOccupancyMaxActiveBlocksPerMultiprocessor(g1, gemm1_kernel<MOE_MODE_FP8>, kGemmThreads, 0);
        e2 = hipOccupancyMaxActiveBlocksPerMultiprocessor(g2, gemm2_kernel<MOE_MODE_FP8>, kGemmThreads, 0);
    } else if (mode == MOE_MODE_BF16) {
        e1 = hipOccupancyMaxActiveBlocksPerMultiprocessor(g1, gemm1_kernel<MOE_MODE_BF16>, kGemmThreads, 0);
        e2 = hipOccupancyMaxActiveBlocksPerMultiprocessor(g2, gemm2_kernel<MOE_MODE_BF16>, kGemmThreads, 0);
    } else {
        e1 = hipOccupancyMaxActiveBlocksPerMultiprocessor(g1, gemm1_kernel<MOE_MODE_F32ACT>, kGemmThreads, 0);
        e2 = hipOccupancyMaxActiveBlocksPerMultiprocessor(g2, gemm2_kernel<MOE_MODE_F32ACT>, kGemmThreads, 0);
    }
    return e1 != hipSuccess ? e1 : e2;
}

}  // namespace moe
