// Backward pass of the fused MoE layer with recompute (BF16 mode) on gfx950.
//
// The MoE megakernel on the PipeLink page (section 5.3) serves forward,
// backward and recompute passes; this is the backward of the layer of
// tilelang.dataflow section 3.5 by the chain rule, with g, u and h recomputed
// from x and W1 instead of being kept from the forward.  For each routed row
// p (token t, expert e, weight w):
//   recompute   [g u] = x_t . W1[e]^T,  h = bf16(silu(g) u)
//   q = dout_t . W2[e]                 (the unweighted gradient of h)
//   dtopk_w[p] = <q, h>;  dh = w q;  dg = bf16(dh u silu'(g)),  du = bf16(dh silu(g))
//   dX_p = [dg du] . W1[e]             dx_t = sum over the token's slots, ascending j
//   dW1[e] = sum_p [dg du]^T x_t       dW2[e] = sum_p bf16(w dout_t)^T h
// All GEMMs are bf16 16x16x32 MFMAs with fp32 accumulation, written as
// C = A . B^T with both operands K-contiguous: the row GEMMs run per 16-row
// group block of the padded layout (gathered token rows or the layer's own
// rows, one expert's weight rows), the weight GEMMs per expert with K running
// over the expert's padded rows of transposed operands.  Transposes go
// through LDS tiles.  These kernels favour simplicity over speed: one K step
// of 32 values per barrier pair, no ring.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ unsigned f32_to_bf16(float f) {
    unsigned u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ float bf16_to_f32(unsigned short b) { return __uint_as_float((unsigned)b << 16); }

// --------------------------------------------------------------- GEMM
// C[m][n] = sum_k A[m][k] B[n][k], bf16 operands (K contiguous), fp32 C.
// ROWS mode: the M rows are one 16-row group block i of the padded layout
//   (expert tile_expert[i], first row tile_row0[i]); A row r is the token row
//   a_rows[r] / a_div of A (zeros for a padding row) when a_rows is set, else
//   row r of A; B is expert e's matrix (B + e * b_estride); the tile covers 64
//   output columns; K = [0, K).
// EXPERT mode: block (e, m-tile, n-tile) of 64 x 64; A and B rows are m and n;
//   K = [poff[e], poff[e+1]) (an expert's padded rows), values past the end
//   read as zero; C = C + e * c_estride.  An expert with no rows stores zeros.
struct BwdGemmArgs {
    const uint16_t* A;
    int64_t lda;
    const int32_t* a_rows;
    int32_t a_div;
    const uint16_t* B;
    int64_t ldb, b_estride;
    float* C;
    int64_t ldc, c_estride;
    int32_t N, K;
    const int32_t* tile_expert;
    const int32_t* tile_row0;
    const int32_t* ctl;   // ctl[kStatTiles]: group blocks in use
    const int32_t* poff;  // padded offsets [E+1]
};

constexpr int kBwdThreads = 256;
constexpr int kLdsRow = 40;  // bf16 per LDS row: 32 values + 8 of padding (no bank conflicts on fragment reads)

__device__ __forceinline__ v4f mfma_bf16(const v4i& a, const v4i& b, const v4f& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c, 0,
                                                   0, 0);
}

template <bool EXPERT>
__global__ __launch_bounds__(kBwdThreads) void bwd_gemm_kernel(BwdGemmArgs a) {
    constexpr int BM = EXPERT ? 64 : 16;
    __shared__ __attribute__((aligned(16))) uint16_t sA[BM * kLdsRow];
    __shared__ __attribute__((aligned(16))) uint16_t sB[64 * kLdsRow];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lr = lane & 15, lg = lane >> 4;
    int e, m0, n0, k0, k1;
    if constexpr (EXPERT) {
        e = blockIdx.x;
        m0 = 64 * blockIdx.y;
        n0 = 64 * blockIdx.z;
        k0 = a.poff[e];
        k1 = a.poff[e + 1];
    } else {
        const int i = blockIdx.x;
        if (i >= a.ctl[kStatTiles]) return;
        e = a.tile_expert[i];
        m0 = a.tile_row0[i];
        n0 = 64 * blockIdx.y;
        k0 = 0;
        k1 = a.K;
    }
    // this thread's 16-byte piece of each tile: row tid / 4, 8 values at 8 * (tid % 4)
    const int lrow = tid >> 2, lch = tid & 3;
    const uint16_t* arow = nullptr;
    if (lrow < BM) {
        if constexpr (EXPERT) {
            arow = a.A + (int64_t)(m0 + lrow) * a.lda;
        } else if (a.a_rows) {
            const int p = a.a_rows[m0 + lrow];
            arow = p >= 0 ? a.A + (int64_t)(p / a.a_div) * a.lda : nullptr;
        } else {
            arow = a.A + (int64_t)(m0 + lrow) * a.lda;
        }
    }
    const uint16_t* brow =
        EXPERT ? a.B + (int64_t)(n0 + lrow) * a.ldb : a.B + (int64_t)e * a.b_estride + (int64_t)(n0 + lrow) * a.ldb;
    constexpr int NF = EXPERT ? 4 : 1;  // 16-column fragments per wave
    v4f acc[NF];
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[f] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int k = k0; k < k1; k += 32) {
        const int kk = k + 8 * lch;
        const bool in = kk < k1;  // K ranges are multiples of 16, pieces are 8 values
        const v4i z = {0, 0, 0, 0};
        if (lrow < BM) {
            const v4i va = (arow && in) ? *reinterpret_cast<const v4i*>(arow + kk) : z;
            *reinterpret_cast<v4i*>(&sA[lrow * kLdsRow + 8 * lch]) = va;
        }
        const v4i vb = in ? *reinterpret_cast<const v4i*>(brow + kk) : z;
        *reinterpret_cast<v4i*>(&sB[lrow * kLdsRow + 8 * lch]) = vb;
        __syncthreads();
        const int ar = EXPERT ? 16 * w + lr : lr;
        const v4i fa = *reinterpret_cast<const v4i*>(&sA[ar * kLdsRow + 8 * lg]);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const int br = EXPERT ? 16 * f + lr : 16 * w + lr;
            const v4i fb = *reinterpret_cast<const v4i*>(&sB[br * kLdsRow + 8 * lg]);
            acc[f] = mfma_bf16(fa, fb, acc[f]);
        }
        __syncthreads();
    }
    // lane (lr, lg) holds C[4 lg + i][lr] of each 16 x 16 fragment
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (EXPERT) {
                const int64_t m = m0 + 16 * w + 4 * lg + i, n = n0 + 16 * f + lr;
                a.C[(int64_t)e * a.c_estride + m * a.ldc + n] = acc[f][i];
            } else {
                const int64_t m = m0 + 4 * lg + i, n = n0 + 16 * w + lr;
                a.C[m * a.ldc + n] = acc[f][i];
            }
        }
}

// --------------------------------------------------------------- transpose
// out[b][c][r] = v(b, r, c) for r < R, c < C (64 x 64 tiles through LDS):
//   v = in[b][src(r)][c], src(r) = rows ? rows[r] / map_div : r; with rows set,
//   r >= poff[E] (past the padded rows in use) or rows[r] < 0 gives 0; with
//   roww, v = bf16(roww[rows[r]] * in), the routing weight of the row's assignment.
struct TransArgs {
    const uint16_t* in;
    int64_t ldi, in_bstride;
    uint16_t* out;
    int64_t ldo, out_bstride;
    int32_t R, C;
    const int32_t* rows;
    int32_t map_div;
    const float* roww;
    const int32_t* n_used;  // rows >= *n_used are written as zeros (may be null)
};

__global__ __launch_bounds__(256) void transpose_kernel(TransArgs a) {
    // 64 x 64 tile; every global access is 16 bytes (8 values): a thread loads
    // two 8-value pieces of input rows and writes two 8-value pieces of output
    // rows gathered from a column of the LDS tile
    __shared__ __attribute__((aligned(16))) uint16_t t[64][72];
    const int r0 = 64 * blockIdx.y, c0 = 64 * blockIdx.x;
    const int64_t b = blockIdx.z;
    const int nu = a.n_used ? *a.n_used : a.R;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int piece = threadIdx.x + 256 * h;  // 512 pieces: 64 rows x 8
        const int i = piece >> 3, c = 8 * (piece & 7);
        const int r = r0 + i;
        v4i v = {0, 0, 0, 0};
        if (r < a.R && r < nu && c0 + c < a.C) {
            int64_t src = r;
            bool ok = true;
            float sc = 1.f;
            if (a.rows) {
                const int p = a.rows[r];
                ok = p >= 0;
                src = ok ? p / a.map_div : 0;
                if (ok && a.roww) sc = a.roww[p];
            }
            if (ok) {
                v = *reinterpret_cast<const v4i*>(a.in + b * a.in_bstride + src * a.ldi + c0 + c);
                if (a.roww) {
                    unsigned wd[4] = {(unsigned)v.x, (unsigned)v.y, (unsigned)v.z, (unsigned)v.w};
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const unsigned lo = f32_to_bf16(sc * bf16_to_f32((uint16_t)(wd[q] & 0xffffu)));
                        const unsigned hi = f32_to_bf16(sc * bf16_to_f32((uint16_t)(wd[q] >> 16)));
                        wd[q] = lo | (hi << 16);
                    }
                    v = v4i{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
                }
            }
        }
        *reinterpret_cast<v4i*>(&t[i][c]) = v;
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int piece = threadIdx.x + 256 * h;  // 64 output rows (c) x 8 pieces of 8 r's
        const int ci = piece >> 3, rr = 8 * (piece & 7);
        const int c = c0 + ci, r = r0 + rr;
        if (c >= a.C || r >= a.R) continue;
        uint16_t* dst = a.out + b * a.out_bstride + (int64_t)c * a.ldo + r;
        if (r + 8 <= a.R) {
            unsigned wd[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) wd[q] = (unsigned)t[rr + 2 * q][ci] | ((unsigned)t[rr + 2 * q + 1][ci] << 16);
            *reinterpret_cast<v4i*>(dst) = v4i{(int)wd[0], (int)wd[1], (int)wd[2], (int)wd[3]};
        } else {
            for (int q = 0; q < 8 && r + q < a.R; ++q) dst[q] = t[rr + q][ci];
        }
    }
}

// ------------------------------------------------------------ activation
// One workgroup per padded row r below padded_offsets[E]: from the recomputed
// GU = [g u] (fp32 [n_pad, 2 d_e]) and q (fp32 [n_pad, d_e]) form h (bf16),
// dg and du (bf16, [n_pad, 2 d_e]) and dtopk_w of the row's assignment (a
// fixed-order reduction); padding rows get zeros.
struct ActArgs {
    const float* GU;
    const float* Q;
    const int32_t* row_src;
    const int32_t* poff_end;  // &padded_offsets[E]
    const float* topk_w;
    uint16_t* H;
    uint16_t* dGU;
    float* dtopk_w;
    int32_t d_e;
};

__global__ __launch_bounds__(256) void bwd_act_kernel(ActArgs a) {
    __shared__ float part[4];
    const int r = blockIdx.x;
    if (r >= *a.poff_end) return;
    const int p = a.row_src[r];
    const int d_e = a.d_e;
    const float wt = p >= 0 ? a.topk_w[p] : 0.f;
    float dot = 0.f;
    for (int c = threadIdx.x; c < d_e; c += blockDim.x) {
        uint16_t hb = 0, gb = 0, ub = 0;
        if (p >= 0) {
            const float g = a.GU[(int64_t)r * 2 * d_e + c], u = a.GU[(int64_t)r * 2 * d_e + d_e + c];
            const float q = a.Q[(int64_t)r * d_e + c];
            const float sig = 1.0f / (1.0f + expf(-g));
            const float silu = g * sig;
            const float h = bf16_to_f32((uint16_t)f32_to_bf16((g / (1.0f + expf(-g))) * u));
            hb = (uint16_t)f32_to_bf16(h);
            dot += q * h;
            const float dh = wt * q;
            const float dsilu = sig * (1.0f + g * (1.0f - sig));
            gb = (uint16_t)f32_to_bf16((dh * u) * dsilu);
            ub = (uint16_t)f32_to_bf16(dh * silu);
        }
        a.H[(int64_t)r * d_e + c] = hb;
        a.dGU[(int64_t)r * 2 * d_e + c] = gb;
        a.dGU[(int64_t)r * 2 * d_e + d_e + c] = ub;
    }
    // fixed-order sum: within the wave by halving offsets, then the 4 waves in order
    for (int off = 32; off > 0; off >>= 1) dot += __shfl_down(dot, off, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = dot;
    __syncthreads();
    if (threadIdx.x == 0 && p >= 0) a.dtopk_w[p] = ((part[0] + part[1]) + part[2]) + part[3];
}

// ---------------------------------------------------------------- dx
// dx[t][c..c+4) = sum over the token's valid slots (ascending j) of the rows
// dXp[ppos[t k + j]]; a dropped slot gets dtopk_w = 0.
struct DxArgs {
    const float* dXp;
    const int32_t* ppos;
    const int32_t* ids;
    float* dx;
    float* dtopk_w;
    int32_t T, k, E, d_h;
};

__global__ __launch_bounds__(256) void bwd_dx_kernel(DxArgs a) {
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int cpr = a.d_h / 4;
    if (gid >= (int64_t)a.T * cpr) return;
    const int t = (int)(gid / cpr);
    const int c = (int)(gid - (int64_t)t * cpr) * 4;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < a.k; ++j) {
        const int64_t p = (int64_t)t * a.k + j;
        if ((unsigned)a.ids[p] >= (unsigned)a.E) {
            if (c == 0) a.dtopk_w[p] = 0.f;
            continue;
        }
        const float4 v = *reinterpret_cast<const float4*>(a.dXp + (int64_t)a.ppos[p] * a.d_h + c);
        s.x += v.x;
        s.y += v.y;
        s.z += v.z;
        s.w += v.w;
    }
    *reinterpret_cast<float4*>(a.dx + (int64_t)t * a.d_h + c) = s;
}

}  // namespace

hipError_t launch_bwd_gemm_rows(const uint16_t* A, int64_t lda, const int32_t* a_rows, int a_div, const uint16_t* B,
                                int64_t ldb, int64_t b_estride, float* C, int64_t ldc, int N, int K,
                                const int32_t* tile_expert, const int32_t* tile_row0, const int32_t* ctl,
                                int64_t tile_cap, hipStream_t s) {
    if (tile_cap <= 0) return hipSuccess;
    BwdGemmArgs a{};
    a.A = A;
    a.lda = lda;
    a.a_rows = a_rows;
    a.a_div = a_div;
    a.B = B;
    a.ldb = ldb;
    a.b_estride = b_estride;
    a.C = C;
    a.ldc = ldc;
    a.N = N;
    a.K = K;
    a.tile_expert = tile_expert;
    a.tile_row0 = tile_row0;
    a.ctl = ctl;
    hipLaunchKernelGGL(bwd_gemm_kernel<false>, dim3((unsigned)tile_cap, (unsigned)(N / 64)), dim3(kBwdThreads), 0, s,
                       a);
    return hipGetLastError();
}

hipError_t launch_bwd_gemm_experts(const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb, float* C,
                                   int64_t ldc, int64_t c_estride, int E, int M, int N, const int32_t* poff,
                                   hipStream_t s) {
    BwdGemmArgs a{};
    a.A = A;
    a.lda = lda;
    a.B = B;
    a.ldb = ldb;
    a.C = C;
    a.ldc = ldc;
    a.c_estride = c_estride;
    a.N = N;
    a.poff = poff;
    hipLaunchKernelGGL(bwd_gemm_kernel<true>, dim3((unsigned)E, (unsigned)(M / 64), (unsigned)(N / 64)),
                       dim3(kBwdThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_transpose(const uint16_t* in, int64_t ldi, int64_t in_bstride, uint16_t* out, int64_t ldo,
                            int64_t out_bstride, int R, int C, int batch, const int32_t* rows, int map_div,
                            const float* roww, const int32_t* n_used, hipStream_t s) {
    if (R <= 0 || C <= 0 || batch <= 0) return hipSuccess;
    TransArgs a{in, ldi, in_bstride, out, ldo, out_bstride, R, C, rows, map_div, roww, n_used};
    hipLaunchKernelGGL(transpose_kernel, dim3((unsigned)((C + 63) / 64), (unsigned)((R + 63) / 64), (unsigned)batch),
                       dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_bwd_act(const float* GU, const float* Q, const int32_t* row_src, const int32_t* poff_end,
                          const float* topk_w, uint16_t* H, uint16_t* dGU, float* dtopk_w, int d_e, int64_t n_pad_cap,
                          hipStream_t s) {
    if (n_pad_cap <= 0) return hipSuccess;
    ActArgs a{GU, Q, row_src, poff_end, topk_w, H, dGU, dtopk_w, d_e};
    hipLaunchKernelGGL(bwd_act_kernel, dim3((unsigned)n_pad_cap), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_bwd_dx(const float* dXp, const int32_t* ppos, const int32_t* ids, float* dx, float* dtopk_w, int T,
                         int k, int E, int d_h, hipStream_t s) {
    const int64_t n = (int64_t)T * (d_h / 4);
    if (n == 0) return hipSuccess;
    DxArgs a{dXp, ppos, ids, dx, dtopk_w, T, k, E, d_h};
    hipLaunchKernelGGL(bwd_dx_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace moe
