/*
 * moe_oracle.c -- plain, slow CPU oracle of the fused MoE forward layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls this file;
 * only the test-suite, the smoke check and the benchmark's CPU-baseline leg
 * load it.  It shares no code, header or table with the HIP path.
 *
 * What it computes (tilelang.dataflow README, section 3.5 "Fused MoE: map ->
 * reshared -> map"): tokens are grouped by expert from their routing
 * metadata, GEMM-1 applies the gate and up shards of the expert's weights and
 * forms the gated intermediate, GEMM-2 applies the down projection, scales by
 * the routing weight and the rows are written back per token.  The result is
 * the plain MoE definition
 *
 *     out[t] = sum_{j<k} w[t,j] * W2[e] . ( silu(W1g[e] . x[t]) * (W1u[e] . x[t]) ),
 *     e = ids[t,j],
 *
 * with the activation taken on the unrounded fp32 accumulator (PipeLink,
 * section 5.5 "Fused GEMM and Activation": the FP32 accumulator stays
 * unrounded through the activation, the activation is then stored as BF16).
 *
 * Precision: arithmetic is fp32 (the accumulator precision the pages name).
 * Every operation is evaluated in double and rounded to float right after
 * (exact emulation of fp32 +,-,*,/ because 53 >= 2*24+2).  Flag
 * ORACLE_ACC64 skips that rounding so the same code runs in fp64; the
 * fp32-vs-fp64 gap bounds the oracle's own rounding error.
 *
 * Reading of the pages where they are silent (each listed in the design
 * notes): OCP E4M3FN is the FP8 format; dequantisation is code * fp32 scale;
 * in FP8 mode the intermediate is requantised per row per 128 columns with
 * scale amax/448; ids outside [0,E) are dropped; the top-k sum runs in
 * ascending slot order from +0.0 with one final rounding.
 *
 * MXFP8 mode (the pages name MXFP8 as a variant of the Mixture-of-Kittens MoE
 * kernels, PipeLink section 5.3, without defining it; the definition taken is
 * the OCP Microscaling (MX) format): E4M3FN elements in blocks of 32
 * consecutive values along the reduction dimension, each block with one
 * E8M0 scale (value 2^(s-127), s = 255 is NaN); dequantised value = element *
 * scale.  The intermediate is requantised per row per 32 columns with the
 * shared exponent floor(log2(amax)) - 8 (8 = the largest E4M3 exponent) and
 * saturating round-to-nearest-even elements.
 *
 * INT8 mode (tokens quantised to int8 before the expert GEMMs, which
 * dequantise them: the CUCo page, section 4 "Evaluation", DeepSeek-V3 MoE
 * Dispatch and Combine, steps (1) and (3); the page fixes neither the
 * granularity nor the weights' type): one fp32 scale per token, dequantised
 * value = int8 code * scale; the weights are bf16 (the page computes in a
 * higher precision than the tokens travel in) and the intermediate is
 * rounded to bf16 as in BF16 mode.
 *
 * Clamped activation (flag ORACLE_ACT_CLAMPED; the pages name the GPT-OSS
 * variant of SwiGLU as an independent activation owner, PipeLink section 5.3,
 * without defining it; the definition taken is the published GPT-OSS one):
 * the gate is clamped above at 7, the up value to [-7, 7], and
 *     h = gate * sigmoid(1.702 * gate) * (up + 1).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENOMEM 2

/* modes: which dtypes the layer is fed */
#define ORACLE_MODE_F32ACT 0 /* x fp32, W bf16, out fp32 */
#define ORACLE_MODE_BF16 1   /* x bf16, W bf16, out bf16 */
#define ORACLE_MODE_FP8 2    /* x e4m3 + scales, W e4m3 + 128x128 block scales, out bf16 */
#define ORACLE_MODE_MXFP8 3  /* x, W e4m3 with E8M0 scales per 32 along the reduction dimension, out bf16 */
#define ORACLE_MODE_INT8 4   /* x int8 codes + one fp32 scale per token, W bf16, out bf16 */

/* flags */
#define ORACLE_MIRROR_H 1 /* round the intermediate where the method stores it */
#define ORACLE_ACC64 2    /* evaluate in fp64 instead of fp32 */
#define ORACLE_ACT_CLAMPED 4 /* clamped activation (GPT-OSS variant) in place of SwiGLU */
#define ACT_LIMIT 7.0        /* clamp bound of the clamped activation */
#define ACT_ALPHA 1.702f     /* sigmoid slope of the clamped activation (an fp32 constant) */

#define QBLK 128 /* block-scale granularity along every dimension */
#define MXBLK 32 /* MX block: values along the reduction dimension sharing one scale */

/* ------------------------------------------------------------------ codecs */

/* OCP 8-bit floating point, E4M3FN variant: 1 sign bit, 4 exponent bits with
 * bias 7, 3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6;
 * S.1111.111 is NaN; there is no infinity; the largest finite value is 448. */
double oracle_e4m3_decode(uint8_t code) {
    int sign = code >> 7;
    int ex = (code >> 3) & 15;
    int man = code & 7;
    double mag;
    if (ex == 15 && man == 7) return NAN;
    if (ex == 0)
        mag = ldexp((double)man / 8.0, -6);
    else
        mag = ldexp(1.0 + (double)man / 8.0, ex - 7);
    return sign ? -mag : mag;
}

/* The 256 decoded values, filled once from the definition above so the
 * inner loops below index a table instead of re-deriving each value. */
static double e4m3_table[256];
static int e4m3_table_ready = 0;

static void oracle_init(void) {
    int c;
    if (e4m3_table_ready) return;
    for (c = 0; c < 256; ++c) e4m3_table[c] = oracle_e4m3_decode((uint8_t)c);
    e4m3_table_ready = 1;
}

/* Nearest E4M3FN code to v, ties to the code with an even mantissa field;
 * finite magnitudes above 448 saturate to 448; NaN maps to 0x7F.  Written as a
 * search over the 127 non-negative finite codes so it follows the format's
 * definition directly. */
uint8_t oracle_e4m3_encode(double v) {
    uint8_t sign;
    double a, best_d;
    int c, best;
    oracle_init();
    if (isnan(v)) return 0x7F;
    sign = signbit(v) ? 0x80 : 0x00;
    a = fabs(v);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    best = 0;
    best_d = a; /* distance to code 0 */
    for (c = 1; c <= 0x7E; ++c) {
        double d = fabs(e4m3_table[c] - a);
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best_d = d;
            best = c;
        }
    }
    return (uint8_t)(sign | best);
}

/* OCP E8M0 scale: an 8-bit biased exponent, value 2^(s-127); 255 is NaN. */
double oracle_e8m0_decode(uint8_t s) { return s == 255 ? NAN : ldexp(1.0, (int)s - 127); }

/* bfloat16: the upper 16 bits of an IEEE binary32.  Encoding rounds the
 * binary32 value to nearest with ties to even on the dropped 16 bits; NaN
 * stays a quiet NaN. */
uint16_t oracle_bf16_encode(float f) {
    uint32_t u, lsb;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
    lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

float oracle_bf16_decode(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ------------------------------------------------------------- arithmetic */

/* One rounding step: to binary32 unless the fp64 flag is set. */
static inline double R(double v, int f64) { return f64 ? v : (double)(float)v; }

/* Per-row-per-128 requantisation of a chunk of the intermediate (FP8 mode):
 * s = amax / 448 (s = 1 for an all-zero chunk); value -> decode(encode(v/s)) * s.
 * Exported for the tests. */
void oracle_requant_chunk(double* a, int64_t n, int f64) {
    double amax = 0.0, s;
    int64_t i;
    oracle_init();
    for (i = 0; i < n; ++i)
        if (fabs(a[i]) > amax) amax = fabs(a[i]);
    s = amax > 0.0 ? R(amax / 448.0, f64) : 1.0;
    for (i = 0; i < n; ++i) {
        double q = e4m3_table[oracle_e4m3_encode(R(a[i] / s, f64))];
        a[i] = R(q * s, f64);
    }
}

/* MX requantisation of one block of the intermediate (MXFP8 mode): shared
 * exponent X = floor(log2(amax)) - 8, stored as the E8M0 byte X + 127 clamped
 * to [0, 254] (byte 127 for an all-zero block); value -> decode(encode(v /
 * 2^X)) * 2^X, the encode saturating at 448.  The division and product by a
 * power of two are exact.  Writes the scale byte to *scale if non-NULL.
 * Exported for the tests. */
void oracle_mx_requant_block(double* a, int64_t n, uint8_t* scale) {
    double amax = 0.0, sc;
    int64_t i;
    int ex = 0, b = 127;
    oracle_init();
    for (i = 0; i < n; ++i)
        if (fabs(a[i]) > amax) amax = fabs(a[i]);
    if (amax > 0.0) {
        frexp(amax, &ex); /* amax = f * 2^ex, f in [0.5, 1): floor(log2(amax)) = ex - 1 */
        b = ex - 1 - 8 + 127;
        if (b < 0) b = 0;
        if (b > 254) b = 254;
    }
    sc = ldexp(1.0, b - 127);
    for (i = 0; i < n; ++i) a[i] = e4m3_table[oracle_e4m3_encode(a[i] / sc)] * sc;
    if (scale) *scale = (uint8_t)b;
}

/* Dequantised element loaders.  Scales are fp32 (FP8 mode) or E8M0 bytes
 * (MXFP8 mode), passed untyped. */
static inline double ld_x(int mode, int f64, const void* x, const void* xs, int64_t d_h, int64_t t, int64_t c) {
    if (mode == ORACLE_MODE_F32ACT) return ((const float*)x)[t * d_h + c];
    if (mode == ORACLE_MODE_BF16) return oracle_bf16_decode(((const uint16_t*)x)[t * d_h + c]);
    if (mode == ORACLE_MODE_INT8) /* x_scale [T]: one per token */
        return R((double)((const int8_t*)x)[t * d_h + c] * ((const float*)xs)[t], f64);
    if (mode == ORACLE_MODE_MXFP8)  /* x_scale [T, d_h/32] */
        return e4m3_table[((const uint8_t*)x)[t * d_h + c]] *
               oracle_e8m0_decode(((const uint8_t*)xs)[t * (d_h / MXBLK) + c / MXBLK]);
    return R(e4m3_table[((const uint8_t*)x)[t * d_h + c]] * ((const float*)xs)[t * (d_h / QBLK) + c / QBLK], f64);
}

/* W is [E, rows, cols] row-major (cols = the reduction dimension); FP8 scales
 * are [E, rows/128, cols/128], MXFP8 scales [E, rows, cols/32]. */
static inline double ld_w(int mode, int f64, const void* w, const void* ws, int64_t rows, int64_t cols,
                          int64_t e, int64_t r, int64_t c) {
    int64_t i = (e * rows + r) * cols + c;
    if (mode == ORACLE_MODE_MXFP8)
        return e4m3_table[((const uint8_t*)w)[i]] *
               oracle_e8m0_decode(((const uint8_t*)ws)[(e * rows + r) * (cols / MXBLK) + c / MXBLK]);
    if (mode != ORACLE_MODE_FP8) return oracle_bf16_decode(((const uint16_t*)w)[i]);
    return R(e4m3_table[((const uint8_t*)w)[i]] *
                 ((const float*)ws)[(e * (rows / QBLK) + r / QBLK) * (cols / QBLK) + c / QBLK],
             f64);
}

static int check_dims(int mode, int64_t T, int E, int k, int64_t d_h, int64_t d_e) {
    if (T < 0 || E < 1 || k < 1 || d_h < 1 || d_e < 1) return 0;
    if (mode < 0 || mode > 4) return 0;
    if (mode == ORACLE_MODE_FP8 && (d_h % QBLK || d_e % QBLK)) return 0;
    if (mode == ORACLE_MODE_MXFP8 && (d_h % MXBLK || d_e % MXBLK)) return 0;
    return 1;
}

/* Expert FFN of one assignment: y = W2[e] . (silu(g) * u), g and u from
 * W1[e] rows [0,d_e) and [d_e,2 d_e) (with ORACLE_ACT_CLAMPED the clamped
 * activation of g and u instead).  Accumulations run in ascending index
 * order.  a is scratch of d_e doubles, y receives d_h values. */
static void expert_ffn(int mode, int flags, int64_t d_h, int64_t d_e, const void* x, const void* xs, int64_t t,
                       const void* w1, const void* w1s, const void* w2, const void* w2s, int64_t e, double* a,
                       double* y) {
    int f64 = (flags & ORACLE_ACC64) != 0;
    int64_t r, c, n;
    for (r = 0; r < d_e; ++r) {
        double g = 0.0, u = 0.0, sg;
        for (c = 0; c < d_h; ++c) {
            double xv = ld_x(mode, f64, x, xs, d_h, t, c);
            g = R(g + R(ld_w(mode, f64, w1, w1s, 2 * d_e, d_h, e, r, c) * xv, f64), f64);
            u = R(u + R(ld_w(mode, f64, w1, w1s, 2 * d_e, d_h, e, d_e + r, c) * xv, f64), f64);
        }
        if (flags & ORACLE_ACT_CLAMPED) {
            /* g <- min(g, 7), u <- clamp(u, -7, 7): exact; then
             * g * sigmoid(alpha g) * (u + 1), sigmoid(z) = 1 / (1 + exp(-z)) */
            double z;
            if (g > ACT_LIMIT) g = ACT_LIMIT;
            if (u > ACT_LIMIT) u = ACT_LIMIT;
            if (u < -ACT_LIMIT) u = -ACT_LIMIT;
            z = R((double)ACT_ALPHA * g, f64);
            sg = f64 ? g / (1.0 + exp(-z)) : R(g * R(1.0 / R(1.0 + (double)expf((float)-z), 0), 0), 0);
            a[r] = R(sg * R(u + 1.0, f64), f64);
        } else {
            /* SiLU(g) = g / (1 + exp(-g)) */
            sg = f64 ? g / (1.0 + exp(-g)) : R(g / R(1.0 + (double)expf((float)-g), 0), 0);
            a[r] = R(sg * u, f64);
        }
    }
    if (flags & ORACLE_MIRROR_H) {
        if (mode == ORACLE_MODE_FP8) {
            for (r = 0; r < d_e; r += QBLK) oracle_requant_chunk(a + r, QBLK, f64);
        } else if (mode == ORACLE_MODE_MXFP8) {
            for (r = 0; r < d_e; r += MXBLK) oracle_mx_requant_block(a + r, MXBLK, NULL);
        } else {
            for (r = 0; r < d_e; ++r) a[r] = oracle_bf16_decode(oracle_bf16_encode((float)a[r]));
        }
    }
    for (n = 0; n < d_h; ++n) {
        double s = 0.0;
        for (r = 0; r < d_e; ++r) s = R(s + R(ld_w(mode, f64, w2, w2s, d_h, d_e, e, n, r) * a[r], f64), f64);
        y[n] = s;
    }
}

/*
 * Forward pass for the tokens listed in rows[0..nrows) (all T tokens when rows
 * is NULL, nrows then ignored).  out_acc [nrows, d_h] receives the fp32 (or
 * fp64) top-k sum before the final cast; out (optional) receives it cast to the
 * mode's output dtype (fp32 in F32ACT mode, bf16 bits otherwise).
 */
int moe_oracle_forward(int mode, int64_t T, int E, int k, int64_t d_h, int64_t d_e, const void* x,
                       const void* x_scale, const int32_t* topk_ids, const float* topk_w, const void* w1,
                       const void* w1_scale, const void* w2, const void* w2_scale, int flags,
                       const int64_t* rows, int64_t nrows, double* out_acc, void* out) {
    int64_t i;
    int f64 = (flags & ORACLE_ACC64) != 0;
    int failed = 0;
    if (!check_dims(mode, T, E, k, d_h, d_e)) return ORACLE_EINVAL;
    if (!x || !topk_ids || !topk_w || !w1 || !w2 || !out_acc) return ORACLE_EINVAL;
    if ((mode == ORACLE_MODE_FP8 || mode == ORACLE_MODE_MXFP8) && (!x_scale || !w1_scale || !w2_scale))
        return ORACLE_EINVAL;
    if (mode == ORACLE_MODE_INT8 && !x_scale) return ORACLE_EINVAL;
    if (!rows) nrows = T;
    oracle_init();
#pragma omp parallel for schedule(dynamic, 1)
    for (i = 0; i < nrows; ++i) {
        int64_t t = rows ? rows[i] : i;
        double* a = (double*)malloc(sizeof(double) * (size_t)(d_e + d_h));
        double* y = a ? a + d_e : NULL;
        double* acc = out_acc + i * d_h;
        int64_t n;
        int j;
        if (!a || t < 0 || t >= T) {
#pragma omp atomic write
            failed = 1;
            free(a);
            continue;
        }
        for (n = 0; n < d_h; ++n) acc[n] = 0.0;
        for (j = 0; j < k; ++j) {
            int64_t p = t * k + j;
            int32_t e = topk_ids[p];
            double wt = topk_w[p];
            if (e < 0 || e >= E) continue; /* dropped assignment */
            expert_ffn(mode, flags, d_h, d_e, x, x_scale, t, w1, w1_scale, w2, w2_scale, e, a, y);
            for (n = 0; n < d_h; ++n) acc[n] = R(acc[n] + R(wt * y[n], f64), f64);
        }
        if (out) {
            for (n = 0; n < d_h; ++n) {
                if (mode == ORACLE_MODE_F32ACT)
                    ((float*)out)[i * d_h + n] = (float)acc[n];
                else
                    ((uint16_t*)out)[i * d_h + n] = oracle_bf16_encode((float)acc[n]);
            }
        }
        free(a);
    }
    return failed ? ORACLE_EINVAL : ORACLE_OK;
}

/*
 * Routing metadata of the grouped-by-expert layout (tilelang.dataflow README,
 * section 3.5, step 1: group sizes, offsets, padded offsets and the expert of
 * each group block).  Assignment p = t*k + j has expert ids[p]; ids outside
 * [0,E) are dropped.  Within an expert, assignments keep ascending p (a stable
 * counting sort, written as one ascending pass).  Each expert's group is padded
 * to a multiple of bm rows; an expert with no rows gets no block.
 *
 *   counts[E]            rows per expert
 *   offsets[E+1]         exclusive prefix sum of counts
 *   padded_offsets[E+1]  exclusive prefix sum of bm*ceil(counts/bm)
 *   pos[N]               offsets[e] + rank of p within e, -1 if dropped
 *   sorted_p[N]          sorted_p[pos[p]] = p for the first offsets[E] entries, -1 after
 *   ppos[N]              padded_offsets[e] + rank, -1 if dropped
 *   row_src[n_pad_cap]   p at ppos[p], -1 on padding rows and beyond padded_offsets[E]
 *   tile_expert[tile_cap], tile_row0[tile_cap]  expert and first padded row of
 *                        each bm-row block in ascending expert order, -1 after
 *   stats[2]             {dropped, number of blocks}
 */
int moe_oracle_route(const int32_t* ids, int64_t N, int E, int bm, int32_t* counts, int32_t* offsets,
                     int32_t* padded_offsets, int32_t* pos, int32_t* sorted_p, int32_t* ppos, int32_t* row_src,
                     int64_t n_pad_cap, int32_t* tile_expert, int32_t* tile_row0, int64_t tile_cap,
                     int64_t* stats) {
    int64_t p, i;
    int e;
    int64_t ntiles = 0, dropped = 0;
    int32_t* seen;
    if (!ids || N < 0 || E < 1 || bm < 1) return ORACLE_EINVAL;
    seen = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    if (!seen) return ORACLE_ENOMEM;
    for (e = 0; e < E; ++e) counts[e] = 0;
    for (p = 0; p < N; ++p) {
        if (ids[p] >= 0 && ids[p] < E)
            counts[ids[p]]++;
        else
            dropped++;
    }
    offsets[0] = 0;
    padded_offsets[0] = 0;
    for (e = 0; e < E; ++e) {
        int32_t tiles = (counts[e] + bm - 1) / bm;
        offsets[e + 1] = offsets[e] + counts[e];
        padded_offsets[e + 1] = padded_offsets[e] + tiles * bm;
        ntiles += tiles;
    }
    if (padded_offsets[E] > n_pad_cap || ntiles > tile_cap) {
        free(seen);
        return ORACLE_EINVAL;
    }
    for (p = 0; p < N; ++p) sorted_p[p] = -1;
    for (i = 0; i < n_pad_cap; ++i) row_src[i] = -1;
    for (p = 0; p < N; ++p) {
        int32_t id = ids[p];
        if (id < 0 || id >= E) {
            pos[p] = -1;
            ppos[p] = -1;
            continue;
        }
        pos[p] = offsets[id] + seen[id];
        ppos[p] = padded_offsets[id] + seen[id];
        seen[id]++;
        sorted_p[pos[p]] = (int32_t)p;
        row_src[ppos[p]] = (int32_t)p;
    }
    for (i = 0; i < tile_cap; ++i) {
        tile_expert[i] = -1;
        tile_row0[i] = -1;
    }
    i = 0;
    for (e = 0; e < E; ++e) {
        int32_t r0;
        for (r0 = padded_offsets[e]; r0 < padded_offsets[e + 1]; r0 += bm) {
            tile_expert[i] = e;
            tile_row0[i] = r0;
            ++i;
        }
    }
    stats[0] = dropped;
    stats[1] = ntiles;
    free(seen);
    return ORACLE_OK;
}

/*
 * Backward pass of the layer with recompute (the pages' MoE megakernel serves
 * forward, backward and recompute passes from the same components: PipeLink
 * section 5.3; the derivative itself is the chain rule of the forward above).
 * BF16 mode only (x, W1, W2 and dout bf16).  Nothing of the forward is kept:
 * g, u and the intermediate are recomputed from x and W1.
 *
 * For each valid assignment p = t*k + j (e = ids[p], w = topk_w[p]), in fp32:
 *   g_r, u_r, a_r = silu(g_r) u_r as in the forward, h_r = a_r rounded to bf16
 *     (with ORACLE_MIRROR_H, as the forward stores it; else h_r = a_r)
 *   q_r   = sum_n dout[t][n] W2[e][n][r]                (n ascending)
 *   dtopk_w[p] = sum_r q_r h_r                           (r ascending)
 *   dh_r  = w q_r
 *   dg_r  = dh_r u_r silu'(g_r),  du_r = dh_r silu(g_r),
 *     silu'(g) = s (1 + g (1 - s)), s = 1 / (1 + exp(-g))
 *   dx[t][c]       += sum_r dg_r W1[e][r][c] + du_r W1[e][d_e + r][c]
 *   dW1[e][r][c]   += dg_r x[t][c],  dW1[e][d_e + r][c] += du_r x[t][c]
 *   dW2[e][n][r]   += (w dout[t][n]) h_r
 * With ORACLE_MIRROR_H the rounding points of the method are mirrored: dg and
 * du are rounded to bf16 before they enter dx and dW1, and w dout[t][n] is
 * rounded to bf16 before it enters dW2 (the backward GEMMs take bf16
 * operands).  Accumulation orders: dx per token over its slots in ascending
 * j (and within one slot r ascending, gate before up); dW1 and dW2 over the
 * assignments of an expert in ascending p.  Dropped ids contribute nothing and
 * get dtopk_w = 0.  Outputs: dx [T, d_h], dw1 [E, 2 d_e, d_h], dw2
 * [E, d_h, d_e], dtopk_w [T, k], all fp32 (fp64 values with ORACLE_ACC64, then
 * stored as float).  Returns ORACLE_EINVAL for a mode other than BF16 or bad
 * shapes, ORACLE_ENOMEM if scratch cannot be allocated.
 */
int moe_oracle_backward(int mode, int64_t T, int E, int k, int64_t d_h, int64_t d_e, const void* x,
                        const int32_t* topk_ids, const float* topk_w, const void* w1, const void* w2,
                        const uint16_t* dout, int flags, float* dx, float* dw1, float* dw2, float* dtopk_w) {
    int f64 = (flags & ORACLE_ACC64) != 0;
    int mirror = (flags & ORACLE_MIRROR_H) != 0;
    int64_t t, p, r, c, n, i;
    int j;
    double *g, *u, *h, *dg, *du, *q, *dxr, *gw1, *gw2;
    if (mode != ORACLE_MODE_BF16 || !check_dims(mode, T, E, k, d_h, d_e)) return ORACLE_EINVAL;
    if (!x || !topk_ids || !topk_w || !w1 || !w2 || !dout || !dx || !dw1 || !dw2 || !dtopk_w) return ORACLE_EINVAL;
    oracle_init();
    g = (double*)malloc(sizeof(double) * (size_t)(6 * d_e + 2 * d_h));
    gw1 = (double*)calloc((size_t)(E * 2 * d_e * d_h), sizeof(double));
    gw2 = (double*)calloc((size_t)(E * d_h * d_e), sizeof(double));
    if (!g || !gw1 || !gw2) {
        free(g);
        free(gw1);
        free(gw2);
        return ORACLE_ENOMEM;
    }
    u = g + d_e;
    h = u + d_e;
    dg = h + d_e;
    du = dg + d_e;
    q = du + d_e;
    dxr = q + d_e; /* d_h: dx of the current token */
    for (t = 0; t < T; ++t) {
        for (c = 0; c < d_h; ++c) dxr[c] = 0.0;
        for (j = 0; j < k; ++j) {
            int32_t e;
            double wt, dsum = 0.0;
            p = t * k + j;
            e = topk_ids[p];
            wt = topk_w[p];
            if (e < 0 || e >= E) {
                dtopk_w[p] = 0.0f;
                continue;
            }
            /* recompute: gate and up accumulators, the activation and h */
            for (r = 0; r < d_e; ++r) {
                double gg = 0.0, uu = 0.0, sg;
                for (c = 0; c < d_h; ++c) {
                    double xv = ld_x(mode, f64, x, NULL, d_h, t, c);
                    gg = R(gg + R(ld_w(mode, f64, w1, NULL, 2 * d_e, d_h, e, r, c) * xv, f64), f64);
                    uu = R(uu + R(ld_w(mode, f64, w1, NULL, 2 * d_e, d_h, e, d_e + r, c) * xv, f64), f64);
                }
                g[r] = gg;
                u[r] = uu;
                sg = f64 ? gg / (1.0 + exp(-gg)) : R(gg / R(1.0 + (double)expf((float)-gg), 0), 0);
                h[r] = R(sg * uu, f64);
                if (mirror) h[r] = oracle_bf16_decode(oracle_bf16_encode((float)h[r]));
            }
            /* q = dout[t] . W2[e] (the unweighted gradient of h) */
            for (r = 0; r < d_e; ++r) {
                double s = 0.0;
                for (n = 0; n < d_h; ++n)
                    s = R(s + R(oracle_bf16_decode(dout[t * d_h + n]) * ld_w(mode, f64, w2, NULL, d_h, d_e, e, n, r), f64),
                          f64);
                q[r] = s;
            }
            for (r = 0; r < d_e; ++r) dsum = R(dsum + R(q[r] * h[r], f64), f64);
            dtopk_w[p] = (float)dsum;
            /* activation backward */
            for (r = 0; r < d_e; ++r) {
                double dh = R(wt * q[r], f64), sig, silu, dsilu;
                sig = f64 ? 1.0 / (1.0 + exp(-g[r])) : R(1.0 / R(1.0 + (double)expf((float)-g[r]), 0), 0);
                silu = R(g[r] * sig, f64);
                dsilu = R(sig * R(1.0 + R(g[r] * R(1.0 - sig, f64), f64), f64), f64);
                dg[r] = R(R(dh * u[r], f64) * dsilu, f64);
                du[r] = R(dh * silu, f64);
                if (mirror) {
                    dg[r] = oracle_bf16_decode(oracle_bf16_encode((float)dg[r]));
                    du[r] = oracle_bf16_decode(oracle_bf16_encode((float)du[r]));
                }
            }
            /* dx of this slot, added to the token's sum */
            for (c = 0; c < d_h; ++c) {
                double s = 0.0;
                for (r = 0; r < d_e; ++r) {
                    s = R(s + R(dg[r] * ld_w(mode, f64, w1, NULL, 2 * d_e, d_h, e, r, c), f64), f64);
                    s = R(s + R(du[r] * ld_w(mode, f64, w1, NULL, 2 * d_e, d_h, e, d_e + r, c), f64), f64);
                }
                dxr[c] = R(dxr[c] + s, f64);
            }
            /* weight gradients, accumulated in ascending p per expert */
            for (r = 0; r < d_e; ++r)
                for (c = 0; c < d_h; ++c) {
                    double xv = ld_x(mode, f64, x, NULL, d_h, t, c);
                    i = (e * 2 * d_e + r) * d_h + c;
                    gw1[i] = R(gw1[i] + R(dg[r] * xv, f64), f64);
                    i = (e * 2 * d_e + d_e + r) * d_h + c;
                    gw1[i] = R(gw1[i] + R(du[r] * xv, f64), f64);
                }
            for (n = 0; n < d_h; ++n) {
                double dy = R(wt * oracle_bf16_decode(dout[t * d_h + n]), f64);
                if (mirror) dy = oracle_bf16_decode(oracle_bf16_encode((float)dy));
                for (r = 0; r < d_e; ++r) {
                    i = (e * d_h + n) * d_e + r;
                    gw2[i] = R(gw2[i] + R(dy * h[r], f64), f64);
                }
            }
        }
        for (c = 0; c < d_h; ++c) dx[t * d_h + c] = (float)dxr[c];
    }
    for (i = 0; i < E * 2 * d_e * d_h; ++i) dw1[i] = (float)gw1[i];
    for (i = 0; i < E * d_h * d_e; ++i) dw2[i] = (float)gw2[i];
    free(g);
    free(gw1);
    free(gw2);
    return ORACLE_OK;
}
