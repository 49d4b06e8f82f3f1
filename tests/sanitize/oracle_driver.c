/* Sanitizer run of the CPU oracle (built with -fsanitize=address,undefined by
 * tests/test_sanitizers.py): routing and the forward pass in every mode on
 * small random inputs, with invalid and duplicate ids, a row subset, E = 1 and
 * k = 8, plus every codec entry point over its whole input range.  Any
 * out-of-bounds access, use of freed memory or undefined behaviour aborts the
 * run; wrong return codes exit with status 1.  Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double oracle_e4m3_decode(uint8_t);
uint8_t oracle_e4m3_encode(double);
uint16_t oracle_bf16_encode(float);
float oracle_bf16_decode(uint16_t);
double oracle_e8m0_decode(uint8_t);
void oracle_requant_chunk(double*, int64_t, int);
void oracle_mx_requant_block(double*, int64_t, uint8_t*);
int moe_oracle_forward(int, int64_t, int, int, int64_t, int64_t, const void*, const void*, const int32_t*,
                       const float*, const void*, const void*, const void*, const void*, int, const int64_t*,
                       int64_t, double*, void*);
int moe_oracle_route(const int32_t*, int64_t, int, int, int32_t*, int32_t*, int32_t*, int32_t*, int32_t*, int32_t*,
                     int32_t*, int64_t, int32_t*, int32_t*, int64_t, int64_t*);
int moe_oracle_backward(int, int64_t, int, int, int64_t, int64_t, const void*, const int32_t*, const float*,
                        const void*, const void*, const uint16_t*, int, float*, float*, float*, float*);

static uint64_t rs = 88172645463325252ull;
static uint32_t rnd(void) {
    rs ^= rs << 13;
    rs ^= rs >> 7;
    rs ^= rs << 17;
    return (uint32_t)rs;
}
static float frnd(void) { return (float)((rnd() & 0xffffff) / 16777216.0 * 2.0 - 1.0); }

static int backward_case(int64_t T, int E, int k, int64_t d_h, int64_t d_e, int flags) {
    uint16_t* x = malloc(2 * T * d_h + 2);
    uint16_t* w1 = malloc(2 * E * 2 * d_e * d_h);
    uint16_t* w2 = malloc(2 * E * d_h * d_e);
    uint16_t* dout = malloc(2 * T * d_h + 2);
    int32_t* ids = malloc(4 * T * k + 4);
    float* tw = malloc(4 * T * k + 4);
    float *dx = malloc(4 * T * d_h + 4), *dw1 = malloc(4 * E * 2 * d_e * d_h), *dw2 = malloc(4 * E * d_h * d_e);
    float* dtw = malloc(4 * T * k + 4);
    int64_t i;
    int rc;
    for (i = 0; i < T * d_h; ++i) { x[i] = oracle_bf16_encode(frnd()); dout[i] = oracle_bf16_encode(frnd()); }
    for (i = 0; i < E * 2 * d_e * d_h; ++i) w1[i] = oracle_bf16_encode(frnd() * 0.1f);
    for (i = 0; i < E * d_h * d_e; ++i) w2[i] = oracle_bf16_encode(frnd() * 0.1f);
    for (i = 0; i < T * k; ++i) { ids[i] = (rnd() % 5 == 0) ? -1 : (int32_t)(rnd() % E); tw[i] = frnd(); }
    rc = moe_oracle_backward(1, T, E, k, d_h, d_e, x, ids, tw, w1, w2, dout, flags, dx, dw1, dw2, dtw);
    free(x); free(w1); free(w2); free(dout); free(ids); free(tw); free(dx); free(dw1); free(dw2); free(dtw);
    return rc;
}

static int route_case(int64_t N, int E, int bm) {
    int32_t* ids = malloc(sizeof(int32_t) * (N ? N : 1));
    int64_t n_pad_cap = N + (E < N ? E : N) * (bm - 1), tile_cap = n_pad_cap / bm + 1, stats[2], i;
    int32_t *counts = malloc(4 * E), *off = malloc(4 * (E + 1)), *poff = malloc(4 * (E + 1));
    int32_t *pos = malloc(4 * (N + 1)), *sp = malloc(4 * (N + 1)), *ppos = malloc(4 * (N + 1));
    int32_t *rows = malloc(4 * (n_pad_cap + 1)), *te = malloc(4 * tile_cap), *tr = malloc(4 * tile_cap);
    int rc;
    for (i = 0; i < N; ++i) ids[i] = (rnd() % 9 == 0) ? -1 - (int32_t)(rnd() % 3) : (int32_t)(rnd() % (E + 2));
    rc = moe_oracle_route(ids, N, E, bm, counts, off, poff, pos, sp, ppos, rows, n_pad_cap, te, tr, tile_cap, stats);
    free(ids); free(counts); free(off); free(poff); free(pos); free(sp); free(ppos); free(rows); free(te); free(tr);
    return rc;
}

static int forward_case(int mode, int64_t T, int E, int k, int64_t d_h, int64_t d_e, int subset, int flags) {
    size_t xb = mode == 0 ? 4 : mode == 1 ? 2 : 1, wb = (mode == 2 || mode == 3) ? 1 : 2;
    unsigned char* x = malloc(xb * T * d_h + 1);
    unsigned char* w1 = malloc(wb * E * 2 * d_e * d_h);
    unsigned char* w2 = malloc(wb * E * d_h * d_e);
    int32_t* ids = malloc(sizeof(int32_t) * T * k + 4);
    float* tw = malloc(sizeof(float) * T * k + 4);
    void *xs = NULL, *w1s = NULL, *w2s = NULL;
    int64_t i, rows[3] = {T - 1, 0, T / 2}, nrows = subset ? 3 : T;
    double* acc = malloc(sizeof(double) * (nrows ? nrows : 1) * d_h);
    void* out = malloc(4 * (nrows ? nrows : 1) * d_h);
    int rc;
    for (i = 0; i < T * d_h; ++i) {
        if (mode == 0) ((float*)x)[i] = frnd();
        else if (mode == 1) ((uint16_t*)x)[i] = oracle_bf16_encode(frnd());
        else if (mode == 4) ((int8_t*)x)[i] = (int8_t)((int)(rnd() % 255) - 127);
        else { uint8_t c; do { c = (uint8_t)rnd(); } while ((c & 0x7f) == 0x7f); x[i] = c; }
    }
    for (i = 0; i < (int64_t)(E * 3 * d_e * d_h); ++i) {
        unsigned char* w = i < E * 2 * d_e * d_h ? w1 : w2;
        int64_t j = i < E * 2 * d_e * d_h ? i : i - E * 2 * d_e * d_h;
        if (wb == 2) ((uint16_t*)w)[j] = oracle_bf16_encode(frnd() * 0.1f);
        else { uint8_t c; do { c = (uint8_t)rnd(); } while ((c & 0x7f) == 0x7f); w[j] = c; }
    }
    for (i = 0; i < T * k; ++i) {
        ids[i] = (rnd() % 7 == 0) ? E + 3 : (int32_t)(rnd() % E);
        tw[i] = frnd();
    }
    if (mode == 2) {
        xs = malloc(4 * T * (d_h / 128) + 4);
        w1s = malloc(4 * E * (2 * d_e / 128) * (d_h / 128));
        w2s = malloc(4 * E * (d_h / 128) * (d_e / 128));
        for (i = 0; i < T * (d_h / 128); ++i) ((float*)xs)[i] = 0.01f + fabsf(frnd());
        for (i = 0; i < E * (2 * d_e / 128) * (d_h / 128); ++i) ((float*)w1s)[i] = 0.001f + fabsf(frnd()) * 0.01f;
        for (i = 0; i < E * (d_h / 128) * (d_e / 128); ++i) ((float*)w2s)[i] = 0.001f + fabsf(frnd()) * 0.01f;
    } else if (mode == 3) {
        xs = malloc(T * (d_h / 32) + 1);
        w1s = malloc(E * 2 * d_e * (d_h / 32));
        w2s = malloc(E * d_h * (d_e / 32));
        for (i = 0; i < T * (d_h / 32); ++i) ((uint8_t*)xs)[i] = (uint8_t)(118 + rnd() % 8);
        for (i = 0; i < E * 2 * d_e * (d_h / 32); ++i) ((uint8_t*)w1s)[i] = (uint8_t)(112 + rnd() % 8);
        for (i = 0; i < E * d_h * (d_e / 32); ++i) ((uint8_t*)w2s)[i] = (uint8_t)(112 + rnd() % 8);
    } else if (mode == 4) {
        xs = malloc(4 * T + 4);
        for (i = 0; i < T; ++i) ((float*)xs)[i] = 0.001f + fabsf(frnd()) * 0.02f;
    }
    rc = moe_oracle_forward(mode, T, E, k, d_h, d_e, x, xs, ids, tw, w1, w1s, w2, w2s, flags, subset ? rows : NULL,
                            nrows, acc, out);
    free(x); free(w1); free(w2); free(ids); free(tw); free(xs); free(w1s); free(w2s); free(acc); free(out);
    return rc;
}

int main(void) {
    int bad = 0, c, mode, f;
    double v[128];
    uint8_t sc;
    for (c = 0; c < 256; ++c) {
        double d = oracle_e4m3_decode((uint8_t)c);
        if ((c & 0x7f) != 0x7f && oracle_e4m3_encode(d) != (uint8_t)c && d != 0.0) bad |= 1;
        (void)oracle_e8m0_decode((uint8_t)c);
    }
    for (c = 0; c < 65536; c += 7) (void)oracle_bf16_encode(oracle_bf16_decode((uint16_t)c));
    for (c = 0; c < 128; ++c) v[c] = frnd() * 100.0;
    oracle_requant_chunk(v, 128, 0);
    oracle_requant_chunk(v, 128, 1);
    oracle_mx_requant_block(v, 32, &sc);
    memset(v, 0, sizeof(v));
    oracle_requant_chunk(v, 128, 0);
    oracle_mx_requant_block(v, 32, &sc);
    bad |= route_case(0, 4, 16) != 0;
    bad |= route_case(1, 1, 16) != 0;
    bad |= route_case(1000, 7, 16) != 0;
    bad |= route_case(4097, 256, 16) != 0;
    bad |= route_case(333, 40, 5) != 0;
    for (mode = 0; mode <= 4; ++mode)
        for (f = 0; f < 8; ++f) {
            if (f & 2) continue;
            bad |= forward_case(mode, 9, 3, 2, 256, 128, 0, f) != 0;
            bad |= forward_case(mode, 7, 1, 1, 128, 128, 1, f) != 0;
            bad |= forward_case(mode, 5, 4, 8, 128, 256, 0, f | 2) != 0;
        }
    bad |= forward_case(1, 0, 3, 2, 128, 128, 0, 1) != 0;
    bad |= backward_case(7, 3, 2, 128, 128, 1) != 0;
    bad |= backward_case(4, 1, 3, 128, 256, 2) != 0;
    bad |= backward_case(0, 2, 2, 128, 128, 1) != 0;
    /* invalid shapes must be refused */
    bad |= forward_case(2, 4, 2, 1, 100, 128, 0, 1) == 0;
    bad |= forward_case(5, 4, 2, 1, 128, 128, 0, 1) == 0;
    printf(bad ? "oracle sanitizer run: FAILED\n" : "oracle sanitizer run: ok\n");
    return bad ? 1 : 0;
}
