/*
 * Drives every entry of the CPU oracle (oracle/oracle_gdn.c, test infrastructure) on small
 * inputs and edge cases, for a build with AddressSanitizer and UndefinedBehaviorSanitizer:
 * any out-of-bounds access, leak or undefined operation aborts the run.  Exit status 0
 * means every call returned what its contract says.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_gdn_forward(const float*, const float*, const float*, const float*, const float*, const float*,
                       double*, double*, int, int, int, int, int, int, unsigned, int);
int oracle_linear_attn_block_causal(const float*, const float*, const float*, const float*, const float*,
                                    double*, double*, double*, int, int, int, int, int, int, double, int);
int oracle_softmax_attn_block_causal(const float*, const float*, const float*, double*, int, int, int, int,
                                     int, int, int, double, int);
int oracle_temporal_conv_block(const float*, const float*, const float*, const float*, double*, double*, int,
                               int, int, int);
int oracle_rope3d(const float*, double*, int, int, int, int, int, int, int, int, int, double);

static float* rnd(size_t n, unsigned* s) {
    float* p = (float*)malloc(sizeof(float) * (n ? n : 1));
    for (size_t i = 0; i < n; ++i) {
        *s = *s * 1664525u + 1013904223u;
        p[i] = ((float)(*s >> 8) / 16777216.0f) * 2.0f - 1.0f;
    }
    return p;
}

static int fails = 0;
#define EXPECT(cond)                                                  \
    do {                                                              \
        if (!(cond)) {                                                \
            fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond); \
            ++fails;                                                  \
        }                                                             \
    } while (0)

int main(void) {
    unsigned s = 12345u;
    const int shapes[][6] = {/* B, H, F, N, dk, dv */ {1, 2, 3, 5, 4, 4}, {2, 1, 1, 1, 3, 5}, {1, 1, 0, 4, 2, 2},
                             {1, 3, 2, 7, 8, 6}};
    for (size_t c = 0; c < sizeof shapes / sizeof shapes[0]; ++c) {
        const int B = shapes[c][0], H = shapes[c][1], F = shapes[c][2], N = shapes[c][3], dk = shapes[c][4],
                  dv = shapes[c][5];
        const size_t T = (size_t)F * N, BH = (size_t)B * H;
        float *q = rnd(BH * T * dk, &s), *k = rnd(BH * T * dk, &s), *v = rnd(BH * T * dv, &s);
        float *al = rnd(BH * T, &s), *be = rnd(BH * T, &s), *st = rnd(BH * dv * dk, &s), *z = rnd(BH * dk, &s);
        for (size_t i = 0; i < BH * T; ++i) { al[i] = al[i] * al[i]; be[i] = 0.5f + 0.5f * be[i]; }
        if (BH * T) al[0] = 0.0f; /* the FLT_MIN clamp */
        double* out = (double*)calloc(BH * T * dv + 1, sizeof(double));
        double* so = (double*)calloc(BH * dv * dk + 1, sizeof(double));
        double* zo = (double*)calloc(BH * dk + 1, sizeof(double));
        for (unsigned flags = 0; flags < 8; ++flags) {
            EXPECT(oracle_gdn_forward(q, k, v, al, be, st, so, out, B, H, F, N, dk, dv, flags, 2) == 0);
            EXPECT(oracle_gdn_forward(q, k, v, al, be, NULL, NULL, out, B, H, F, N, dk, dv, flags, 1) == 0);
        }
        EXPECT(oracle_linear_attn_block_causal(q, k, v, NULL, NULL, so, zo, out, B, H, F, N, dk, dv, 1e-6, 2) == 0);
        if (dk == dv) {
            EXPECT(oracle_linear_attn_block_causal(q, k, v, st, z, NULL, NULL, out, B, H, F, N, dk, dv, 1e-6, 1) == 0);
        }
        EXPECT(oracle_softmax_attn_block_causal(q, k, v, out, B, H, F, F, N, dk, dv, 0.5, 2) == 0);
        if (F > 1) {  /* queries: the last frame only, keys: all F frames */
            EXPECT(oracle_softmax_attn_block_causal(q + (size_t)(F - 1) * N * dk, k, v, out, 1, 1, 1, F, N, dk, dv,
                                                    0.5, 1) == 0);
        }
        free(q); free(k); free(v); free(al); free(be); free(st); free(z); free(out); free(so); free(zo);
    }
    /* argument errors return -1 without touching memory */
    EXPECT(oracle_gdn_forward(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, -1, 1, 1, 1, 2, 2, 0, 1) == -1);
    EXPECT(oracle_softmax_attn_block_causal(NULL, NULL, NULL, NULL, 1, 1, 3, 2, 4, 2, 2, 1.0, 1) == -1);
    EXPECT(oracle_rope3d(NULL, NULL, 1, 1, 1, 1, 1, 6, 3, 2, 0, 10.0) == -1); /* odd part */

    { /* temporal convolution, with and without the carries and bias */
        const int B = 2, F = 3, P = 5, C = 4;
        float *x = rnd((size_t)B * F * P * C, &s), *ci = rnd((size_t)B * P * C, &s), *w = rnd(3 * C, &s),
              *bias = rnd(C, &s);
        double* y = (double*)calloc((size_t)B * F * P * C, sizeof(double));
        double* co = (double*)calloc((size_t)B * P * C, sizeof(double));
        EXPECT(oracle_temporal_conv_block(x, ci, w, bias, y, co, B, F, P, C) == 0);
        EXPECT(oracle_temporal_conv_block(x, NULL, w, NULL, y, NULL, B, F, P, C) == 0);
        EXPECT(oracle_temporal_conv_block(x, ci, w, bias, y, co, B, 0, P, C) == 0);
        free(x); free(ci); free(w); free(bias); free(y); free(co);
    }
    { /* 3D rotary embedding: parts of every size, including empty ones */
        const int B = 1, H = 2, F = 3, gh = 2, gw = 3, d = 12;
        const size_t n = (size_t)B * H * F * gh * gw * d;
        float* x = rnd(n, &s);
        double* y = (double*)calloc(n, sizeof(double));
        EXPECT(oracle_rope3d(x, y, B, H, F, gh, gw, d, 4, 4, 0, 10000.0) == 0);
        EXPECT(oracle_rope3d(x, y, B, H, F, gh, gw, d, 0, 12, 7, 100.0) == 0);
        EXPECT(oracle_rope3d(x, y, B, H, F, gh, gw, d, 12, 0, (1 << 24) - 4, 16.0) == 0);
        free(x); free(y);
    }
    if (fails) fprintf(stderr, "%d check(s) failed\n", fails);
    else printf("oracle sanitizer run: ok\n");
    return fails ? 1 : 0;
}
