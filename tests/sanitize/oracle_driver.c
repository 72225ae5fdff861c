/* Runs every function of the reference MoE layer (oracle/oracle.h) on small inputs, for a
   build with AddressSanitizer and UndefinedBehaviorSanitizer: any out-of-bounds access,
   leak or undefined operation aborts the program.  Exit status 0 = clean. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/oracle.h"

static uint64_t state = 0x9E3779B97F4A7C15ULL;
static double uni(void)
{
    state = state * 6364136223846793005ULL + 1442695040888963407ULL;
    return ((double)(state >> 11) + 0.5) * 0x1.0p-53;
}
static uint16_t bf16_of(double v)
{
    float f = (float)v;
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

static int run_format(int fmt, int64_t T, int32_t H, int32_t I, int32_t E, int32_t k, int shared)
{
    const int n = E + 1;
    uint16_t *x = malloc(sizeof(uint16_t) * (size_t)(T * H));
    float *Wr = malloc(sizeof(float) * (size_t)(E * H)), *bias = malloc(sizeof(float) * (size_t)E);
    for (int64_t i = 0; i < T * H; i++) x[i] = bf16_of(2.0 * uni() - 1.0);
    for (int64_t i = 0; i < (int64_t)E * H; i++) Wr[i] = (float)(0.1 * (2.0 * uni() - 1.0));
    for (int e = 0; e < E; e++) bias[e] = (float)(0.01 * e);
    /* three matrices per expert: gate, up [I][H], down [H][I] */
    void *data[3];
    uint8_t *sc[3];
    float ts[3] = {1.f, 1.f, 1.f};
    const int64_t rows[3] = {I, I, H}, cols[3] = {H, H, I};
    for (int m = 0; m < 3; m++) {
        const int64_t N = rows[m], K = cols[m];
        double *W = malloc(sizeof(double) * (size_t)(N * K));
        for (int64_t i = 0; i < N * K; i++) W[i] = 0.05 * (2.0 * uni() - 1.0);
        if (fmt == ORACLE_FMT_BF16) {
            uint16_t *b = malloc(sizeof(uint16_t) * (size_t)(n * N * K));
            for (int64_t i = 0; i < n * N * K; i++) b[i] = bf16_of(W[i % (N * K)]);
            data[m] = b;
            sc[m] = NULL;
        } else if (fmt == ORACLE_FMT_NVFP4) {
            uint8_t *q = malloc((size_t)(n * N * K / 2));
            uint8_t *sb = malloc((size_t)(n * N * K / 16));
            oracle_nvfp4_quantize(N, K, W, q, sb, &ts[m]);
            for (int e = 1; e < n; e++) {
                memcpy(q + e * N * K / 2, q, (size_t)(N * K / 2));
                memcpy(sb + e * N * K / 16, sb, (size_t)(N * K / 16));
            }
            data[m] = q;
            sc[m] = sb;
        } else {
            uint8_t *q = malloc((size_t)(n * N * K / 2));
            uint16_t *s = malloc(sizeof(uint16_t) * (size_t)(n * N * K / 128));
            oracle_int4_quantize(N, K, W, q, s);
            for (int e = 1; e < n; e++) {
                memcpy(q + e * N * K / 2, q, (size_t)(N * K / 2));
                memcpy(s + e * N * K / 128, s, sizeof(uint16_t) * (size_t)(N * K / 128));
            }
            data[m] = q;
            sc[m] = (uint8_t *)s;
        }
        free(W);
    }
    oracle_expert *ex = malloc(sizeof(oracle_expert) * (size_t)n);
    for (int e = 0; e < n; e++) {
        oracle_matrix *mm[3] = {&ex[e].gate, &ex[e].up, &ex[e].down};
        for (int m = 0; m < 3; m++) {
            const int64_t N = rows[m], K = cols[m];
            mm[m]->format = fmt;
            mm[m]->tensor_scale = ts[m];
            if (fmt == ORACLE_FMT_BF16) {
                mm[m]->data = (uint16_t *)data[m] + e * N * K;
                mm[m]->block_scale = NULL;
            } else {
                mm[m]->data = (uint8_t *)data[m] + e * N * K / 2;
                mm[m]->block_scale = fmt == ORACLE_FMT_NVFP4 ? sc[m] + e * N * K / 16
                                                             : (uint8_t *)((uint16_t *)sc[m] + e * N * K / 128);
            }
        }
    }
    double *logits = malloc(sizeof(double) * (size_t)(T * E)), *w = malloc(sizeof(double) * (size_t)(T * k));
    double *y = malloc(sizeof(double) * (size_t)(T * H));
    int32_t *ids = malloc(sizeof(int32_t) * (size_t)(T * k));
    int rc = oracle_moe_layer(T, H, I, E, k, 1, x, Wr, bias, ex, shared ? &ex[E] : NULL, logits, ids, w, y);
    int32_t *counts = malloc(sizeof(int32_t) * (size_t)E), *offsets = malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *sa = malloc(sizeof(int32_t) * (size_t)(T * k)), *ap = malloc(sizeof(int32_t) * (size_t)(T * k));
    rc |= oracle_permute(T, E, k, ids, counts, offsets, sa, ap);
    oracle_weights(T, E, k, 0, logits, ids, w);
    double acc = 0.0;
    for (int64_t i = 0; i < T * H; i++) acc += fabs(y[i]);
    for (int64_t i = 0; i < (int64_t)H * I; i++) acc += fabs(oracle_matrix_at(&ex[0].down, I, i / I, i % I));
    free(logits); free(w); free(y); free(ids); free(counts); free(offsets); free(sa); free(ap);
    free(ex);
    for (int m = 0; m < 3; m++) {
        free(data[m]);
        free(sc[m]);
    }
    free(x); free(Wr); free(bias);
    if (rc != 0 || !isfinite(acc)) {
        fprintf(stderr, "format %d: rc %d, sum %g\n", fmt, rc, acc);
        return 1;
    }
    return 0;
}

int main(void)
{
    double s = 0.0;
    for (uint32_t c = 0; c < 16; c++) s += oracle_e2m1_value(c) + oracle_int4_value(c);
    for (uint32_t c = 0; c < 256; c++)
        if ((c & 0x7f) != 0x7f) s += oracle_e4m3_value(c);
    for (int i = -2000; i <= 2000; i++) {
        s += oracle_e4m3_encode(i * 0.37) + oracle_e2m1_encode(i * 0.0071);
    }
    /* selection with heavy ties, every k */
    double lg[4 * 8];
    int32_t ids[4 * 8];
    for (int i = 0; i < 32; i++) lg[i] = (double)(i % 3) - 1.0;
    for (int k = 1; k <= 8; k++)
        if (oracle_select(4, 8, k, lg, ids) != 0) return 1;
    if (oracle_select(1, 8, 9, lg, ids) == 0) return 1; /* k > E is rejected */
    int bad = 0;
    bad |= run_format(ORACLE_FMT_BF16, 5, 64, 32, 9, 3, 1);
    bad |= run_format(ORACLE_FMT_BF16, 2, 32, 16, 1, 1, 0);
    bad |= run_format(ORACLE_FMT_NVFP4, 3, 64, 32, 6, 4, 1);
    bad |= run_format(ORACLE_FMT_INT4, 3, 128, 128, 4, 2, 1);
    printf("oracle driver: %s (%g)\n", bad ? "FAILED" : "ok", s);
    return bad;
}
