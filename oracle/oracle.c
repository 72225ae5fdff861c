/*
 * oracle.c -- reference implementation of the Flint-style sparse MoE FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): the GPU library never links this code.
 * Plain single-threaded C; every sum is in double with its loop index ascending and
 * no value is rounded on the way.  The steps follow the pages' description of the layer
 * in order: a router producing one logit per routed expert, top-6 selection with sigmoid
 * scores, the always-on shared expert, the experts' FFNs and the weighted combine.
 *
 * Pinned by tests/test_oracle_pins.py (brute force, closed forms, invariants and the
 * torch float8 codec).  Agreement with the real Flint layer is parity unpinned: no page
 * prints a value of the layer.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static double bf16_bits_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* E2M1 (the element type of NVFP4, recipes.vllm.ai "RecursiveSI/flint", Overview):
   1 sign bit (bit 3), 2 exponent bits with bias 1, 1 mantissa bit.  Exponent field 0
   is subnormal: value = m * 0.5.  Otherwise value = (1 + m/2) * 2^(e-1). */
double oracle_e2m1_value(uint32_t code)
{
    uint32_t e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * (double)m : (1.0 + 0.5 * (double)m) * ldexp(1.0, (int)e - 1);
    return (code & 8u) ? -mag : mag;
}

/* E4M3FN (the block-scale type of NVFP4): 1 sign, 4 exponent bits with bias 7,
   3 mantissa bits, no infinities, S.1111.111 is NaN.  Exponent field 0 is subnormal:
   m/8 * 2^-6. */
double oracle_e4m3_value(uint32_t code)
{
    uint32_t e = (code >> 3) & 15u, m = code & 7u;
    if (e == 15u && m == 7u) return NAN;
    double mag = (e == 0) ? ((double)m / 8.0) * ldexp(1.0, -6)
                          : (1.0 + (double)m / 8.0) * ldexp(1.0, (int)e - 7);
    return (code & 0x80u) ? -mag : mag;
}

/* A nibble read as a two's complement 4-bit integer: bit 3 has weight -8. */
double oracle_int4_value(uint32_t code)
{
    return (double)(int)(code & 7u) - ((code & 8u) ? 8.0 : 0.0);
}

double oracle_matrix_at(const oracle_matrix *m, int64_t K, int64_t n, int64_t k)
{
    if (m->format == ORACLE_FMT_BF16) {
        const uint16_t *w = (const uint16_t *)m->data;
        return bf16_bits_to_double(w[n * K + k]);
    }
    if (m->format == ORACLE_FMT_INT4) {
        const uint8_t *q = (const uint8_t *)m->data;
        uint8_t byte = q[n * (K / 2) + k / 2];
        uint32_t code = (k % 2 == 0) ? (byte & 15u) : (byte >> 4);
        const uint16_t *sc = (const uint16_t *)m->block_scale;
        return oracle_int4_value(code) * bf16_bits_to_double(sc[n * (K / 128) + k / 128]);
    }
    const uint8_t *q = (const uint8_t *)m->data;
    uint8_t byte = q[n * (K / 2) + k / 2];
    uint32_t code = (k % 2 == 0) ? (byte & 15u) : (byte >> 4);
    double scale = oracle_e4m3_value(m->block_scale[n * (K / 16) + k / 16]);
    return oracle_e2m1_value(code) * scale * (double)m->tensor_scale;
}

/* Router: one logit per routed expert, a linear map of the token's hidden state
   (the plainest reading of "sigmoid routing", recipes.vllm.ai "RecursiveSI/flint",
   Overview).  The optional bias is a per-expert logit offset. */
void oracle_router(int64_t T, int32_t H, int32_t E, const uint16_t *x, const float *Wr,
                   const float *bias, double *logits)
{
    for (int64_t t = 0; t < T; t++) {
        for (int32_t e = 0; e < E; e++) {
            double s = 0.0;
            for (int32_t h = 0; h < H; h++)
                s += bf16_bits_to_double(x[t * H + h]) * (double)Wr[(int64_t)e * H + h];
            if (bias) s += (double)bias[e];
            logits[t * E + e] = s;
        }
    }
}

/* Top-k selection (k = 6 of 256 on the pages: neoteo.com table row "Eksperci";
   recipes.vllm.ai Overview).  Reading: select on the logits, which orders experts as
   their sigmoid scores do; ties go to the lowest index; -0 equals +0.  Each of the k
   rounds takes the largest unchosen logit, scanning experts in ascending order and
   replacing the candidate only on a strictly larger value. */
int oracle_select(int64_t T, int32_t E, int32_t k, const double *logits, int32_t *ids)
{
    if (k < 1 || k > E) return -1;
    char *chosen = (char *)malloc((size_t)E);
    if (!chosen) return -1;
    for (int64_t t = 0; t < T; t++) {
        const double *l = logits + t * E;
        for (int32_t e = 0; e < E; e++) {
            if (isnan(l[e])) { free(chosen); return -1; }
        }
        memset(chosen, 0, (size_t)E);
        for (int32_t j = 0; j < k; j++) {
            int32_t best = -1;
            for (int32_t e = 0; e < E; e++) {
                if (chosen[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            chosen[best] = 1;
            ids[t * k + j] = best;
        }
    }
    free(chosen);
    return 0;
}

/* Sigmoid scores of the chosen experts (recipes.vllm.ai Overview, "sigmoid routing"),
   renormalised to sum to one over the k chosen experts (reading adopted here). */
void oracle_weights(int64_t T, int32_t E, int32_t k, int32_t renormalize,
                    const double *logits, const int32_t *ids, double *w)
{
    for (int64_t t = 0; t < T; t++) {
        double sum = 0.0;
        for (int32_t j = 0; j < k; j++) {
            double l = logits[t * E + ids[t * k + j]];
            double s = 1.0 / (1.0 + exp(-l));
            w[t * k + j] = s;
            sum += s;
        }
        if (renormalize) {
            for (int32_t j = 0; j < k; j++) w[t * k + j] /= sum;
        }
    }
}

/* Grouping of assignments by expert, the data movement a fused MoE kernel implies
   (recipes.vllm.ai Overview, "fused MoE").  Assignments are visited in ascending order
   and appended to their expert's group, which makes the grouping stable. */
int oracle_permute(int64_t T, int32_t E, int32_t k, const int32_t *ids, int32_t *counts,
                   int32_t *offsets, int32_t *sorted_assign, int32_t *assign_pos)
{
    int64_t n = T * k;
    for (int32_t e = 0; e < E; e++) counts[e] = 0;
    for (int64_t a = 0; a < n; a++) {
        if (ids[a] < 0 || ids[a] >= E) return -1;
        counts[ids[a]]++;
    }
    offsets[0] = 0;
    for (int32_t e = 0; e < E; e++) offsets[e + 1] = offsets[e] + counts[e];
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    if (!cursor) return -1;
    for (int32_t e = 0; e < E; e++) cursor[e] = offsets[e];
    for (int64_t a = 0; a < n; a++) {
        int32_t p = cursor[ids[a]]++;
        sorted_assign[p] = (int32_t)a;
        assign_pos[a] = p;
    }
    free(cursor);
    return 0;
}

/* One expert.  Reading: a SwiGLU FFN, out = D (silu(G x) * (U x)) with
   silu(g) = g / (1 + exp(-g)); the pages do not name the activation. */
void oracle_expert_ffn(int32_t H, int32_t I, const oracle_expert *ex, const double *x,
                       double *scratch, double *out)
{
    double *a = scratch;
    for (int32_t i = 0; i < I; i++) {
        double g = 0.0, u = 0.0;
        for (int32_t h = 0; h < H; h++) g += oracle_matrix_at(&ex->gate, H, i, h) * x[h];
        for (int32_t h = 0; h < H; h++) u += oracle_matrix_at(&ex->up, H, i, h) * x[h];
        a[i] = g / (1.0 + exp(-g)) * u;
    }
    for (int32_t n = 0; n < H; n++) {
        double s = 0.0;
        for (int32_t i = 0; i < I; i++) s += oracle_matrix_at(&ex->down, I, n, i) * a[i];
        out[n] = s;
    }
}

/* The combine: the shared expert is always active with weight one (news.ditty.ir,
   third paragraph; neoteo.com table row "Eksperci"; reading: ungated), then the routed
   experts in selection order, each scaled by its gate weight. */
void oracle_moe_tokens(int32_t H, int32_t I, int32_t E, int32_t k, const oracle_expert *experts,
                       const oracle_expert *shared, const uint16_t *x, const int32_t *ids,
                       const double *w, int64_t n_tokens, const int64_t *tokens, double *y)
{
    (void)E;
    double *xt = (double *)malloc(sizeof(double) * (size_t)H);
    double *o = (double *)malloc(sizeof(double) * (size_t)H);
    double *scratch = (double *)malloc(sizeof(double) * (size_t)(2 * I));
    for (int64_t i = 0; i < n_tokens; i++) {
        int64_t t = tokens[i];
        double *yt = y + i * H;
        for (int32_t h = 0; h < H; h++) xt[h] = bf16_bits_to_double(x[t * H + h]);
        for (int32_t h = 0; h < H; h++) yt[h] = 0.0;
        if (shared) {
            oracle_expert_ffn(H, I, shared, xt, scratch, o);
            for (int32_t h = 0; h < H; h++) yt[h] += o[h];
        }
        for (int32_t j = 0; j < k; j++) {
            int32_t e = ids[t * k + j];
            oracle_expert_ffn(H, I, &experts[e], xt, scratch, o);
            double wj = w[t * k + j];
            for (int32_t h = 0; h < H; h++) yt[h] += wj * o[h];
        }
    }
    free(xt);
    free(o);
    free(scratch);
}

int oracle_moe_layer(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k, int32_t renormalize,
                     const uint16_t *x, const float *Wr, const float *bias,
                     const oracle_expert *experts, const oracle_expert *shared,
                     double *logits, int32_t *ids, double *w, double *y)
{
    oracle_router(T, H, E, x, Wr, bias, logits);
    int rc = oracle_select(T, E, k, logits, ids);
    if (rc != 0) return rc;
    oracle_weights(T, E, k, renormalize, logits, ids, w);
    int64_t *tokens = (int64_t *)malloc(sizeof(int64_t) * (size_t)(T > 0 ? T : 1));
    for (int64_t t = 0; t < T; t++) tokens[t] = t;
    oracle_moe_tokens(H, I, E, k, experts, shared, x, ids, w, T, tokens, y);
    free(tokens);
    return 0;
}

/* Nearest grid point among the non-negative codes 0..n_codes-1 of a monotone code
   table, ties to the even code; values above the largest finite one saturate. */
static uint32_t nearest_code(double mag, double (*value)(uint32_t), uint32_t n_codes)
{
    uint32_t best = 0;
    double best_d = fabs(mag - value(0));
    for (uint32_t c = 1; c < n_codes; c++) {
        double d = fabs(mag - value(c));
        if (d < best_d || (d == best_d && (c & 1u) == 0u && (best & 1u) != 0u)) {
            best = c;
            best_d = d;
        }
    }
    return best;
}

uint32_t oracle_e4m3_encode(double v)
{
    double mag = fabs(v);
    uint32_t c = (mag >= 448.0) ? 0x7Eu : nearest_code(mag, oracle_e4m3_value, 0x7Fu);
    return signbit(v) ? (c | 0x80u) : c;
}

uint32_t oracle_e2m1_encode(double v)
{
    double mag = fabs(v);
    uint32_t c = (mag >= 6.0) ? 7u : nearest_code(mag, oracle_e2m1_value, 8u);
    return signbit(v) ? (c | 8u) : c;
}

void oracle_nvfp4_quantize(int64_t N, int64_t K, const double *W, uint8_t *q, uint8_t *sb,
                           float *st)
{
    double amax = 0.0;
    for (int64_t i = 0; i < N * K; i++)
        if (fabs(W[i]) > amax) amax = fabs(W[i]);
    float ts = (amax == 0.0) ? 1.0f : (float)(amax / (6.0 * 448.0));
    *st = ts;
    for (int64_t n = 0; n < N; n++) {
        for (int64_t b = 0; b < K / 16; b++) {
            const double *blk = W + n * K + b * 16;
            double bmax = 0.0;
            for (int i = 0; i < 16; i++)
                if (fabs(blk[i]) > bmax) bmax = fabs(blk[i]);
            uint32_t sc = oracle_e4m3_encode(bmax / (6.0 * (double)ts));
            sb[n * (K / 16) + b] = (uint8_t)sc;
            double bs = oracle_e4m3_value(sc) * (double)ts;
            for (int i = 0; i < 16; i += 2) {
                uint32_t c0 = (bs == 0.0) ? 0u : oracle_e2m1_encode(blk[i] / bs);
                uint32_t c1 = (bs == 0.0) ? 0u : oracle_e2m1_encode(blk[i + 1] / bs);
                q[n * (K / 2) + (b * 16 + i) / 2] = (uint8_t)(c0 | (c1 << 4));
            }
        }
    }
}

/* double -> bf16 bits, round to nearest even (finite values in the normal bf16 range, or
   zero): 8 significant bits. */
static uint16_t double_to_bf16_rne(double v)
{
    if (v == 0.0) return signbit(v) ? 0x8000u : 0u;
    int e2;
    double f = frexp(fabs(v), &e2);      /* |v| = f * 2^e2, f in [0.5, 1) */
    double m = nearbyint(f * 256.0);     /* 8 significant bits, ties to even */
    if (m == 256.0) {
        m = 128.0;
        e2 += 1;
    }
    uint32_t bits = ((uint32_t)(e2 - 1 + 127) << 7) | ((uint32_t)m - 128u);
    return (uint16_t)(signbit(v) ? (bits | 0x8000u) : bits);
}

void oracle_int4_quantize(int64_t N, int64_t K, const double *W, uint8_t *q, uint16_t *s)
{
    for (int64_t n = 0; n < N; n++) {
        for (int64_t g = 0; g < K / 128; g++) {
            const double *grp = W + n * K + g * 128;
            double amax = 0.0;
            for (int i = 0; i < 128; i++)
                if (fabs(grp[i]) > amax) amax = fabs(grp[i]);
            uint16_t sb = double_to_bf16_rne(amax / 7.0);
            s[n * (K / 128) + g] = sb;
            double sv = bf16_bits_to_double(sb);
            for (int i = 0; i < 128; i += 2) {
                int32_t c[2];
                for (int j = 0; j < 2; j++) {
                    double r = (sv == 0.0) ? 0.0 : nearbyint(grp[i + j] / sv);
                    if (r > 7.0) r = 7.0;
                    if (r < -8.0) r = -8.0;
                    c[j] = (int32_t)r & 15;
                }
                q[n * (K / 2) + (g * 128 + i) / 2] = (uint8_t)(c[0] | (c[1] << 4));
            }
        }
    }
}
