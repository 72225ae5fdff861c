/*
 * oracle.h -- reference implementation of the Flint-style sparse MoE FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
 * CPU-baseline leg of the benchmark may load, call or link this code.  The GPU
 * library never includes this header, never links this library and shares no
 * source with it; the two meet only in the seeded input generators.
 *
 * What the layer computes (sources are the pages about the Flint model):
 *   - recipes.vllm.ai page "RecursiveSI/flint", section Overview: 256 experts, top-6
 *     sigmoid routing plus a shared expert; an NVFP4 checkpoint that is run as W4A16.
 *   - neoteo.com article, specification table, row "Eksperci": 256 routed experts per
 *     MoE layer, 6 chosen per token plus one shared expert that is always active.
 *   - news.ditty.ir article, third paragraph: 6 of 256 experts per token plus one
 *     shared expert that is always on.
 * Readings where the pages are silent (SwiGLU experts, renormalised top-k weights,
 * lowest-index tie-break, ungated shared expert of weight 1, NVFP4 bit layout) are
 * stated at each function below.
 *
 * Every sum is taken in double with its loop index ascending; nothing is rounded
 * until the caller reads the double results.  Fidelity of these readings to the real
 * Flint checkpoint is parity unpinned: the pages print no value of the layer.
 */
#ifndef FLINT_ORACLE_H
#define FLINT_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_FMT_BF16 = 0, ORACLE_FMT_NVFP4 = 1, ORACLE_FMT_INT4 = 2 };

/* One weight matrix of N rows by K columns, K contiguous.
   bf16:  data = uint16 bf16 bits [N][K].
   nvfp4: data = uint8 [N][K/2], two E2M1 codes per byte, low nibble = even column;
          block_scale = E4M3 codes [N][K/16]; tensor_scale = one float.
   int4:  data = uint8 [N][K/2], two signed 4-bit integers (two's complement, -8..7) per
          byte, low nibble = even column; block_scale points at bf16 bits (uint16)
          [N][K/128], one scale per 128 consecutive columns; tensor_scale unused.
          The pages name an INT4 checkpoint without its layout (mrchatgpt.org
          explainer, section 4; neoteo.com article); this symmetric, group-of-128,
          bf16-scale form is the plainest common W4A16 reading. */
typedef struct {
    int32_t format;
    const void *data;
    const uint8_t *block_scale;
    float tensor_scale;
} oracle_matrix;

/* Expert e (0..E-1 routed, E = shared) is described by three matrices:
   gate [I][H], up [I][H], down [H][I]. */
typedef struct {
    oracle_matrix gate, up, down;
} oracle_expert;

/* E2M1 code (4 bits, bit 3 = sign) -> value. */
double oracle_e2m1_value(uint32_t code);
/* E4M3FN code (8 bits) -> value; 0x7F / 0xFF (NaN) return NaN. */
double oracle_e4m3_value(uint32_t code);
/* Signed 4-bit integer (two's complement nibble) -> value in -8..7. */
double oracle_int4_value(uint32_t code);
/* INT4 group quantiser (test data only): per row and group of 128 columns,
   s = bf16(amax / 7) rounded to nearest even (0 if amax = 0), q = W / s rounded to
   nearest even and clamped to -8..7 (0 where s = 0).  q uint8 [N][K/2], s bf16 bits
   [N][K/128]; K % 128 == 0. */
void oracle_int4_quantize(int64_t N, int64_t K, const double *W, uint8_t *q, uint16_t *s);
/* Element (n, k) of a matrix, widened exactly to double. */
double oracle_matrix_at(const oracle_matrix *m, int64_t K, int64_t n, int64_t k);

/* Router: logits[t][e] = sum_h x[t][h] * Wr[e][h] (+ bias[e]).  x bf16 bits [T][H],
   Wr float [E][H], bias float [E] or NULL, logits double [T][E]. */
void oracle_router(int64_t T, int32_t H, int32_t E, const uint16_t *x, const float *Wr,
                   const float *bias, double *logits);

/* Selection on logits: ids[t][0..k-1] = the k experts ordered by (logit descending,
   index ascending).  Returns 0, or -1 if a logit is NaN or k is out of range. */
int oracle_select(int64_t T, int32_t E, int32_t k, const double *logits, int32_t *ids);

/* Gate weights: w[t][j] = sigmoid(logits[t][ids[t][j]]), divided by their sum over j
   when renormalize != 0. */
void oracle_weights(int64_t T, int32_t E, int32_t k, int32_t renormalize,
                    const double *logits, const int32_t *ids, double *w);

/* Grouping of the T*k assignments a = t*k + j by expert: counts[E], exclusive
   offsets[E+1], sorted_assign[T*k] (grouped by expert, a ascending inside a group),
   assign_pos[a] = position of a in sorted_assign.  Returns 0, or -1 on a bad id. */
int oracle_permute(int64_t T, int32_t E, int32_t k, const int32_t *ids, int32_t *counts,
                   int32_t *offsets, int32_t *sorted_assign, int32_t *assign_pos);

/* One SwiGLU expert applied to one token: out = D (silu(G x) * (U x)).
   x double [H], out double [H], scratch double [2*I]. */
void oracle_expert_ffn(int32_t H, int32_t I, const oracle_expert *ex, const double *x,
                       double *scratch, double *out);

/* The MoE combine for a list of tokens, given routing:
   y[i] = o_shared + sum_j w[t][j] * o_{ids[t][j]}   (t = tokens[i]; shared term only if
   shared != NULL), in that order.  x bf16 bits [T][H]; ids [T][k]; w double [T][k];
   experts[0..E-1] routed; y double [n_tokens][H]. */
void oracle_moe_tokens(int32_t H, int32_t I, int32_t E, int32_t k, const oracle_expert *experts,
                       const oracle_expert *shared, const uint16_t *x, const int32_t *ids,
                       const double *w, int64_t n_tokens, const int64_t *tokens, double *y);

/* Whole layer for all T tokens: router, selection, weights, experts, combine.
   Writes logits [T][E], ids [T][k], w [T][k], y [T][H].  Returns oracle_select's code. */
int oracle_moe_layer(int64_t T, int32_t H, int32_t I, int32_t E, int32_t k, int32_t renormalize,
                     const uint16_t *x, const float *Wr, const float *bias,
                     const oracle_expert *experts, const oracle_expert *shared,
                     double *logits, int32_t *ids, double *w, double *y);

/* NVFP4 quantiser (produces test weights; not part of the layer).  For W [N][K] given
   as doubles: tensor scale st = amax / (6 * 448) (1 if amax == 0), block scale
   sb = RNE_e4m3(amax_block / (6 * st)), code q = RNE_e2m1(w / (sb * st)) with ties to
   the even code and saturation at 6.  Writes q [N][K/2], sb [N][K/16], *st. */
void oracle_nvfp4_quantize(int64_t N, int64_t K, const double *W, uint8_t *q, uint8_t *sb,
                           float *st);
/* Round-to-nearest-even onto the E4M3FN grid with saturation at 448: returns the code. */
uint32_t oracle_e4m3_encode(double v);
/* Round-to-nearest-even onto the E2M1 grid with saturation at 6: returns the code. */
uint32_t oracle_e2m1_encode(double v);

#ifdef __cplusplus
}
#endif
#endif
