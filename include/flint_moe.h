/*
 * flint_moe.h -- C ABI of the MI355X (gfx950) Flint-style sparse MoE FFN layer.
 *
 * The layer (pages about the Flint model: recipes.vllm.ai "RecursiveSI/flint",
 * section Overview; neoteo.com specification table, row "Eksperci"; news.ditty.ir,
 * third paragraph):  each token is routed by sigmoid scores to the top 6 of 256 routed
 * experts, and one shared expert is always active.  Readings where the pages are silent:
 * router logits are a linear map of the token (fp32 weights, fp32 accumulation), the
 * selection orders experts by logit (descending) with the lowest index winning ties,
 * the k sigmoid scores are renormalised to sum to one, every expert is a SwiGLU FFN
 * down(silu(gate x) * up x), and the shared expert is ungated with weight one.
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers unless stated; all work is queued asynchronously on
 *     `stream` (a hipStream_t; NULL = the null stream).  No call allocates memory or
 *     synchronises the host.  The caller owns every buffer.
 *   - Tensors are row-major and dense.  bf16 values are passed as their uint16 bits.
 *   - Inputs are never written.  Outputs are fully overwritten (no pre-zeroing needed)
 *     and must not alias inputs.
 *   - Every call returns a status (FLINT_OK == 0).  Arguments are validated before any
 *     HIP call, so invalid arguments are reported without touching the device.
 *     Nothing throws across the ABI.
 *   - T == 0 is a no-op returning FLINT_OK once the descriptor is valid.
 *   - Supported shapes: 1 <= E <= 256; 1 <= k <= min(8, E); n_shared in {0, 1};
 *     hidden % 64 == 0 and 64 <= hidden <= 8192; inter % 32 == 0 and
 *     32 <= inter <= 4096; 0 <= T <= 65536.  INT4 weights also need hidden % 128 == 0 and
 *     inter % 128 == 0 (a scale group is 128 columns).  Every pointer must be 16-byte
 *     aligned.  (The inter % 32 granularity admits one GPU's share of a layer split over
 *     inter, e.g. inter = 96 for 8 shares of 768.)
 *   - Dense layers: E == 0 with k == 0 and n_shared == 1 describes a dense SwiGLU FFN
 *     (the Flint model has 2 dense layers beside its 47 MoE layers: neoteo.com
 *     specification table, row "Warstwy"; their intermediate size is not given, so
 *     it is `inter`):
 *     y = bf16(down(silu(gate x) * up x)) with the sh_* weights, no router and no
 *     routing.  flint_moe_forward and flint_moe_layer accept it (routing arguments,
 *     w_router and logit_bias unused and may be NULL; the routed weight pointers and
 *     their scales must be NULL); flint_moe_route and flint_moe_permute return
 *     FLINT_ERR_SHAPE.
 *   - Calls on one stream are ordered; calls that share a workspace must not overlap.
 *   - A workspace's first 4 MiB (the head) hold the persistent launches' launch counters,
 *     the error flags and exchange words: zero them once before first use
 *     (flint_moe_workspace_init, or any zero fill) and leave them to the library
 *     afterwards.  Head words: u32 at byte 8 = error flags (read and cleared by
 *     flint_moe_workspace_status); u32 at byte 12 = reserved; u32 at byte 16 = a diagnostic
 *     switch, 0 in normal use: nonzero makes every bounded wait of the persistent launches
 *     give up at once (it exists so that the timeout report can be tested; results are then
 *     unreliable); u32 [256] at byte 1024 = launch counters, each the number of persistent
 *     launches (single-token and small-batch layer launches, small-batch router launches)
 *     made on the workspace so far.
 */
#ifndef FLINT_MOE_H
#define FLINT_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------------------ */
enum {
    FLINT_OK = 0,
    FLINT_ERR_NULL = 1,        /* a required pointer is NULL                            */
    FLINT_ERR_SHAPE = 2,       /* descriptor or T outside the supported range           */
    FLINT_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned                      */
    FLINT_ERR_WORKSPACE = 4,   /* ws_bytes < flint_moe_workspace_bytes(desc, T, format)  */
    FLINT_ERR_FORMAT = 5,      /* unknown weight format or missing scale arrays         */
    FLINT_ERR_HIP = 6          /* a kernel launch failed; see flint_moe_status_string    */
};

/* ---- workspace error flags (flint_moe_workspace_status) ---------------------------- */
enum {
    /* A bounded wait of a persistent launch (the single-token layer, the dense single-token
       layer, the small-batch layer and its router launch, every layer of a decode chain)
       ran out: its workgroups were not all resident
       at once (another kernel held CUs), so that call's outputs are unreliable.  The
       launch still ended normally, and later calls are unaffected: every launch's exchange
       words carry a tag of their own. */
    FLINT_WS_WAIT_TIMEOUT = 1
};

/* ---- weight formats ---------------------------------------------------------------- */
enum {
    FLINT_WFMT_BF16 = 0,
    /* NVFP4 run as W4A16 (recipes.vllm.ai "RecursiveSI/flint", Overview: the NVFP4
       checkpoint is run as W4A16).  Reading of the format: 16 consecutive elements along
       K share one E4M3FN scale; elements are E2M1 (bit 3 = sign, magnitudes
       0, .5, 1, 1.5, 2, 3, 4, 6), two per byte, the even column in the low nibble; one
       fp32 scale per (expert, matrix).  value = e2m1 * e4m3 * tensor_scale. */
    FLINT_WFMT_NVFP4 = 1,
    /* INT4 run as W4A16 (the pages name an INT4 checkpoint beside BF16 and NVFP4 without
       its layout: mrchatgpt.org explainer, section 4; neoteo.com article).  Reading of
       the format: signed 4-bit integers (two's complement, -8..7), two per byte, the even
       column in the low nibble; one bf16 scale per row and group of 128 consecutive
       columns along K; no zero point, no tensor scale.  value = q * scale.  The kernels
       dequantise to bf16 (q * scale rounded once) for the bf16 products, except the
       single-token path, which sums q * x per group in fp32 and scales the sum. */
    FLINT_WFMT_INT4 = 2
};

/* ---- route flags ------------------------------------------------------------------- */
enum {
    FLINT_ROUTE_LOGITS_IN = 1  /* `logits` is an input; the router product is skipped    */
};

/* Layer shape.  hidden = H, inter = I (per expert, the shared expert too),
   n_experts = E routed experts, top_k = k, n_shared = 0 or 1,
   renormalize = 1: w_j = s_j / sum_i s_i; 0: w_j = s_j (s = sigmoid of the logit). */
typedef struct {
    int32_t hidden;
    int32_t inter;
    int32_t n_experts;
    int32_t top_k;
    int32_t n_shared;
    int32_t renormalize;
} flint_moe_desc;

/* Expert weights.  Each matrix is stored with K (its input dimension) contiguous:
   gate and up are [I][H] per expert, down is [H][I] per expert.  Routed experts are
   stored expert-major; the shared expert has its own pointers (NULL iff n_shared == 0).
     BF16:  gate, up: uint16 [E][I][H];  down: uint16 [E][H][I].
     NVFP4: gate, up: uint8 [E][I][H/2]; down: uint8 [E][H][I/2]  (packed E2M1);
            *_sf: E4M3 block scales, gate/up [E][I][H/16], down [E][H][I/16];
            gate_ts, up_ts, down_ts: fp32 [E] tensor scales (device memory);
            sh_ts: fp32 [3] = gate, up, down tensor scales of the shared expert.
     INT4:  gate, up: uint8 [E][I][H/2]; down: uint8 [E][H][I/2]  (packed nibbles);
            *_sf: bf16 group scales (uint16 bits), gate/up [E][I][H/128], down
            [E][H][I/128]; every *_ts pointer NULL.
   Scale pointers must be NULL for BF16. */
typedef struct {
    int32_t format;
    const void *gate, *up, *down;
    const void *sh_gate, *sh_up, *sh_down;
    const uint8_t *gate_sf, *up_sf, *down_sf;
    const uint8_t *sh_gate_sf, *sh_up_sf, *sh_down_sf;
    const float *gate_ts, *up_ts, *down_ts;
    const float *sh_ts;
} flint_moe_weights;

/* Optional routing outputs of flint_moe_layer; any member may be NULL. */
typedef struct {
    float *logits;          /* [T][E] fp32                                     */
    int32_t *topk_ids;      /* [T][k]                                           */
    float *topk_w;          /* [T][k]                                           */
    int32_t *counts;        /* [E]                                              */
    int32_t *offsets;       /* [E+1]                                            */
    int32_t *sorted_assign; /* [T*k]                                            */
    int32_t *assign_pos;    /* [T*k]                                            */
} flint_moe_routing;

/* Workspace bytes that route/permute/forward/layer need for any T <= T_max with the
   given weight format.  Returns 0 for an invalid descriptor or T_max < 0. */
size_t flint_moe_workspace_bytes(const flint_moe_desc *desc, int64_t T_max, int32_t format);

/* Zero the first 4 MiB of a workspace (a small fill kernel on `stream`; no
   allocation).  Call once per workspace before its first use. */
int flint_moe_workspace_init(void *ws, size_t ws_bytes, void *stream);

/* The error flags (FLINT_WS_*) that calls on this workspace have raised since the last
   status call, written to *flags (a device int32, 4-byte aligned) by a one-thread kernel on
   `stream`, which also clears them; queue it after the calls to check, and read *flags once
   the stream has reached it.  0 = no error.  ws_bytes >= 4 MiB. */
int flint_moe_workspace_status(void *ws, size_t ws_bytes, int32_t *flags, void *stream);

/* Static text for a status code; for FLINT_ERR_HIP it also names the last HIP error
   seen by this library (the text is per thread and stays valid until the next call). */
const char *flint_moe_status_string(int status);

/* Router and selection: every token's router scores over the 256 routed experts and the
   top 6 of them, weighted by sigmoid scores (recipes.vllm.ai "RecursiveSI/flint", Overview:
   top-6 sigmoid routing; neoteo.com specification table, row "Eksperci": 6 of 256).
     logits[t][e] = sum_h x[t][h] * w_router[e][h] + (logit_bias ? logit_bias[e] : 0),
   accumulated in fp32 (x: bf16 [T][H]; w_router: fp32 [E][H]; logit_bias: fp32 [E]).
   topk_ids[t][0..k) = the k experts ordered by (logit descending, index ascending) on
   the fp32 logits, with -0 == +0 and NaN ordered below -inf;
   topk_w[t][j] = sigmoid(logit) in fp32, divided by the sum over j if desc->renormalize.
   flags & FLINT_ROUTE_LOGITS_IN: `logits` is read instead (x, w_router may be NULL).
   Otherwise `logits` may be NULL (kept in the workspace) or receives the logits. */
int flint_moe_route(const flint_moe_desc *desc, int64_t T, const uint16_t *x,
                    const float *w_router, const float *logit_bias, float *logits,
                    int32_t *topk_ids, float *topk_w, uint32_t flags, void *ws,
                    size_t ws_bytes, void *stream);

/* Grouping of the T*k assignments a = t*k + j by expert id, the data movement in front of
   a fused MoE expert kernel (recipes.vllm.ai "RecursiveSI/flint", Overview, the fused MoE
   kernel): counts[e] = #assignments of expert e; offsets = exclusive scan (offsets[E] = T*k);
   sorted_assign = assignments grouped by expert, ascending a inside a group;
   assign_pos[a] = position of a in sorted_assign.  Integer, bit-exact.
   Ids outside [0, E) are a caller error: such an assignment is dropped (in no count, its
   assign_pos is -1, and sorted_assign holds -1 from offsets[E] on); flint_moe_forward then
   leaves it out of the combine.
   ws may be NULL; given flint_moe_workspace_bytes(desc, T, ...) bytes, large T
   (T*k > 4096) uses a faster multi-block grouping with the same result. */
int flint_moe_permute(const flint_moe_desc *desc, int64_t T, const int32_t *topk_ids,
                      int32_t *counts, int32_t *offsets, int32_t *sorted_assign,
                      int32_t *assign_pos, void *ws, size_t ws_bytes, void *stream);

/* Experts and combine: the selected experts and the always-active shared expert, each a
   SwiGLU FFN, summed with the routing weights (news.ditty.ir, third paragraph, and
   neoteo.com specification table, row "Eksperci": 6 routed experts plus one shared expert
   that is always active; the SwiGLU form and the weight-one shared expert are readings):
     y[t] = bf16( o_shared(t) + sum_j topk_w[t][j] * o_{topk_ids[t][j]}(t) ),
     o_e(t) = down_e( silu(gate_e x_t) * (up_e x_t) ),
   summed in fp32 in that order (shared first, then j ascending), which makes y
   deterministic.  The expert intermediate h is rounded to bf16 before `down`; on the
   grouped-GEMM path (T > 32) each per-slot output o is also rounded to bf16 before the
   combine, while the streaming path (T <= 32) combines o in fp32.
   topk_ids/topk_w/offsets/sorted_assign/assign_pos are the outputs of route and
   permute for the same T (an assignment whose assign_pos is outside [0, T*k) is left out
   of the sum).  y: bf16 [T][H].
   A dense layer (n_experts == 0) with one token, 512 <= I <= 4096 and H <= 2048 (any
   weight format) runs as one persistent launch that exchanges h through the workspace
   head, like flint_moe_layer's single-token launch below (same device and head
   requirements). */
int flint_moe_forward(const flint_moe_desc *desc, const flint_moe_weights *weights, int64_t T,
                      const uint16_t *x, const int32_t *topk_ids, const float *topk_w,
                      const int32_t *offsets, const int32_t *sorted_assign,
                      const int32_t *assign_pos, uint16_t *y, void *ws, size_t ws_bytes,
                      void *stream);

/* The whole layer (the MoE FFN layer of the pages above: router, top-6 of 256 routed
   experts, shared expert, combine): route (x, w_router, logit_bias), permute and forward,
   with the same results as the three calls above.  `routing` (may be NULL) receives the intermediate
   routing tensors the caller asks for.  A single token (T == 1) runs as one persistent
   launch of one workgroup per CU (on a device with at least 256 CUs) whose workgroups
   exchange logits and h through tagged words at the start of the workspace (see
   flint_moe_workspace_init); it rounds h to bf16 like the other paths and combines the
   per-slot outputs in fp32; a dense layer's single bf16 token likewise (see
   flint_moe_forward).  2 <= T <= 16 tokens with bf16 weights run as one persistent launch
   of the whole layer in the same way; other batches of up to 32 tokens compute the logits,
   the top-k selection, the grouping and the expert plan in one persistent launch (logits
   exchanged as tagged words) before the expert kernels, with the results of the route and
   permute calls.  These launches need all 256 workgroups resident at once; they are
   chosen only on a device with at least 256 CUs where one workgroup fits on a CU.  A wait
   there that runs out (other work holding CUs) raises FLINT_WS_WAIT_TIMEOUT in the
   workspace (flint_moe_workspace_status). */
int flint_moe_layer(const flint_moe_desc *desc, const flint_moe_weights *weights, int64_t T,
                    const uint16_t *x, const float *w_router, const float *logit_bias,
                    uint16_t *y, const flint_moe_routing *routing, void *ws, size_t ws_bytes,
                    void *stream);

/* For callers that cannot allocate (code under HIP graph capture, tight serving loops,
   harnesses that forbid hipMalloc): flint_moe_layer without a workspace argument.  Its
   workspace is a 16 MiB array in device memory that the library holds on every GPU it runs
   on until the process ends (zero when the library is loaded there); the call allocates
   nothing.  Every call on one GPU shares that GPU's array, so calls that overlap on one GPU
   (other streams, other threads) race: order them, e.g. on one stream.  The array's head is
   the workspace head described above, never cleared by a call; its error flags are not
   reported (use flint_moe_layer with a workspace of your own to read them).
   Returns FLINT_ERR_WORKSPACE when flint_moe_workspace_bytes(desc, T, format) exceeds
   16 MiB (at H = 2048, I = 768, E = 256, k = 6 with a shared expert: T above 157);
   otherwise exactly as flint_moe_layer. */
int flint_moe_layer_noalloc(const flint_moe_desc *desc, const flint_moe_weights *weights, int64_t T,
                            const uint16_t *x, const float *w_router, const float *logit_bias,
                            uint16_t *y, const flint_moe_routing *routing, void *stream);

/* ---- persistent decode across layers ---------------------------------------------- */
/* One MoE layer of a chain: its expert weights, router weights [E][H] fp32 and optional
   logit bias [E] (device pointers, checked like flint_moe_layer's). */
typedef struct {
    flint_moe_weights weights;
    const float *w_router;
    const float *logit_bias;
} flint_moe_layer_ref;

enum {
    FLINT_CHAIN_RESIDUAL = 1  /* the next layer's token is bf16(x_l + y_l) instead of y_l */
};

/* A decode batch of T tokens (1 <= T <= 16) through n_layers MoE layers, one after the
   other, one persistent launch per layer:
     x_0 = x;  y_l = layer_l(x_l) exactly as flint_moe_layer computes it for T tokens;
     x_{l+1} = y_l, or bf16(x_l + y_l) (one fp32 sum, rounded once) with FLINT_CHAIN_RESIDUAL.
   The pages' GB200 runtime has a low-latency decode path for up to 8 requests and the
   Apple runtime a Metal megakernel (recipes.vllm.ai "RecursiveSI/flint", Overview;
   mrchatgpt.org explainer, section 4, the item on kernels).  Every layer is the persistent
   launch flint_moe_layer uses for T tokens (T = 1: the single-token launch; 2 <= T <= 16:
   the small-batch launch); its last phase also forms the next layer's tokens and leaves
   them in the workspace head for the next launch, so the chain costs no work between
   layers.  (Running several layers inside one launch, trading the tokens through tagged
   words, was measured slower on this GPU: the layer loop costs the kernel registers that
   its single-layer form keeps for loads in flight.)
   layers: host array [n_layers] (read during the call only).  All layers share `desc` and
   one weight format.  x: bf16 [T][H]; y: bf16 [n_layers][T][H], every layer's output y_l;
   topk_ids / topk_w: [n_layers][T][k] or NULL; logits: [n_layers][T][E] fp32 or NULL.
   Needs the persistent launch for T: E >= 1, k <= 8, a device with at least 256 CUs where
   one workgroup fits on a CU, and for T = 1 hidden % 256 == 0, hidden <= 2048,
   inter <= 1024 and the down rows of one 1/256 slice of hidden in whole 16-byte chunks; for
   T >= 2 hidden <= 2048, inter <= 1024 and E <= 256 (FLINT_ERR_SHAPE otherwise, also for T
   outside 1..16).  ws: at least flint_moe_workspace_bytes(desc, T, format) bytes,
   initialised once (flint_moe_workspace_init).  0 <= n_layers <= 4096. */
int flint_moe_decode_chain(const flint_moe_desc *desc, const flint_moe_layer_ref *layers,
                           int32_t n_layers, uint32_t flags, int64_t T, const uint16_t *x, uint16_t *y,
                           int32_t *topk_ids, float *topk_w, float *logits, void *ws,
                           size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif
