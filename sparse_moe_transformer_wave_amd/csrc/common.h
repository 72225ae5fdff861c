// common.h -- device helpers and the internal launch interface of libflint_moe.
//
// Everything here is gfx950 (CDNA4) code: 64-lane wavefronts, bf16 MFMA with fp32
// accumulation (v_mfma_f32_16x16x32_bf16), LDS tiling.  No other target is built.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace flint {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Layer shape as the kernels see it.
struct Shape {
    int H, I, E, k, S, renorm;
};

// Streaming (GEMV-like) path handles T up to this many tokens; larger T uses the
// grouped GEMM.  Two 16-token MFMA row tiles cover it.
constexpr int kGemvMaxT = 32;
constexpr int kUnitRows = 16;  // rows (tokens) per streaming work unit: one MFMA token tile

// Work units the plan may list: touched experts, plus the extra units of experts split
// into kUnitRows-row pieces on the streaming path (T <= kGemvMaxT).
__host__ __device__ inline int64_t plan_unit_capacity(int E, int k, int S, int64_t T)
{
    const int64_t ts = T < kGemvMaxT ? T : kGemvMaxT;
    return (int64_t)E + S + (ts * k + kUnitRows - 1) / kUnitRows + (int64_t)S * ((ts + kUnitRows - 1) / kUnitRows);
}
// Grouped GEMM tile: BM rows (tokens) x 256 B-rows x 64 K.
constexpr int kGemmBM = 256;

// One weight matrix kind (gate, up or down) of all experts.
// Routed expert e (< E) lives at routed + e * mat_bytes; the shared expert at `shared`.
// NVFP4 adds block scales (sf_*) and fp32 tensor scales (ts_routed[e], *ts_shared).
struct WMat {
    const uint8_t *routed, *shared;
    const uint8_t *sf_routed, *sf_shared;
    const float *ts_routed, *ts_shared;
};
struct WSet {
    int fmt;  // 0 bf16, 1 nvfp4, 2 int4 (sf_* = bf16 scale per 128 columns, no ts_*)
    WMat gate, up, down;
};

// Bytes of block / group scales per matrix row of K columns: NVFP4 one E4M3 byte per 16,
// INT4 one bf16 per 128.
__host__ __device__ constexpr size_t scale_row_bytes(int fmt, size_t K)
{
    return fmt == 1 ? K / 16 : fmt == 2 ? K / 64 : 0;
}

// Per-expert work description built on the device from the expert offsets.
//   meta[0] = number of units U' (touched routed experts in ascending id, then the shared
//             one; on the streaming path an expert of more than kUnitRows rows is split
//             into consecutive units of at most kUnitRows rows)
//   meta[1] = number of grouped-GEMM items
//   touched[u] (expert), tbase[u] (first slot), tcount[u] (rows) for u < U'
//   items[i] = (u << 16) | m_tile
struct Plan {
    int *meta;
    int *touched, *tbase, *tcount;
    int *items;
};

// Workspace carve-up (byte offsets from the workspace base), computed on the host.
struct WsLayout {
    size_t logits, ids, w, counts, offsets, sa, ap;
    size_t sync, plan, hist, h, o;
    size_t total;
    int max_items;
    int plan_units;  // capacity of the plan's touched / tbase / tcount arrays
};
WsLayout ws_layout(const Shape &s, int64_t T);
Plan plan_view(void *ws, const WsLayout &L, const Shape &s);

// ---- launches (return hipSuccess or the launch error) -----------------------------
hipError_t launch_router(const Shape &s, int64_t T, const uint16_t *x, const float *Wr,
                         const float *bias, float *logits, hipStream_t st);
hipError_t launch_topk(const Shape &s, int64_t T, const float *logits, int32_t *ids, float *w,
                       hipStream_t st);
// hist: ceil(T*k / 1024) * E ints of workspace for the multi-block grouping (T*k > 4096).
hipError_t launch_permute(const Shape &s, int64_t T, const int32_t *ids, int32_t *counts,
                          int32_t *offsets, int32_t *sa, int32_t *ap, const Plan *plan,
                          int32_t *hist, hipStream_t st);
hipError_t launch_plan(const Shape &s, int64_t T, const int32_t *offsets, const Plan &plan,
                       hipStream_t st);
// T <= kGemvMaxT: router, top-k, grouping and plan in one persistent launch (kPersistentGrid
// workgroups of 1024 threads exchanging logits through tagged words in the workspace head);
// supported when every workgroup fits at once, E <= 256, k <= 8 and S <= 1.
bool router_select_supported(const Shape &s, int64_t T);
hipError_t launch_router_select(const Shape &s, int64_t T, const uint16_t *x, const float *Wr,
                                const float *bias, float *logits, int32_t *ids, float *w,
                                int32_t *counts, int32_t *offsets, int32_t *sa, int32_t *ap,
                                const Plan &plan, uint8_t *head, hipStream_t st);
// Workspace head: the first kSyncBytes of every workspace (zeroed once before first use).
//   u32 at kHeadError     error flags (FLINT_WS_WAIT_TIMEOUT); cleared by the status call
//   u32 at kHeadReserved  unused (zero)
//   u32 at kHeadDiag      diagnostic switch: nonzero makes every bounded wait give up at once
//   u32 [kPersistentGrid] at kHeadCounters  launch counters, one per workgroup index: every
//                         persistent launch has exactly kPersistentGrid workgroups and
//                         workgroup b adds one to counter b, so all counters hold the number
//                         of persistent launches before the current one, which gives its tag
//   exchange words of the persistent launches from kHeadXchg on: the single-token layers'
//   up to kHeadFewXchg, the small-batch layer's and the small-batch router launch's from
//   there (4 MiB in all)
constexpr size_t kSyncBytes = 4096 * 1024, kHeadFewXchg = 96 * 1024;
constexpr size_t kHeadError = 8, kHeadReserved = 12, kHeadDiag = 16, kHeadCounters = 1024, kHeadXchg = 2048;
constexpr int kPersistentGrid = 256;
constexpr uint32_t kWsWaitTimeout = 1u;  // FLINT_WS_WAIT_TIMEOUT
static_assert(kHeadCounters + 4 * kPersistentGrid <= kHeadXchg, "launch counters overlap the exchange words");
// Tag of the persistent launch that follows `launches` earlier ones: 1 .. 2^32 - 1, never 0
// (the value of a zeroed exchange word); it repeats only after 2^32 - 1 launches.
__host__ __device__ inline uint32_t launch_tag(uint32_t launches)
{
    return launches % 0xffffffffu + 1u;
}
// Copies the head's error flags to *out and clears them (one thread).
hipError_t launch_ws_status(void *head, int32_t *out, hipStream_t st);
// Single-token layer in one persistent launch (decode1.hip).  `head` = the workspace head.
// decode1_supported also checks that the current device has a CU for every workgroup and
// that one workgroup of the launch fits on a CU (registers and LDS).
bool decode1_supported(const Shape &s, int fmt);
hipError_t launch_decode1(const Shape &s, const WSet &w, const uint16_t *x, const float *Wr,
                          const float *bias, uint16_t *y, float *logits, int32_t *ids, float *tw,
                          int32_t *counts, int32_t *offsets, int32_t *sa, int32_t *ap, void *head,
                          hipStream_t st);
// Dense SwiGLU layer (E = 0, the one expert held as the shared expert), one token in any
// weight format, in one persistent launch (decode1.hip); same head and CU check as
// launch_decode1.
// A small decode batch (2 <= T <= 16) in one persistent launch (decode_few.hip); the same
// residency checks as decode1_supported.
bool decode_few_supported(const Shape &s, int fmt, int64_t T);
hipError_t launch_decode_few(const Shape &s, const WSet &w, int64_t T, const uint16_t *x, const float *Wr,
                             const float *bias, uint16_t *y, float *logits, int32_t *ids, float *tw,
                             int32_t *counts, int32_t *offsets, int32_t *sa, int32_t *ap, void *head,
                             hipStream_t st);
// A small batch through L layers (decode_few.hip), layer l0 + l of the whole chain at
// position l: its tokens come from x (the chain's first layer) or the head's token buffer
// (l0 + l) % 2, its next layer's go to the other buffer; `hand_on` as in
// launch_decode_chain.  ids / tw may be null: the routing then goes to the scratch arrays
// (T k each).  y: [L][T][H]; ids, tw: [L][T][k]; logits: [L][T][E] or null.
hipError_t launch_decode_few_chain(const Shape &s, const WSet *w, const float *const *Wr,
                                   const float *const *bias, int L, int l0, bool residual, int64_t T,
                                   const uint16_t *x, bool hand_on, uint16_t *y, int32_t *ids, float *tw,
                                   float *logits, int32_t *ids_scratch, float *tw_scratch, void *head,
                                   hipStream_t st);
constexpr int kChainMaxT = 16;  // tokens of a decode chain: 1 (single-token launch) or 2 .. 16
bool dense1_supported(const Shape &s, int fmt);
hipError_t launch_dense1(const Shape &s, const WSet &w, const uint16_t *x, uint16_t *y, void *head,
                         hipStream_t st);
// One token through L layers, one single-token launch per layer: layer l + 1's token is
// y_l, or bf16(x_l + y_l) with `residual`, handed on through the workspace head.  x = null
// starts from the token a previous call left there (`hand_on`).  y: [L][H]; ids, tw: [L][k],
// logits [L][E], or null.
constexpr int kChainChunk = 16;  // layers whose descriptors the host gathers at a time
hipError_t launch_decode_chain(const Shape &s, const WSet *w, const float *const *Wr,
                               const float *const *bias, int L, bool residual, const uint16_t *x,
                               bool hand_on, uint16_t *y, int32_t *ids, float *tw, float *logits,
                               void *head, hipStream_t st);

// Streaming path (T <= kGemvMaxT) from an existing plan.
hipError_t launch_gemv_forward(const Shape &s, const WSet &w, int64_t T, const uint16_t *x,
                               const float *topk_w, const int32_t *sa, const int32_t *ap,
                               const Plan &plan, uint16_t *h, float *o, uint16_t *y, hipStream_t st);
hipError_t launch_gemm_forward(const Shape &s, const WSet &w, int64_t T, const uint16_t *x,
                               const float *topk_w, const int32_t *sa, const int32_t *ap,
                               const Plan &plan, uint16_t *h, uint16_t *o, uint16_t *y,
                               hipStream_t st);

// ---- device helpers -----------------------------------------------------------------
__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f2bf(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).
// Operand layout on a wave64: lane l holds A[l % 16][8 (l / 16) + i] and
// B[8 (l / 16) + i][l % 16] for i < 8; D[4 (l / 16) + i][l % 16] for i < 4.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }

// E4M3FN byte -> fp32 (exact; the NaN code is not expected in scale arrays).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c)
{
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
    return (c & 0x80u) ? -v : v;
}

// Eight E2M1 nibbles (one 32-bit word, low nibble first) times a block scale, as 8 bf16
// (4 words).  gfx950's FP4 conversion applies only the exponent of its scale operand (its
// sign too is ignored: a sweep over every finite E4M3 scale showed negative scales coming
// back positive), so it yields e2m1 * 2^floor(log2 |scale|) exactly; one fp32 multiply by
// the remaining signed mantissa factor (+-(1 + m/8) for an E4M3 scale) completes the
// product.  A 2-bit times a 4-bit significand is exact in fp32 and in bf16, so keeping the
// upper halves (v_perm_b32) is exact.  A zero scale gives zeros.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x4 dequant8(uint32_t q, float scale)
{
    const float mant = __uint_as_float((__float_as_uint(scale) & 0x807fffffu) | 0x3f800000u);
    const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, scale, 0);
    const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, scale, 1);
    const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, scale, 2);
    const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, scale, 3);
    auto pack = [mant](f32x2 v) {
        return __builtin_amdgcn_perm(__float_as_uint(v[1] * mant), __float_as_uint(v[0] * mant), 0x07060302u);
    };
    u32x4 r{pack(v0), pack(v1), pack(v2), pack(v3)};
    if (scale == 0.f) r = u32x4{0u, 0u, 0u, 0u};
    return r;
}
// The same values with one select instead of four: a zero scale gives a zero mantissa
// factor (the conversion itself then scales by 2^-127, still finite), so every product is
// (signed) zero.  The streaming kernels use this form, which measured 1-4 % faster there;
// the prefill GEMM keeps dequant8 (this form measured 8 % slower in it).
__device__ __forceinline__ u32x4 dequant8_stream(uint32_t q, float scale)
{
    const float mant = scale == 0.f ? 0.f : __uint_as_float((__float_as_uint(scale) & 0x807fffffu) | 0x3f800000u);
    const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, scale, 0);
    const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, scale, 1);
    const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, scale, 2);
    const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(q, scale, 3);
    auto pack = [mant](f32x2 v) {
        return __builtin_amdgcn_perm(__float_as_uint(v[1] * mant), __float_as_uint(v[0] * mant), 0x07060302u);
    };
    return u32x4{pack(v0), pack(v1), pack(v2), pack(v3)};
}

// INT4 (W4A16): signed nibble i of a word (two's complement, low nibble first) as an int.
__device__ __forceinline__ int int4_at(uint32_t q, int i)
{
    return (int)(q << (28 - 4 * i)) >> 28;
}

// Eight INT4 nibbles times their group scale, as 8 bf16 (4 words): each q * s is formed
// in fp32 (exact: 4 x 8 significant bits) and rounded once to bf16 (nearest even, two at
// a time by the packed conversion).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x4 dequant8_int4(uint32_t q, float scale)
{
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const f32x2_t v = {(float)int4_at(q, 2 * i) * scale, (float)int4_at(q, 2 * i + 1) * scale};
        const bf16x2_t b = __builtin_convertvector(v, bf16x2_t);
        w[i] = __builtin_bit_cast(uint32_t, b);
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}

// Eight INT4 nibbles as exact bf16 integers (4 words): a small integer converted to fp32
// has at most 4 significant bits, so its upper half is its bf16 value.
__device__ __forceinline__ u32x4 int4_bf16x8(uint32_t q)
{
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; i++)
        w[i] = __builtin_amdgcn_perm(__float_as_uint((float)int4_at(q, 2 * i + 1)),
                                     __float_as_uint((float)int4_at(q, 2 * i)), 0x07060302u);
    return u32x4{w[0], w[1], w[2], w[3]};
}

// Wave-wide reductions with DPP: xor-1 and xor-2 quad permutes, then the half-row and
// row mirrors leave every lane of a 16-lane row with the row's result; the four row
// results are read back as scalars.  A fixed combination order keeps sums deterministic.
#define FLINT_DPP(v, ctrl) __builtin_amdgcn_update_dpp((v), (v), (ctrl), 0xf, 0xf, false)
__device__ __forceinline__ float wave_sum(float v)
{
    v += __int_as_float(FLINT_DPP(__float_as_int(v), 0xB1));   // quad_perm [1,0,3,2]
    v += __int_as_float(FLINT_DPP(__float_as_int(v), 0x4E));   // quad_perm [2,3,0,1]
    v += __int_as_float(FLINT_DPP(__float_as_int(v), 0x141));  // row_half_mirror
    v += __int_as_float(FLINT_DPP(__float_as_int(v), 0x140));  // row_mirror
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (a + b) + (c + d);
}

// Router products of expert row e with the tokens t = t0 + ts q (q < TW, t < T), by one
// wave: a lane owns 8 consecutive h per 2048-wide slice (two float4 of the fp32 row and
// 16 bytes of each token's bf16 x), every load of a slice in flight together; out[q] =
// the fp32 sum over H (DPP-reduced, valid in every lane).
template <int TW>
__device__ __forceinline__ void router_dot_wave(int T, int H, int e, int t0, int ts,
                                                const uint16_t *__restrict__ x,
                                                const float *__restrict__ Wr, float *out)
{
    const int lane = threadIdx.x & 63;
    float acc[TW];
#pragma unroll
    for (int q = 0; q < TW; q++) acc[q] = 0.f;
    const float4 *w4 = reinterpret_cast<const float4 *>(Wr + (size_t)e * H);
    const int nc = H / 8;  // 8-element chunks per row
    for (int c0 = 0; c0 < nc; c0 += 256) {
        float4 w[8];
        u32x4 xv[TW][4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int c = c0 + lane + 64 * i;
            if (c < nc) {
                w[2 * i] = w4[2 * c];
                w[2 * i + 1] = w4[2 * c + 1];
            }
        }
#pragma unroll
        for (int q = 0; q < TW; q++) {
            const int t = t0 + ts * q;
            if (t < T)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int c = c0 + lane + 64 * i;
                    if (c < nc) xv[q][i] = *reinterpret_cast<const u32x4 *>(x + (size_t)t * H + 8 * c);
                }
        }
#pragma unroll
        for (int q = 0; q < TW; q++) {
            const int t = t0 + ts * q;
            if (t < T)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int c = c0 + lane + 64 * i;
                    if (c < nc) {
                        const float4 a = w[2 * i], b = w[2 * i + 1];
                        const uint32_t x0 = xv[q][i][0], x1 = xv[q][i][1], x2 = xv[q][i][2], x3 = xv[q][i][3];
                        float sum = acc[q];
                        sum += bf2f(x0 & 0xffffu) * a.x;
                        sum += bf2f(x0 >> 16) * a.y;
                        sum += bf2f(x1 & 0xffffu) * a.z;
                        sum += bf2f(x1 >> 16) * a.w;
                        sum += bf2f(x2 & 0xffffu) * b.x;
                        sum += bf2f(x2 >> 16) * b.y;
                        sum += bf2f(x3 & 0xffffu) * b.z;
                        sum += bf2f(x3 >> 16) * b.w;
                        acc[q] = sum;
                    }
                }
        }
    }
#pragma unroll
    for (int q = 0; q < TW; q++) out[q] = t0 + ts * q < T ? wave_sum(acc[q]) : 0.f;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v)
{
    v = max(v, (uint32_t)FLINT_DPP((int)v, 0xB1));
    v = max(v, (uint32_t)FLINT_DPP((int)v, 0x4E));
    v = max(v, (uint32_t)FLINT_DPP((int)v, 0x141));
    v = max(v, (uint32_t)FLINT_DPP((int)v, 0x140));
    const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(a, b), max(c, d));
}

// ---- top-k ---------------------------------------------------------------------------
// Order-preserving 64-bit key: high word = monotone image of the fp32 logit (-0 mapped to
// +0, NaN below -inf), low word = 0xffff - e so that equal logits prefer the lower index.
__device__ __forceinline__ uint64_t select_key(float v, int e)
{
    const uint32_t u = __float_as_uint(v);
    uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    ord = u == 0x80000000u ? 0x80000000u : ord;               // -0 == +0
    ord = (u & 0x7fffffffu) > 0x7f800000u ? 0u : ord;         // NaN: below everything
    return ((uint64_t)ord << 32) | (uint64_t)(0xffffu - (uint32_t)e);
}

// Four tokens per wave: the 16 lanes of DPP row g (lanes 16 g ... 16 g + 15) select for
// token t0 + g (rows past T do nothing useful and write nothing).  Lane L of a row holds
// experts L + 16 i (i < 16) as 32-bit keys: the order of the logit (select_key's high
// word) plus one, 0 = no expert or already taken, so a NaN logit (order 0) still ranks
// above those.  Each of the k rounds takes the row maximum of the keys and, among equal
// keys, the lowest expert: every lane offers its lowest matching expert and the row
// minimum wins.  Both reductions stay inside the row (DPP quad permutes and the half-row
// and row mirrors), so no cross-row or scalar step is on the dependent path.  The row's
// lane 0 writes ids[t][0..k) and the sigmoid weights (renormalised to sum 1 if renorm).
// lg: logits of token t at lg + t * ldl.
__device__ __forceinline__ uint32_t row16_max(uint32_t v)
{
    v = max(v, (uint32_t)FLINT_DPP((int)v, 0xB1));
    v = max(v, (uint32_t)FLINT_DPP((int)v, 0x4E));
    v = max(v, (uint32_t)FLINT_DPP((int)v, 0x141));
    v = max(v, (uint32_t)FLINT_DPP((int)v, 0x140));
    return v;
}
__device__ __forceinline__ uint32_t row16_min(uint32_t v)
{
    v = min(v, (uint32_t)FLINT_DPP((int)v, 0xB1));
    v = min(v, (uint32_t)FLINT_DPP((int)v, 0x4E));
    v = min(v, (uint32_t)FLINT_DPP((int)v, 0x141));
    v = min(v, (uint32_t)FLINT_DPP((int)v, 0x140));
    return v;
}
__device__ __forceinline__ void topk_4tokens(const float *__restrict__ lg, int ldl, int t0, int T, int E,
                                             int k, int renorm, int32_t *__restrict__ ids,
                                             float *__restrict__ wout)
{
    const int lane = threadIdx.x & 63, g = lane >> 4, L = lane & 15, t = t0 + g;
    const bool live = t < T;
    const float *lt = lg + (size_t)(live ? t : t0) * ldl;
    float lv[16];
#pragma unroll
    for (int i = 0; i < 16; i++) lv[i] = lt[L + 16 * i < E ? L + 16 * i : 0];  // all reads in flight together
    uint32_t key[16];
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int e = L + 16 * i;
        key[i] = (live && e < E) ? (uint32_t)(select_key(lv[i], e) >> 32) + 1u : 0u;
    }
    int sel[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        if (j >= k) break;
        uint32_t m = key[0];
#pragma unroll
        for (int i = 1; i < 16; i++) m = max(m, key[i]);
        m = row16_max(m);
        uint32_t first = 0xffffu;  // this lane's lowest expert with key m
#pragma unroll
        for (int i = 15; i >= 0; i--)
            if (key[i] == m) first = (uint32_t)(L + 16 * i);
        const uint32_t win = row16_min(first);
#pragma unroll
        for (int i = 0; i < 16; i++)
            if ((uint32_t)(L + 16 * i) == win) key[i] = 0u;
        sel[j] = (int)win;
    }
    if (live && L == 0) {
        float sg[8];
        float sum = 0.f;
        for (int j = 0; j < k; j++) {
            sg[j] = 1.0f / (1.0f + expf(-lt[sel[j]]));
            sum += sg[j];
        }
        for (int j = 0; j < k; j++) {
            ids[(size_t)t * k + j] = sel[j];
            wout[(size_t)t * k + j] = renorm ? sg[j] / sum : sg[j];
        }
    }
}

// One token per wave (the small-batch launch, where the selecting workgroup has more waves
// than tokens): lane l holds experts l + 64 i (i < 4) as the same 32-bit keys.  Each round
// takes the wave maximum; among equal keys the lowest expert wins: the first i with a match
// in any lane (one ballot per i), and in it the lowest lane.  Lane j < k then writes
// ids[j] and the j-th sigmoid weight (renormalised over the k selected, summed in j order).
// lt: the token's E logits.
__device__ __forceinline__ void topk_wave(const float *__restrict__ lt, int E, int k, int renorm,
                                          int32_t *__restrict__ ids, float *__restrict__ wout)
{
    const int lane = threadIdx.x & 63;
    float lv[4];
#pragma unroll
    for (int i = 0; i < 4; i++) lv[i] = lt[lane + 64 * i < E ? lane + 64 * i : 0];
    uint32_t key[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int e = lane + 64 * i;
        key[i] = e < E ? (uint32_t)(select_key(lv[i], e) >> 32) + 1u : 0u;
    }
    int mine = 0;  // lane j < k: the j-th selected expert
#pragma unroll
    for (int j = 0; j < 8; j++) {
        if (j >= k) break;
        const uint32_t m = wave_max_u32(max(max(key[0], key[1]), max(key[2], key[3])));
        const uint64_t b0 = __ballot(key[0] == m), b1 = __ballot(key[1] == m);
        const uint64_t b2 = __ballot(key[2] == m), b3 = __ballot(key[3] == m);
        const int i = b0 ? 0 : b1 ? 1 : b2 ? 2 : 3;
        const int wl = __builtin_ctzll(b0 ? b0 : b1 ? b1 : b2 ? b2 : b3);
        if (lane == wl) {
            key[0] = i == 0 ? 0u : key[0];
            key[1] = i == 1 ? 0u : key[1];
            key[2] = i == 2 ? 0u : key[2];
            key[3] = i == 3 ? 0u : key[3];
        }
        if (lane == j) mine = wl + 64 * i;
    }
    const float sg = 1.0f / (1.0f + expf(-lt[lane < k ? mine : 0]));
    float sum = 0.f;
    for (int j = 0; j < k; j++) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sg), j));
    if (lane < k) {
        ids[lane] = mine;
        wout[lane] = renorm ? sg / sum : sg;
    }
}


}  // namespace flint
