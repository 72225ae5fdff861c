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
// Grouped GEMM tile: BM rows (tokens) x 128 B-rows x 64 K.
constexpr int kGemmBM = 128;

// One weight matrix kind (gate, up or down) of all experts.
// Routed expert e (< E) lives at routed + e * mat_bytes; the shared expert at `shared`.
// NVFP4 adds block scales (sf_*) and fp32 tensor scales (ts_routed[e], *ts_shared).
struct WMat {
    const uint8_t *routed, *shared;
    const uint8_t *sf_routed, *sf_shared;
    const float *ts_routed, *ts_shared;
};
struct WSet {
    int fmt;  // 0 bf16, 1 nvfp4
    WMat gate, up, down;
};

// Per-expert work description built on the device from the expert offsets.
//   meta[0] = number of touched experts U' (routed with a token, then the shared one)
//   meta[1] = number of grouped-GEMM items
//   touched[u], tbase[u] (first slot), tcount[u] (rows) for u < U'
//   items[i] = (u << 16) | m_tile
//   counters[H/16] completion counters of the decode down pass (zeroed by the planner)
struct Plan {
    int *meta;
    int *touched, *tbase, *tcount;
    int *items;
    int *counters;
};

// Workspace carve-up (byte offsets from the workspace base), computed on the host.
struct WsLayout {
    size_t logits, ids, w, counts, offsets, sa, ap;
    size_t plan, h, o;
    size_t total;
    int max_items;
};
WsLayout ws_layout(const Shape &s, int64_t T);
Plan plan_view(void *ws, const WsLayout &L, const Shape &s);

// ---- launches (return hipSuccess or the launch error) -----------------------------
hipError_t launch_router(const Shape &s, int64_t T, const uint16_t *x, const float *Wr,
                         const float *bias, float *logits, hipStream_t st);
hipError_t launch_topk(const Shape &s, int64_t T, const float *logits, int32_t *ids, float *w,
                       hipStream_t st);
hipError_t launch_permute(const Shape &s, int64_t T, const int32_t *ids, int32_t *counts,
                          int32_t *offsets, int32_t *sa, int32_t *ap, const Plan *plan,
                          hipStream_t st);
hipError_t launch_plan(const Shape &s, int64_t T, const int32_t *offsets, const Plan &plan,
                       hipStream_t st);
hipError_t launch_gemv_forward(const Shape &s, const WSet &w, int64_t T, const uint16_t *x,
                               const float *topk_w, const int32_t *sa, const int32_t *ap,
                               const Plan &plan, float *h, float *o32, uint16_t *y,
                               hipStream_t st);
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

// One E2M1 nibble times a block scale, as bf16 bits.  The product of a 2-bit and a
// 4-bit significand is exact in fp32 and in bf16, so truncating to bf16 is exact.
__device__ __forceinline__ uint32_t e2m1_scaled_bf16(uint32_t nib, float scale)
{
    uint32_t mag = nib & 7u;
    float v = (mag < 2u) ? 0.5f * (float)mag : __uint_as_float((mag << 22) + (126u << 23));
    uint32_t b = __float_as_uint(v * scale) >> 16;
    return b | ((nib & 8u) << 12);
}

// Eight E2M1 nibbles (one 32-bit word, low nibble first) x scale -> 8 bf16 (4 words).
__device__ __forceinline__ u32x4 dequant8(uint32_t q, float scale)
{
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        uint32_t lo = e2m1_scaled_bf16((q >> (8 * i)) & 15u, scale);
        uint32_t hi = e2m1_scaled_bf16((q >> (8 * i + 4)) & 15u, scale);
        r[i] = lo | (hi << 16);
    }
    return r;
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

}  // namespace flint
