// route.hip -- router logits and top-k selection.
//
// Router (recipes.vllm.ai "RecursiveSI/flint", Overview: sigmoid routing over 256
// experts): logits[t][e] = sum_h x[t][h] * Wr[e][h] (+ bias[e]), fp32 accumulation.
// Selection (neoteo.com specification table, row "Eksperci": 6 of 256 routed experts per
// token): top-k by (logit descending, index ascending), sigmoid weights renormalised.
#include "common.h"

namespace flint {

// ---------------------------------------------------------------- decode router (T <= 32)
// One wave per expert row: the fp32 row is read once (all 16-byte loads of a 2 KB slice in
// flight together) and dotted against every token (x is tiny and stays in L2).  E
// single-wave workgroups stream the whole router matrix from all CUs at once.
template <int MAXT>
__global__ __launch_bounds__(64) void router_small_kernel(int T, int H, int E,
                                                          const uint16_t *__restrict__ x,
                                                          const float *__restrict__ Wr,
                                                          const float *__restrict__ bias,
                                                          float *__restrict__ logits)
{
    const int e = blockIdx.x;
    const int lane = threadIdx.x;
    float acc[MAXT];
#pragma unroll
    for (int t = 0; t < MAXT; t++) acc[t] = 0.f;
    const float4 *w4 = reinterpret_cast<const float4 *>(Wr + (size_t)e * H);
    constexpr int NB = 8;  // float4 loads per lane per batch (a 2048-wide slice)
    for (int c0 = 0; c0 < H / 4; c0 += 64 * NB) {
        float4 w[NB];
#pragma unroll
        for (int i = 0; i < NB; i++) {
            const int c = c0 + 64 * i + lane;
            w[i] = c < H / 4 ? w4[c] : float4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int t = 0; t < MAXT; t++) {
            if (t < T) {
                const uint16_t *xt = x + (size_t)t * H;
#pragma unroll
                for (int i = 0; i < NB; i++) {
                    const int c = c0 + 64 * i + lane;
                    if (c < H / 4) {
                        u32x2 xv = *reinterpret_cast<const u32x2 *>(xt + 4 * c);
                        acc[t] += bf2f(xv[0] & 0xffffu) * w[i].x;
                        acc[t] += bf2f(xv[0] >> 16) * w[i].y;
                        acc[t] += bf2f(xv[1] & 0xffffu) * w[i].z;
                        acc[t] += bf2f(xv[1] >> 16) * w[i].w;
                    }
                }
            }
        }
    }
    const float b = bias ? bias[e] : 0.f;
#pragma unroll
    for (int t = 0; t < MAXT; t++) {
        if (t < T) {
            float s = wave_sum(acc[t]);
            if (lane == 0) logits[(size_t)t * E + e] = s + b;
        }
    }
}

// ---------------------------------------------------------------- prefill router (T > 32)
// Tiled fp32 GEMM: a 64-token x 64-expert tile per 256-thread workgroup, K staged in
// LDS 32 at a time, 4x4 outputs per thread.
__global__ __launch_bounds__(256) void router_tiled_kernel(int T, int H, int E,
                                                           const uint16_t *__restrict__ x,
                                                           const float *__restrict__ Wr,
                                                           const float *__restrict__ bias,
                                                           float *__restrict__ logits)
{
    __shared__ float xs[32][64 + 4];
    __shared__ float ws[32][64 + 4];
    const int t0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;  // thread owns tokens ty*4.., experts tx*4..
    float acc[4][4] = {};
    for (int k0 = 0; k0 < H; k0 += 32) {
        // stage 64 x 32 of x (bf16 -> f32) and 64 x 32 of Wr, transposed to [k][row]
        for (int i = tid; i < 64 * 32; i += 256) {
            int r = i / 32, kk = i % 32;
            int t = min(t0 + r, T - 1);
            xs[kk][r] = bf2f(x[(size_t)t * H + k0 + kk]);
            int e = min(e0 + r, E - 1);
            ws[kk][r] = Wr[(size_t)e * H + k0 + kk];
        }
        __syncthreads();
#pragma unroll 8
        for (int kk = 0; kk < 32; kk++) {
            float a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; i++) a[i] = xs[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; j++) b[j] = ws[kk][tx * 4 + j];
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < 4; j++) acc[i][j] += a[i] * b[j];
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; i++) {
        int t = t0 + ty * 4 + i;
        if (t >= T) continue;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            int e = e0 + tx * 4 + j;
            if (e < E) logits[(size_t)t * E + e] = acc[i][j] + (bias ? bias[e] : 0.f);
        }
    }
}

hipError_t launch_router(const Shape &s, int64_t T, const uint16_t *x, const float *Wr,
                         const float *bias, float *logits, hipStream_t st)
{
    if (T <= 8) {
        router_small_kernel<8><<<s.E, 64, 0, st>>>((int)T, s.H, s.E, x, Wr, bias, logits);
    } else if (T <= 32) {
        router_small_kernel<32><<<s.E, 64, 0, st>>>((int)T, s.H, s.E, x, Wr, bias, logits);
    } else {
        dim3 grid((unsigned)((T + 63) / 64), (unsigned)((s.E + 63) / 64));
        router_tiled_kernel<<<grid, 256, 0, st>>>((int)T, s.H, s.E, x, Wr, bias, logits);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- top-k select
// One wave per token; each lane holds experts lane, lane+64, lane+128, lane+192.
// k rounds of a wave-wide arg-max; the winning lane retires its entry.
__global__ __launch_bounds__(256) void topk_kernel(int T, int E, int k, int renorm,
                                                   const float *__restrict__ logits,
                                                   int32_t *__restrict__ ids,
                                                   float *__restrict__ wout)
{
    const int t = blockIdx.x * 4 + threadIdx.x / 64;
    if (t >= T) return;
    topk_token(logits + (size_t)t * E, E, k, renorm, ids + (size_t)t * k, wout + (size_t)t * k);
}

hipError_t launch_topk(const Shape &s, int64_t T, const float *logits, int32_t *ids, float *w,
                       hipStream_t st)
{
    unsigned blocks = (unsigned)((T + 3) / 4);
    topk_kernel<<<blocks, 256, 0, st>>>((int)T, s.E, s.k, s.renorm, logits, ids, w);
    return hipGetLastError();
}

}  // namespace flint
