// route.hip -- router logits and top-k selection.
//
// Router (recipes.vllm.ai "RecursiveSI/flint", Overview: sigmoid routing over 256
// experts): logits[t][e] = sum_h x[t][h] * Wr[e][h] (+ bias[e]), fp32 accumulation.
// Selection (neoteo.com specification table, row "Eksperci": 6 of 256 routed experts per
// token): top-k by (logit descending, index ascending), sigmoid weights renormalised.
#include "common.h"

namespace flint {

// ---------------------------------------------------------------- decode router (T <= 32)
// One 256-thread workgroup per expert row; wave w takes tokens w, w + 4, ...  A lane owns 8
// consecutive h (two float4 of the fp32 row, 16 bytes of each token's bf16 x), so every
// load is 16 bytes and all of a wave's loads for a 2048-wide slice are in flight together;
// the row comes from HBM once per workgroup (the other waves hit in cache) and x stays in
// L2.  Each wave reduces its tokens' sums with DPP.
template <int MAXT>
__global__ __launch_bounds__(256) void router_small_kernel(int T, int H, int E,
                                                           const uint16_t *__restrict__ x,
                                                           const float *__restrict__ Wr,
                                                           const float *__restrict__ bias,
                                                           float *__restrict__ logits)
{
    constexpr int TW = (MAXT + 3) / 4;  // tokens per wave
    const int e = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    float sums[TW];
    router_dot_wave<TW>(T, H, e, wave, 4, x, Wr, sums);
    const float bv = bias ? bias[e] : 0.f;
#pragma unroll
    for (int q = 0; q < TW; q++) {
        const int t = wave + 4 * q;
        if (t < T && lane == 0) logits[(size_t)t * E + e] = sums[q] + bv;
    }
}

// ---------------------------------------------------------------- prefill router (T > 32)
// bf16 MFMA with the fp32 router weights split exactly into three bf16 parts:
//   hi = w truncated to bf16, mid = (w - hi) truncated, lo = (w - hi - mid) (exact in bf16),
// so every product x * part is exact in the fp32 accumulator and
// x . w = x . hi + x . mid + x . lo up to fp32 summation rounding (the split is the
// three-term bf16 decomposition of an fp32 operand; Henry, Tang and Heinecke,
// "Leveraging the bfloat16 artificial intelligence datatype for higher-precision
// computations", ARITH 2019).  Tile: 128 tokens x 64 experts x 64 K per 256-thread
// workgroup; each wave owns 32 tokens x 64 experts (2 x 4 MFMA tiles, 3 MFMAs each).
namespace {
constexpr int RBM = 128, RBN = 64, RBK = 32, RLD = RBK + 8;

__device__ __forceinline__ uint32_t trunc_bf16(float v) { return __float_as_uint(v) >> 16; }
}  // namespace

__global__ __launch_bounds__(256) void router_mfma_kernel(int T, int H, int E,
                                                          const uint16_t *__restrict__ x,
                                                          const float *__restrict__ Wr,
                                                          const float *__restrict__ bias,
                                                          float *__restrict__ logits)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[2][RBM][RLD];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][3][RBN][RLD];
    const int t0 = blockIdx.x * RBM, e0 = blockIdx.y * RBN;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
    f32x4 acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // staging: A 128 rows x 4 chunks of 8 bf16 (2 per thread); B 64 rows x 8 float4 (2 per thread)
    const uint16_t *xa[2];
    const float *wb[2];
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int c = tid + 256 * j;
        xa[j] = x + (size_t)min(t0 + (c >> 2), T - 1) * H + (c & 3) * 8;
        wb[j] = Wr + (size_t)min(e0 + (c >> 3), E - 1) * H + (c & 7) * 4;
    }
    u32x4 ra[2];
    float4 rb[2];
    auto gload = [&](int k0) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            ra[j] = *reinterpret_cast<const u32x4 *>(xa[j] + k0);
            rb[j] = *reinterpret_cast<const float4 *>(wb[j] + k0);
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int c = tid + 256 * j;
            *reinterpret_cast<u32x4 *>(&As[buf][c >> 2][(c & 3) * 8]) = ra[j];
            const float vv[4] = {rb[j].x, rb[j].y, rb[j].z, rb[j].w};
            uint32_t hi[4], mid[4], lo[4];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                hi[q] = trunc_bf16(vv[q]);
                const float r1 = vv[q] - __uint_as_float(hi[q] << 16);
                mid[q] = trunc_bf16(r1);
                const float r2 = r1 - __uint_as_float(mid[q] << 16);
                lo[q] = f2bf(r2);
            }
            const int row = c >> 3, col = (c & 7) * 4;
            *reinterpret_cast<u32x2 *>(&Bs[buf][0][row][col]) = u32x2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
            *reinterpret_cast<u32x2 *>(&Bs[buf][1][row][col]) = u32x2{mid[0] | (mid[1] << 16), mid[2] | (mid[3] << 16)};
            *reinterpret_cast<u32x2 *>(&Bs[buf][2][row][col]) = u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
        }
    };
    const int nk = H / RBK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt++) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * RBK);
        bf16x8 af[2];
#pragma unroll
        for (int ms = 0; ms < 2; ms++)
            af[ms] = as_bf16x8(*reinterpret_cast<const u32x4 *>(&As[buf][wave * 32 + ms * 16 + r][g * 8]));
#pragma unroll
        for (int part = 0; part < 3; part++) {
#pragma unroll
            for (int ns = 0; ns < 4; ns++) {
                const bf16x8 bfr = as_bf16x8(*reinterpret_cast<const u32x4 *>(&Bs[buf][part][ns * 16 + r][g * 8]));
#pragma unroll
                for (int ms = 0; ms < 2; ms++) acc[ms][ns] = mfma16x16x32(af[ms], bfr, acc[ms][ns]);
            }
        }
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }
    // acc[ms][ns][i] = logit of token t0 + wave*32 + ms*16 + 4g + i, expert e0 + ns*16 + r
#pragma unroll
    for (int ms = 0; ms < 2; ms++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int t = t0 + wave * 32 + ms * 16 + 4 * g + i;
            if (t >= T) continue;
#pragma unroll
            for (int ns = 0; ns < 4; ns++) {
                const int e = e0 + ns * 16 + r;
                if (e < E) logits[(size_t)t * E + e] = acc[ms][ns][i] + (bias ? bias[e] : 0.f);
            }
        }
}

hipError_t launch_router(const Shape &s, int64_t T, const uint16_t *x, const float *Wr,
                         const float *bias, float *logits, hipStream_t st)
{
    if (T <= 8) {
        router_small_kernel<8><<<s.E, 256, 0, st>>>((int)T, s.H, s.E, x, Wr, bias, logits);
    } else if (T <= 32) {
        router_small_kernel<32><<<s.E, 256, 0, st>>>((int)T, s.H, s.E, x, Wr, bias, logits);
    } else {
        dim3 grid((unsigned)((T + RBM - 1) / RBM), (unsigned)((s.E + RBN - 1) / RBN));
        router_mfma_kernel<<<grid, 256, 0, st>>>((int)T, s.H, s.E, x, Wr, bias, logits);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------- top-k select
// Four tokens per wave (16 lanes each), four waves per workgroup.
__global__ __launch_bounds__(256) void topk_kernel(int T, int E, int k, int renorm,
                                                   const float *__restrict__ logits,
                                                   int32_t *__restrict__ ids,
                                                   float *__restrict__ wout)
{
    const int t0 = blockIdx.x * 16 + (threadIdx.x >> 6) * 4;
    if (t0 >= T) return;
    topk_4tokens(logits, E, t0, T, E, k, renorm, ids, wout);
}

hipError_t launch_topk(const Shape &s, int64_t T, const float *logits, int32_t *ids, float *w,
                       hipStream_t st)
{
    unsigned blocks = (unsigned)((T + 15) / 16);
    topk_kernel<<<blocks, 256, 0, st>>>((int)T, s.E, s.k, s.renorm, logits, ids, w);
    return hipGetLastError();
}

}  // namespace flint
