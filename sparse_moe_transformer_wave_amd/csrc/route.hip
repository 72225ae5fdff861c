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
// computations", ARITH 2019).  Tile: 128 tokens x 64 experts x 64 K per 512-thread
// workgroup (two waves per SIMD); wave w owns 16 experts (w % 4) x 64 tokens (w / 4)
// (4 MFMA tiles, 3 MFMAs each), so a wave reads its 3 weight-part fragments once per
// 32-K step and its 4 token fragments serve all of them (the weight parts are the larger
// operand: splitting the tile by tokens only made every wave re-read all 3 x 64 expert
// rows from LDS).  Global loads run two K steps ahead in registers (stage k + 2 is
// fetched while stage k is multiplied and stage k + 1 waits to be split into LDS).  LDS
// rows are 128 bytes with 16-byte chunk c of row R at slot c ^ (R & 7): the fragment reads
// (16 rows, one chunk each) then run at the LDS's full rate; with rows padded to 144 bytes
// they took twice as long (two-way bank conflicts, measured on gfx950).  The kernel's time
// barely moved with it (54.8 -> 53.8 us at T = 8192): its reads are not what bounds it.
namespace {
constexpr int RBM = 128, RBN = 64, RBK = 64;

// byte offset of 16-byte chunk c (of 8) of row R in a 128-byte-row tile
__device__ __forceinline__ int rsw(int R, int c) { return R * 128 + 16 * (c ^ (R & 7)); }

__device__ __forceinline__ uint32_t trunc_bf16(float v) { return __float_as_uint(v) >> 16; }

constexpr int RNT = 512;  // threads per workgroup
struct RouterStage {
    u32x4 a[2];   // token chunks tid + 512 j: row c / 8, 8 bf16 at column 8 (c % 8)
    float4 b[2];  // weight chunks tid + 512 j: row c / 16, 4 fp32 at column 4 (c % 16)
};
}  // namespace

__global__ __launch_bounds__(RNT) void router_mfma_kernel(int T, int H, int E,
                                                          const uint16_t *__restrict__ x,
                                                          const float *__restrict__ Wr,
                                                          const float *__restrict__ bias,
                                                          float *__restrict__ logits)
{
    __shared__ __attribute__((aligned(16))) uint8_t As[2][RBM * 128];
    __shared__ __attribute__((aligned(16))) uint8_t Bs[2][3][RBN * 128];
    const int t0 = blockIdx.x * RBM, e0 = blockIdx.y * RBN;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
    const int we = wave & 3, wt = wave >> 2;  // expert group, token half
    f32x4 acc[4];
#pragma unroll
    for (int i = 0; i < 4; i++) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t *xa[2];
    const float *wb[2];
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int c = tid + RNT * j;
        xa[j] = x + (size_t)min(t0 + (c >> 3), T - 1) * H + (c & 7) * 8;
        wb[j] = Wr + (size_t)min(e0 + (c >> 4), E - 1) * H + (c & 15) * 4;
    }
    auto gload = [&](int k0, RouterStage &st) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            st.a[j] = *reinterpret_cast<const u32x4 *>(xa[j] + k0);
            st.b[j] = *reinterpret_cast<const float4 *>(wb[j] + k0);
        }
    };
    auto lstore = [&](int buf, const RouterStage &st) {
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int c = tid + RNT * j;
            *reinterpret_cast<u32x4 *>(&As[buf][rsw(c >> 3, c & 7)]) = st.a[j];
            const float vv[4] = {st.b[j].x, st.b[j].y, st.b[j].z, st.b[j].w};
            uint32_t hi[4], mid[4], lo[4];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                hi[q] = trunc_bf16(vv[q]);
                const float r1 = vv[q] - __uint_as_float(hi[q] << 16);
                mid[q] = trunc_bf16(r1);
                const float r2 = r1 - __uint_as_float(mid[q] << 16);
                lo[q] = f2bf(r2);
            }
            const int row = c >> 4, q = c & 15;  // 8 bytes: half q % 2 of chunk q / 2
            const int off = rsw(row, q >> 1) + 8 * (q & 1);
            *reinterpret_cast<u32x2 *>(&Bs[buf][0][off]) = u32x2{hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16)};
            *reinterpret_cast<u32x2 *>(&Bs[buf][1][off]) = u32x2{mid[0] | (mid[1] << 16), mid[2] | (mid[3] << 16)};
            *reinterpret_cast<u32x2 *>(&Bs[buf][2][off]) = u32x2{lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16)};
        }
    };
    auto compute = [&](int buf) {
#pragma unroll
        for (int kk = 0; kk < RBK / 32; kk++) {
            bf16x8 bfr[3];
#pragma unroll
            for (int part = 0; part < 3; part++)
                bfr[part] = as_bf16x8(*reinterpret_cast<const u32x4 *>(&Bs[buf][part][rsw(we * 16 + r, kk * 4 + g)]));
#pragma unroll
            for (int ms = 0; ms < 4; ms++) {
                const bf16x8 af = as_bf16x8(*reinterpret_cast<const u32x4 *>(&As[buf][rsw(wt * 64 + ms * 16 + r, kk * 4 + g)]));
#pragma unroll
                for (int part = 0; part < 3; part++) acc[ms] = mfma16x16x32(af, bfr[part], acc[ms]);
            }
        }
    };
    // Iteration kt: stage kt in LDS buffer kt % 2, stage kt + 1 in flight in registers
    // (issued two iterations ago), stage kt + 2 issued now into the registers freed by the
    // previous iteration's store.
    const int nk = H / RBK;  // >= 1 (H is a multiple of 64)
    RouterStage s0, s1;
    gload(0, s0);
    if (nk > 1) gload(RBK, s1);
    lstore(0, s0);
    __syncthreads();
    auto step = [&](int kt, RouterStage &nxt, RouterStage &fill) {
        if (kt + 2 < nk) gload((kt + 2) * RBK, fill);
        compute(kt & 1);
        if (kt + 1 < nk) lstore((kt + 1) & 1, nxt);
        __syncthreads();
    };
    for (int kt = 0; kt < nk; kt += 2) {
        step(kt, s1, s0);                      // stage kt + 1 sits in s1; s0 (stored) takes stage kt + 2
        if (kt + 1 < nk) step(kt + 1, s0, s1);  // stage kt + 2 sits in s0; s1 takes stage kt + 3
    }
    // acc[ms][i] = logit of token t0 + wt*64 + ms*16 + 4g + i, expert e0 + we*16 + r
    const int e = e0 + we * 16 + r;
    const float bv = (bias && e < E) ? bias[e] : 0.f;
#pragma unroll
    for (int ms = 0; ms < 4; ms++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int t = t0 + wt * 64 + ms * 16 + 4 * g + i;
            if (t < T && e < E) logits[(size_t)t * E + e] = acc[ms][i] + bv;
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
        router_mfma_kernel<<<grid, RNT, 0, st>>>((int)T, s.H, s.E, x, Wr, bias, logits);
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
