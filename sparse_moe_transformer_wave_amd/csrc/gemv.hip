// gemv.hip -- the streaming expert path for small batches (T <= 32 tokens).
//
// Decode reads every touched expert's weights once from HBM; the cost of a step is the
// active weights, not the checkpoint (qantcore.space review, section 01).  Weights stream
// straight from HBM into MFMA B operands with 16-byte loads (no LDS staging, no reuse to
// exploit); the expert's tokens (<= 32, two 16-row MFMA tiles) form the A operand and
// come from L2.  The shared expert is one more entry of the touched-expert list
// (news.ditty.ir, third paragraph: one shared expert always active).
//
// Pass 1 (gate/up): one workgroup per (touched expert, 16 rows of I); its 4 waves split
//   K and meet in LDS; h = silu(g) * u is stored in fp32.
// Pass 2 (down + combine): one workgroup per (touched expert, 16 rows of H); the fp32 h
//   enters the bf16 MFMA as hi + lo parts, so it keeps ~16 significant bits.  Per-slot
//   outputs go to an fp32 buffer; the last workgroup to finish a 16-row block of H
//   combines it (shared first, then the k routed slots in order) and writes bf16 y.
#include "common.h"

#include <algorithm>

namespace flint {

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

__device__ __forceinline__ const uint8_t *expert_base(const WMat &m, int e, int E, size_t bytes)
{
    return e == E ? m.shared : m.routed + (size_t)e * bytes;
}
__device__ __forceinline__ const uint8_t *expert_sf(const WMat &m, int e, int E, size_t bytes)
{
    return e == E ? m.sf_shared : m.sf_routed + (size_t)e * bytes;
}
__device__ __forceinline__ float expert_ts(const WMat &m, int e, int E)
{
    return e == E ? *m.ts_shared : m.ts_routed[e];
}

// fp32 x8 -> (hi, lo) bf16 x8 with hi = rne(v), lo = rne(v - hi).
__device__ __forceinline__ void split_bf16x8(const float *v, u32x4 &hi, u32x4 &lo)
{
#pragma unroll
    for (int i = 0; i < 4; i++) {
        uint32_t h0 = f2bf(v[2 * i]), h1 = f2bf(v[2 * i + 1]);
        uint32_t l0 = f2bf(v[2 * i] - bf2f(h0)), l1 = f2bf(v[2 * i + 1] - bf2f(h1));
        hi[i] = h0 | (h1 << 16);
        lo[i] = l0 | (l1 << 16);
    }
}

// ------------------------------------------------------------------ pass 1: gate / up
template <int FMT>
__global__ __launch_bounds__(256) void gemv_gateup_kernel(int H, int I, int E, int k, WSet w,
                                                          const uint16_t *__restrict__ x,
                                                          const int32_t *__restrict__ sa,
                                                          Plan p, float *__restrict__ h)
{
    __shared__ float red[4][2][2][64][4];
    const int nrb = I / 16;
    const int u = blockIdx.x / nrb, rb = blockIdx.x - u * nrb;
    if (u >= p.meta[0]) return;
    const int e = p.touched[u], base = p.tbase[u], cnt = p.tcount[u];
    const bool sh = (e == E);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
    const int nmt = (cnt + 15) >> 4;
    const uint16_t *xr[2];
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
        int idx = min(mt * 16 + r, cnt - 1);
        int tok = sh ? idx : sa[base + idx] / k;
        xr[mt] = x + (size_t)tok * H;
    }
    const int row = rb * 16 + r;
    f32x4 ag[2] = {}, au[2] = {};
    float tsg = 1.f, tsu = 1.f;
    if (FMT == 0) {
        const size_t mb = (size_t)I * H * 2;
        const uint16_t *Wg = reinterpret_cast<const uint16_t *>(expert_base(w.gate, e, E, mb)) + (size_t)row * H;
        const uint16_t *Wu = reinterpret_cast<const uint16_t *>(expert_base(w.up, e, E, mb)) + (size_t)row * H;
        const int nch = H / 32;
        constexpr int UNR = 8;
        for (int c0 = wave; c0 < nch; c0 += 4 * UNR) {
            u32x4 bg[UNR], bu[UNR], a0[UNR], a1[UNR];
#pragma unroll
            for (int i = 0; i < UNR; i++) {
                int c = c0 + 4 * i;
                if (c < nch) {
                    int k0 = c * 32 + g * 8;
                    bg[i] = ld16(Wg + k0);
                    bu[i] = ld16(Wu + k0);
                    a0[i] = ld16(xr[0] + k0);
                    if (nmt > 1) a1[i] = ld16(xr[1] + k0);
                }
            }
#pragma unroll
            for (int i = 0; i < UNR; i++) {
                int c = c0 + 4 * i;
                if (c < nch) {
                    ag[0] = mfma16x16x32(as_bf16x8(a0[i]), as_bf16x8(bg[i]), ag[0]);
                    au[0] = mfma16x16x32(as_bf16x8(a0[i]), as_bf16x8(bu[i]), au[0]);
                    if (nmt > 1) {
                        ag[1] = mfma16x16x32(as_bf16x8(a1[i]), as_bf16x8(bg[i]), ag[1]);
                        au[1] = mfma16x16x32(as_bf16x8(a1[i]), as_bf16x8(bu[i]), au[1]);
                    }
                }
            }
        }
    } else {
        // NVFP4: a lane takes 32 consecutive k (16 bytes of codes, 2 block scales) of its
        // row per 128-wide super-chunk; MFMA j consumes the lane's k + 8j .. k + 8j + 7.
        const size_t mb = (size_t)I * H / 2, sb = (size_t)I * H / 16;
        const uint8_t *Qg = expert_base(w.gate, e, E, mb) + (size_t)row * (H / 2);
        const uint8_t *Qu = expert_base(w.up, e, E, mb) + (size_t)row * (H / 2);
        const uint8_t *Sg = expert_sf(w.gate, e, E, sb) + (size_t)row * (H / 16);
        const uint8_t *Su = expert_sf(w.up, e, E, sb) + (size_t)row * (H / 16);
        tsg = expert_ts(w.gate, e, E);
        tsu = expert_ts(w.up, e, E);
        const int nsc = H / 128;
        for (int sc = wave; sc < nsc; sc += 4) {
            const int kb = sc * 128 + g * 32;
            u32x4 qg = ld16(Qg + kb / 2), qu = ld16(Qu + kb / 2);
            uint32_t sgb = *reinterpret_cast<const uint16_t *>(Sg + kb / 16);
            uint32_t sub = *reinterpret_cast<const uint16_t *>(Su + kb / 16);
            u32x4 a0[4], a1[4];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                a0[j] = ld16(xr[0] + kb + 8 * j);
                if (nmt > 1) a1[j] = ld16(xr[1] + kb + 8 * j);
            }
#pragma unroll
            for (int j = 0; j < 4; j++) {
                float sgf = e4m3_to_f32((sgb >> (8 * (j >> 1))) & 0xffu);
                float suf = e4m3_to_f32((sub >> (8 * (j >> 1))) & 0xffu);
                bf16x8 bg = as_bf16x8(dequant8(qg[j], sgf));
                bf16x8 bu = as_bf16x8(dequant8(qu[j], suf));
                ag[0] = mfma16x16x32(as_bf16x8(a0[j]), bg, ag[0]);
                au[0] = mfma16x16x32(as_bf16x8(a0[j]), bu, au[0]);
                if (nmt > 1) {
                    ag[1] = mfma16x16x32(as_bf16x8(a1[j]), bg, ag[1]);
                    au[1] = mfma16x16x32(as_bf16x8(a1[j]), bu, au[1]);
                }
            }
        }
    }
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            red[wave][mt][0][lane][i] = ag[mt][i];
            red[wave][mt][1][lane][i] = au[mt][i];
        }
    __syncthreads();
    for (int j = tid; j < nmt * 256; j += 256) {
        const int mt = j >> 8, rem = j & 255, l = rem >> 2, i = rem & 3;
        float gs = 0.f, us = 0.f;
#pragma unroll
        for (int wv = 0; wv < 4; wv++) {
            gs += red[wv][mt][0][l][i];
            us += red[wv][mt][1][l][i];
        }
        const int m = 4 * (l >> 4) + i, n = l & 15;
        const int ti = mt * 16 + m;
        if (ti < cnt) h[(size_t)(base + ti) * I + rb * 16 + n] = silu(gs * tsg) * (us * tsu);
    }
}

// ------------------------------------------------------------------ pass 2: down + combine
template <int FMT>
__global__ __launch_bounds__(128) void gemv_down_kernel(int T, int H, int I, int E, int k, int S,
                                                        WSet w, const float *__restrict__ h,
                                                        const float *__restrict__ topk_w,
                                                        const int32_t *__restrict__ ap, Plan p,
                                                        float *__restrict__ o32,
                                                        uint16_t *__restrict__ y)
{
    __shared__ float red[2][2][64][4];
    __shared__ int last;
    const int nrb = H / 16;
    const int u = blockIdx.x / nrb, rb = blockIdx.x - u * nrb;
    const int nT = p.meta[0];
    if (u >= nT) return;
    const int e = p.touched[u], base = p.tbase[u], cnt = p.tcount[u];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
    const int nmt = (cnt + 15) >> 4;
    const float *hr[2];
#pragma unroll
    for (int mt = 0; mt < 2; mt++) hr[mt] = h + (size_t)(base + min(mt * 16 + r, cnt - 1)) * I;
    const int row = rb * 16 + r;
    f32x4 acc[2] = {};
    float ts = 1.f;
    if (FMT == 0) {
        const size_t mb = (size_t)H * I * 2;
        const uint16_t *Wd = reinterpret_cast<const uint16_t *>(expert_base(w.down, e, E, mb)) + (size_t)row * I;
        const int nch = I / 32;
        constexpr int UNR = 6;
        for (int c0 = wave; c0 < nch; c0 += 2 * UNR) {
            u32x4 b[UNR];
#pragma unroll
            for (int i = 0; i < UNR; i++) {
                int c = c0 + 2 * i;
                if (c < nch) b[i] = ld16(Wd + c * 32 + g * 8);
            }
#pragma unroll
            for (int i = 0; i < UNR; i++) {
                int c = c0 + 2 * i;
                if (c < nch) {
#pragma unroll
                    for (int mt = 0; mt < 2; mt++) {
                        if (mt < nmt) {
                            const float *hv = hr[mt] + c * 32 + g * 8;
                            float v[8];
                            *reinterpret_cast<float4 *>(v) = *reinterpret_cast<const float4 *>(hv);
                            *reinterpret_cast<float4 *>(v + 4) = *reinterpret_cast<const float4 *>(hv + 4);
                            u32x4 hi, lo;
                            split_bf16x8(v, hi, lo);
                            acc[mt] = mfma16x16x32(as_bf16x8(hi), as_bf16x8(b[i]), acc[mt]);
                            acc[mt] = mfma16x16x32(as_bf16x8(lo), as_bf16x8(b[i]), acc[mt]);
                        }
                    }
                }
            }
        }
    } else {
        const size_t mb = (size_t)H * I / 2, sb = (size_t)H * I / 16;
        const uint8_t *Qd = expert_base(w.down, e, E, mb) + (size_t)row * (I / 2);
        const uint8_t *Sd = expert_sf(w.down, e, E, sb) + (size_t)row * (I / 16);
        ts = expert_ts(w.down, e, E);
        const int nsc = I / 128;
        for (int sc = wave; sc < nsc; sc += 2) {
            const int kb = sc * 128 + g * 32;
            u32x4 q = ld16(Qd + kb / 2);
            uint32_t sbits = *reinterpret_cast<const uint16_t *>(Sd + kb / 16);
#pragma unroll
            for (int j = 0; j < 4; j++) {
                bf16x8 b = as_bf16x8(dequant8(q[j], e4m3_to_f32((sbits >> (8 * (j >> 1))) & 0xffu)));
#pragma unroll
                for (int mt = 0; mt < 2; mt++) {
                    if (mt < nmt) {
                        const float *hv = hr[mt] + kb + 8 * j;
                        float v[8];
                        *reinterpret_cast<float4 *>(v) = *reinterpret_cast<const float4 *>(hv);
                        *reinterpret_cast<float4 *>(v + 4) = *reinterpret_cast<const float4 *>(hv + 4);
                        u32x4 hi, lo;
                        split_bf16x8(v, hi, lo);
                        acc[mt] = mfma16x16x32(as_bf16x8(hi), b, acc[mt]);
                        acc[mt] = mfma16x16x32(as_bf16x8(lo), b, acc[mt]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++) red[wave][mt][lane][i] = acc[mt][i];
    __syncthreads();
    for (int j = tid; j < nmt * 256; j += 128) {
        const int mt = j >> 8, rem = j & 255, l = rem >> 2, i = rem & 3;
        const float v = (red[0][mt][l][i] + red[1][mt][l][i]) * ts;
        const int m = 4 * (l >> 4) + i, n = l & 15;
        const int ti = mt * 16 + m;
        if (ti < cnt) o32[(size_t)(base + ti) * H + rb * 16 + n] = v;
    }
    // Completion count for this 16-row block of H; the last workgroup combines it.
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        int old = __hip_atomic_fetch_add(&p.counters[rb], 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        last = (old == nT - 1);
    }
    __syncthreads();
    if (!last) return;
    __threadfence();
    const int TK = T * k;
    for (int j = tid; j < T * 16; j += 128) {
        const int t = j >> 4, n = rb * 16 + (j & 15);
        float acc_y = S ? __builtin_nontemporal_load(o32 + (size_t)(TK + t) * H + n) : 0.f;
        for (int jj = 0; jj < k; jj++) {
            const int slot = ap[t * k + jj];
            acc_y += topk_w[t * k + jj] * __builtin_nontemporal_load(o32 + (size_t)slot * H + n);
        }
        y[(size_t)t * H + n] = (uint16_t)f2bf(acc_y);
    }
    if (tid == 0) p.counters[rb] = 0;
}

hipError_t launch_gemv_forward(const Shape &s, const WSet &w, int64_t T, const uint16_t *x,
                               const float *topk_w, const int32_t *sa, const int32_t *ap,
                               const Plan &plan, float *h, float *o32, uint16_t *y,
                               hipStream_t st)
{
    const int maxU = (int)std::min<int64_t>(T * s.k, s.E) + s.S;
    unsigned g1 = (unsigned)(maxU * (s.I / 16)), g2 = (unsigned)(maxU * (s.H / 16));
    if (w.fmt == 0) {
        gemv_gateup_kernel<0><<<g1, 256, 0, st>>>(s.H, s.I, s.E, s.k, w, x, sa, plan, h);
        gemv_down_kernel<0><<<g2, 128, 0, st>>>((int)T, s.H, s.I, s.E, s.k, s.S, w, h, topk_w, ap,
                                                 plan, o32, y);
    } else {
        gemv_gateup_kernel<1><<<g1, 256, 0, st>>>(s.H, s.I, s.E, s.k, w, x, sa, plan, h);
        gemv_down_kernel<1><<<g2, 128, 0, st>>>((int)T, s.H, s.I, s.E, s.k, s.S, w, h, topk_w, ap,
                                                 plan, o32, y);
    }
    return hipGetLastError();
}

}  // namespace flint
