// gemv.hip -- the streaming expert path for small batches (T <= 32 tokens).
//
// Decode reads every touched expert's weights once from HBM; the cost of a step is the
// active weights, not the checkpoint (qantcore.space review, section 01).  Weights stream
// straight from HBM into MFMA B operands with 16-byte loads, all of a wave's loads issued
// before the first MFMA; the expert's tokens (<= 32, one or two 16-row MFMA tiles) form
// the A operand and come from L2.  The shared expert is one more entry of the
// touched-expert list (news.ditty.ir, third paragraph: one shared expert always active).
//
// Pass 1 (gate/up): one workgroup per (touched expert, 8 rows of I).  Its B operand holds
//   8 gate rows in MFMA columns 0-7 and the same 8 up rows in columns 8-15, so one MFMA
//   produces g and u side by side; the 4 waves split K and meet in LDS; h = silu(g) * u is
//   rounded to bf16.  The expert's token rows form the MFMA A operand; lanes whose row is
//   past the expert's token count load nothing (most routed experts of a decode step hold
//   one or two tokens).
// Pass 2 (down + combine): one workgroup per 8 rows of H (H / 8 = 256 workgroups at
//   H = 2048, one per CU), covering every touched expert (one wave per expert at a time,
//   all of its weight and h loads in flight together).  The 8 rows fill MFMA columns 0-7;
//   columns 8-15 stay zero and load nothing.
//   Per-slot outputs stay in LDS in fp32 and the workgroup combines them (shared first,
//   then the k routed slots in order) into bf16 y, so no other workgroup is waited for.
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

// ------------------------------------------------------------------ pass 1: gate / up
template <int FMT, int NMT>
__global__ __launch_bounds__(256) void gemv_gateup_kernel(int T, int H, int I, int E, int k, WSet w,
                                                          const uint16_t *__restrict__ x,
                                                          const int32_t *__restrict__ sa_in,
                                                          Plan p, uint16_t *__restrict__ h)
{
    __shared__ float red[4][NMT][64][4];
    const int nrb = I / 8;
    const int u = blockIdx.x / nrb, rb = blockIdx.x - u * nrb;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
    // The unit's plan entry loads together with the unit count (one round trip), then the
    // token indices of the A rows together with the first weights (one more).
    const int nT = p.meta[0];
    const int e = p.touched[u], base = p.tbase[u], cnt = p.tcount[u];
    if (u >= nT) return;
    int tix[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; mt++) {
        const int idx = min(mt * 16 + r, cnt - 1);
        tix[mt] = (e == E) ? idx * k : sa_in[base + idx];  // assignment index; token = tix / k
    }
    const uint16_t *xr[NMT];
    const int nmt = (cnt + 15) >> 4;
    bool has_tok[NMT];  // this lane's A row is one of the expert's tokens
#pragma unroll
    for (int mt = 0; mt < NMT; mt++) has_tok[mt] = mt * 16 + r < cnt;
    const int i0 = rb * 8;
    const int row = i0 + (r & 7);           // gate row (lanes r < 8) or up row (r >= 8)
    const WMat &wm = (r < 8) ? w.gate : w.up;
    f32x4 acc[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; mt++) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (FMT == 0) {
        const uint16_t *W = reinterpret_cast<const uint16_t *>(expert_base(wm, e, E, (size_t)I * H * 2)) +
                            (size_t)row * H;
        const int cpw = H / 128;              // 32-wide chunks per wave (a contiguous K quarter)
        const int kq = wave * cpw * 32 + g * 8;
        constexpr int NB = 16;
        int c0 = 0;
        u32x4 b[NB];
        if (NB <= cpw)  // the first batch of weights goes out before the token rows resolve
#pragma unroll
            for (int i = 0; i < NB; i++) b[i] = ld16(W + kq + i * 32);
#pragma unroll
        for (int mt = 0; mt < NMT; mt++) xr[mt] = x + (size_t)(tix[mt] / k) * H;
        for (; c0 + NB <= cpw; c0 += NB) {   // full batches: every load issued, no branches
            u32x4 a[NMT][NB];
            if (c0 > 0)
#pragma unroll
                for (int i = 0; i < NB; i++) b[i] = ld16(W + kq + (c0 + i) * 32);
#pragma unroll
            for (int mt = 0; mt < NMT; mt++)
                if (NMT == 1 || mt < nmt)
#pragma unroll
                    for (int i = 0; i < NB; i++) a[mt][i] = has_tok[mt] ? ld16(xr[mt] + kq + (c0 + i) * 32) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < NB; i++)
#pragma unroll
                for (int mt = 0; mt < NMT; mt++)
                    if (NMT == 1 || mt < nmt) acc[mt] = mfma16x16x32(as_bf16x8(a[mt][i]), as_bf16x8(b[i]), acc[mt]);
        }
        for (; c0 < cpw; c0++) {               // tail
            const u32x4 b = ld16(W + kq + c0 * 32);
#pragma unroll
            for (int mt = 0; mt < NMT; mt++)
                if (NMT == 1 || mt < nmt)
                    acc[mt] = mfma16x16x32(as_bf16x8(has_tok[mt] ? ld16(xr[mt] + kq + c0 * 32) : u32x4{0u, 0u, 0u, 0u}), as_bf16x8(b), acc[mt]);
        }
    } else {
        // NVFP4: per 128-wide super-chunk a lane takes 32 consecutive k of its row (16
        // bytes of codes, 2 block scales); MFMA j consumes the lane's k + 8j .. k + 8j + 7.
        const uint8_t *Q = expert_base(wm, e, E, (size_t)I * H / 2) + (size_t)row * (H / 2);
        const uint8_t *SF = expert_sf(wm, e, E, (size_t)I * H / 16) + (size_t)row * (H / 16);
#pragma unroll
        for (int mt = 0; mt < NMT; mt++) xr[mt] = x + (size_t)(tix[mt] / k) * H;
        const int nsc = H / 128;
        constexpr int NB = 4;
        for (int s0 = wave; s0 < nsc; s0 += 4 * NB) {
            u32x4 q[NB], a[NMT][NB][4];
            uint32_t sb[NB];
#pragma unroll
            for (int i = 0; i < NB; i++) {
                const int sc = s0 + 4 * i;
                if (sc < nsc) {
                    const int kb = sc * 128 + g * 32;
                    q[i] = ld16(Q + kb / 2);
                    sb[i] = *reinterpret_cast<const uint16_t *>(SF + kb / 16);
                }
            }
#pragma unroll
            for (int mt = 0; mt < NMT; mt++)
                if (NMT == 1 || mt < nmt)
#pragma unroll
                    for (int i = 0; i < NB; i++) {
                        const int sc = s0 + 4 * i;
                        if (sc < nsc)
#pragma unroll
                            for (int j = 0; j < 4; j++)
                                a[mt][i][j] = has_tok[mt] ? ld16(xr[mt] + sc * 128 + g * 32 + 8 * j) : u32x4{0u, 0u, 0u, 0u};
                    }
#pragma unroll
            for (int i = 0; i < NB; i++) {
                const int sc = s0 + 4 * i;
                if (sc < nsc) {
#pragma unroll
                    for (int j = 0; j < 4; j++) {
                        bf16x8 bv = as_bf16x8(dequant8(q[i][j], e4m3_to_f32((sb[i] >> (8 * (j >> 1))) & 0xffu)));
#pragma unroll
                        for (int mt = 0; mt < NMT; mt++)
                            if (NMT == 1 || mt < nmt) acc[mt] = mfma16x16x32(as_bf16x8(a[mt][i][j]), bv, acc[mt]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int mt = 0; mt < NMT; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++) red[wave][mt][lane][i] = acc[mt][i];
    __syncthreads();
    float tsg = 1.f, tsu = 1.f;
    if (FMT == 1) {
        tsg = expert_ts(w.gate, e, E);
        tsu = expert_ts(w.up, e, E);
    }
    // D[m][n] sits in lane 16 (m / 4) + n, element m % 4; g in columns 0-7, u in 8-15.
    for (int j = tid; j < nmt * 128; j += 256) {
        const int mt = j >> 7, m = (j >> 3) & 15, i = j & 7;
        const int lg = 16 * (m >> 2) + i, el = m & 3;
        float gs = 0.f, us = 0.f;
#pragma unroll
        for (int wv = 0; wv < 4; wv++) {
            gs += red[wv][mt][lg][el];
            us += red[wv][mt][lg + 8][el];
        }
        const int ti = mt * 16 + m;
        if (ti < cnt) h[(size_t)(base + ti) * I + i0 + i] = (uint16_t)f2bf(silu(gs * tsg) * (us * tsu));
    }
}

// ------------------------------------------------------------------ pass 2: down + combine
template <int FMT, int NMT>
__global__ __launch_bounds__(512) void gemv_down_kernel(int T, int H, int I, int E, int k, int S,
                                                        WSet w, const uint16_t *__restrict__ h,
                                                        const float *__restrict__ topk_w,
                                                        const int32_t *__restrict__ ap, Plan p,
                                                        uint16_t *__restrict__ y)
{
    __shared__ float o_lds[kGemvMaxT * 8 + kGemvMaxT][8];
    __shared__ int s_e[257], s_base[257], s_cnt[257], s_nT;
    const int n0 = blockIdx.x * 8;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
    // The plan, once, into LDS: the expert loop below then never waits on global memory
    // before it can issue an expert's weight loads.
    for (int u = tid; u < E + S; u += 512) {
        s_e[u] = p.touched[u];
        s_base[u] = p.tbase[u];
        s_cnt[u] = p.tcount[u];
    }
    if (tid == 0) s_nT = p.meta[0];
    const bool on_row = r < 8;  // MFMA column r holds row n0 + r
    const int row = n0 + (r & 7);
    // The combine inputs of this thread's (token, column), fetched before the weights.
    const int ct = tid >> 3;
    float cw[8];
    int cslot[8];
#pragma unroll
    for (int jj = 0; jj < 8; jj++) {
        const bool on = ct < T && jj < k;
        cw[jj] = on ? topk_w[ct * k + jj] : 0.f;
        cslot[jj] = on ? ap[ct * k + jj] : 0;
    }
    __syncthreads();
    const int nT = s_nT;
    for (int u = wave; u < nT; u += 8) {
        const int e = s_e[u], base = s_base[u], cnt = s_cnt[u];
        const int nmt = (cnt + 15) >> 4;
        const uint16_t *hr[NMT];
        bool has_tok[NMT];  // this lane's A row is one of the expert's tokens
#pragma unroll
        for (int mt = 0; mt < NMT; mt++) {
            hr[mt] = h + (size_t)(base + min(mt * 16 + r, cnt - 1)) * I;
            has_tok[mt] = mt * 16 + r < cnt;
        }
        f32x4 acc[NMT];
#pragma unroll
        for (int mt = 0; mt < NMT; mt++) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        float ts = 1.f;
        if (FMT == 0) {
            const uint16_t *Wd = reinterpret_cast<const uint16_t *>(expert_base(w.down, e, E, (size_t)H * I * 2)) +
                                 (size_t)row * I;
            const int nch = I / 32;
            constexpr int NB = NMT == 1 ? 24 : 12;
            int c0 = 0;
            for (; c0 + NB <= nch; c0 += NB) {   // full batches: every load issued, no branches
                u32x4 b[NB], a[NMT][NB];
#pragma unroll
                for (int i = 0; i < NB; i++) b[i] = on_row ? ld16(Wd + (c0 + i) * 32 + g * 8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int mt = 0; mt < NMT; mt++)
                    if (NMT == 1 || mt < nmt)
#pragma unroll
                        for (int i = 0; i < NB; i++) a[mt][i] = has_tok[mt] ? ld16(hr[mt] + (c0 + i) * 32 + g * 8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int i = 0; i < NB; i++)
#pragma unroll
                    for (int mt = 0; mt < NMT; mt++)
                        if (NMT == 1 || mt < nmt) acc[mt] = mfma16x16x32(as_bf16x8(a[mt][i]), as_bf16x8(b[i]), acc[mt]);
            }
            for (; c0 < nch; c0++) {               // tail
                const u32x4 b = on_row ? ld16(Wd + c0 * 32 + g * 8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int mt = 0; mt < NMT; mt++)
                    if (NMT == 1 || mt < nmt)
                        acc[mt] = mfma16x16x32(as_bf16x8(has_tok[mt] ? ld16(hr[mt] + c0 * 32 + g * 8) : u32x4{0u, 0u, 0u, 0u}), as_bf16x8(b), acc[mt]);
            }
        } else {
            const uint8_t *Qd = expert_base(w.down, e, E, (size_t)H * I / 2) + (size_t)row * (I / 2);
            const uint8_t *Sd = expert_sf(w.down, e, E, (size_t)H * I / 16) + (size_t)row * (I / 16);
            ts = expert_ts(w.down, e, E);
            const int nsc = I / 128;
            constexpr int NB = NMT == 1 ? 6 : 3;
            for (int s0 = 0; s0 < nsc; s0 += NB) {
                u32x4 q[NB], a[NMT][NB][4];
                uint32_t sb[NB];
#pragma unroll
                for (int i = 0; i < NB; i++) {
                    q[i] = u32x4{0u, 0u, 0u, 0u};
                    sb[i] = 0u;
                    if (s0 + i < nsc && on_row) {
                        const int kb = (s0 + i) * 128 + g * 32;
                        q[i] = ld16(Qd + kb / 2);
                        sb[i] = *reinterpret_cast<const uint16_t *>(Sd + kb / 16);
                    }
                }
#pragma unroll
                for (int mt = 0; mt < NMT; mt++)
                    if (NMT == 1 || mt < nmt)
#pragma unroll
                        for (int i = 0; i < NB; i++)
                            if (s0 + i < nsc)
#pragma unroll
                                for (int j = 0; j < 4; j++)
                                    a[mt][i][j] = has_tok[mt] ? ld16(hr[mt] + (s0 + i) * 128 + g * 32 + 8 * j) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                for (int i = 0; i < NB; i++) {
                    if (s0 + i < nsc) {
#pragma unroll
                        for (int j = 0; j < 4; j++) {
                            bf16x8 bv = as_bf16x8(dequant8(q[i][j], e4m3_to_f32((sb[i] >> (8 * (j >> 1))) & 0xffu)));
#pragma unroll
                            for (int mt = 0; mt < NMT; mt++)
                                if (NMT == 1 || mt < nmt) acc[mt] = mfma16x16x32(as_bf16x8(a[mt][i][j]), bv, acc[mt]);
                        }
                    }
                }
            }
        }
        // D[m][n]: lane 16 (m / 4) + n, element m % 4; rows of this lane: m = 4 g + i.
#pragma unroll
        for (int mt = 0; mt < NMT; mt++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int ti = mt * 16 + 4 * g + i;
                if ((NMT == 1 || mt < nmt) && ti < cnt && on_row) o_lds[base + ti][r] = acc[mt][i] * ts;
            }
    }
    __syncthreads();
    if (ct < T) {  // T * 8 <= 512 threads: one (token, column) each
        const int n = tid & 7;
        float acc_y = S ? o_lds[T * k + ct][n] : 0.f;
#pragma unroll
        for (int jj = 0; jj < 8; jj++)
            if (jj < k) acc_y += cw[jj] * o_lds[cslot[jj]][n];
        y[(size_t)ct * H + n0 + n] = (uint16_t)f2bf(acc_y);
    }
}

template <int NMT>
static void launch_pair(const Shape &s, const WSet &w, int64_t T, const uint16_t *x,
                        const float *topk_w, const int32_t *sa, const int32_t *ap,
                        const Plan &plan, uint16_t *h, uint16_t *y, hipStream_t st)
{
    const int maxU = (int)std::min<int64_t>(T * s.k, s.E) + s.S;
    const unsigned g1 = (unsigned)(maxU * (s.I / 8)), g2 = (unsigned)(s.H / 8);
    if (w.fmt == 0) {
        gemv_gateup_kernel<0, NMT><<<g1, 256, 0, st>>>((int)T, s.H, s.I, s.E, s.k, w, x, sa, plan, h);
        gemv_down_kernel<0, NMT><<<g2, 512, 0, st>>>((int)T, s.H, s.I, s.E, s.k, s.S, w, h, topk_w, ap, plan, y);
    } else {
        gemv_gateup_kernel<1, NMT><<<g1, 256, 0, st>>>((int)T, s.H, s.I, s.E, s.k, w, x, sa, plan, h);
        gemv_down_kernel<1, NMT><<<g2, 512, 0, st>>>((int)T, s.H, s.I, s.E, s.k, s.S, w, h, topk_w, ap, plan, y);
    }
}

hipError_t launch_gemv_forward(const Shape &s, const WSet &w, int64_t T, const uint16_t *x,
                               const float *topk_w, const int32_t *sa, const int32_t *ap,
                               const Plan &plan, uint16_t *h, uint16_t *y, hipStream_t st)
{
    if (T <= 16)
        launch_pair<1>(s, w, T, x, topk_w, sa, ap, plan, h, y, st);
    else
        launch_pair<2>(s, w, T, x, topk_w, sa, ap, plan, h, y, st);
    return hipGetLastError();
}

}  // namespace flint
