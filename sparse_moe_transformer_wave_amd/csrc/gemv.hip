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
// Pass 2 (down): one workgroup per (touched expert, 64 rows of H), per-slot outputs in
//   fp32 to the workspace.
// Pass 3 (combine): y = o_shared + the k routed slots in order, summed in fp32, to bf16.
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
// Unit = (touched expert, 8 RG rows of I).  Each wave takes a contiguous quarter of K for
// all RG row groups: the token fragments (A) are loaded once and serve every group, so RG
// multiplies the weight bytes in flight without adding A registers.  `cls` restricts a
// launch to units with at most 16 tokens (1) or more (2); 0 takes every unit.
template <int FMT, int NMT, int RG>
__global__ __launch_bounds__(256) void gemv_gateup_kernel(int T, int H, int I, int E, int k, int cls,
                                                          int dense, WSet w, const uint16_t *__restrict__ x,
                                                          const int32_t *__restrict__ sa_in,
                                                          Plan p, uint16_t *__restrict__ h)
{
    __shared__ float red[4][RG][NMT][64][4];
    const int nrb = I / (8 * RG);
    const int u = blockIdx.x / nrb, rb = blockIdx.x - u * nrb;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
    // The unit's plan entry loads together with the unit count (one round trip), then the
    // token indices of the A rows together with the first weights (one more).
    // a dense layer's plan is implicit: unit u holds tokens 16 u .. 16 u + 15 in the same slots
    const int nT = dense ? (T + 15) / 16 : p.meta[0];
    const int e = dense ? E : p.touched[u], base = dense ? 16 * u : p.tbase[u], cnt = dense ? min(16, T - 16 * u) : p.tcount[u];
    if (u >= nT || (cls == 1 && cnt > 16) || (cls == 2 && cnt <= 16)) return;
    int tix[NMT];
#pragma unroll
    for (int mt = 0; mt < NMT; mt++) {
        const int idx = min(mt * 16 + r, cnt - 1);
        // token of the A row: the shared expert's slot T k + t holds token t (a unit of it
        // may start past T k); routed slots hold assignments t k + j (k >= 1)
        tix[mt] = (e == E) ? base - T * k + idx : sa_in[base + idx] / k;
    }
    const uint16_t *xr[NMT];
    const int nmt = (cnt + 15) >> 4;
    bool has_tok[NMT];  // this lane's A row is one of the expert's tokens
#pragma unroll
    for (int mt = 0; mt < NMT; mt++) has_tok[mt] = mt * 16 + r < cnt;
    const int i0 = rb * 8 * RG;             // first row of I of this unit
    const WMat &wm = (r < 8) ? w.gate : w.up;  // gate row (lanes r < 8) or up row (r >= 8)
    // NVFP4 tensor scales, asked for with the weights so the epilogue does not wait for them
    float tsg = 1.f, tsu = 1.f;
    if (FMT == 1) {
        tsg = expert_ts(w.gate, e, E);
        tsu = expert_ts(w.up, e, E);
    }
    f32x4 acc[RG][NMT];
#pragma unroll
    for (int q = 0; q < RG; q++)
#pragma unroll
        for (int mt = 0; mt < NMT; mt++) acc[q][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (FMT == 0) {
        const uint16_t *W0 = reinterpret_cast<const uint16_t *>(expert_base(wm, e, E, (size_t)I * H * 2)) +
                             (size_t)(i0 + (r & 7)) * H;  // row group q: + 8 q rows
        const int cpw = H / 128;              // 32-wide chunks per wave (a contiguous K quarter)
        const int kq = wave * cpw * 32 + g * 8;
        constexpr int NB = 16;
        int c0 = 0;
        u32x4 b[RG][NB];
        if (NB <= cpw)  // the first batch of weights goes out before the token rows resolve
#pragma unroll
            for (int q = 0; q < RG; q++)
#pragma unroll
                for (int i = 0; i < NB; i++) b[q][i] = ld16(W0 + (size_t)q * 8 * H + kq + i * 32);
#pragma unroll
        for (int mt = 0; mt < NMT; mt++) xr[mt] = x + (size_t)tix[mt] * H;
        for (; c0 + NB <= cpw; c0 += NB) {   // full batches: every load issued, no branches
            u32x4 a[NMT][NB];
            if (c0 > 0)
#pragma unroll
                for (int q = 0; q < RG; q++)
#pragma unroll
                    for (int i = 0; i < NB; i++) b[q][i] = ld16(W0 + (size_t)q * 8 * H + kq + (c0 + i) * 32);
#pragma unroll
            for (int mt = 0; mt < NMT; mt++)
                if (NMT == 1 || mt < nmt)
#pragma unroll
                    for (int i = 0; i < NB; i++) a[mt][i] = has_tok[mt] ? ld16(xr[mt] + kq + (c0 + i) * 32) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < NB; i++)
#pragma unroll
                for (int q = 0; q < RG; q++)
#pragma unroll
                    for (int mt = 0; mt < NMT; mt++)
                        if (NMT == 1 || mt < nmt) acc[q][mt] = mfma16x16x32(as_bf16x8(a[mt][i]), as_bf16x8(b[q][i]), acc[q][mt]);
        }
        for (; c0 < cpw; c0++) {               // tail
            u32x4 a[NMT];
#pragma unroll
            for (int mt = 0; mt < NMT; mt++) a[mt] = has_tok[mt] ? ld16(xr[mt] + kq + c0 * 32) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int q = 0; q < RG; q++) {
                const u32x4 bq = ld16(W0 + (size_t)q * 8 * H + kq + c0 * 32);
#pragma unroll
                for (int mt = 0; mt < NMT; mt++)
                    if (NMT == 1 || mt < nmt) acc[q][mt] = mfma16x16x32(as_bf16x8(a[mt]), as_bf16x8(bq), acc[q][mt]);
            }
        }
    } else {
        // NVFP4 / INT4: per 128-wide super-chunk a lane takes 32 consecutive k of its row
        // (16 bytes of codes; NVFP4: 2 block scales, INT4: the one scale of the 128-column
        // group); MFMA j consumes the lane's k + 8j .. k + 8j + 7.
        const size_t srow = scale_row_bytes(FMT, H);
        const uint8_t *Q0 = expert_base(wm, e, E, (size_t)I * H / 2) + (size_t)(i0 + (r & 7)) * (H / 2);
        const uint8_t *SF0 = expert_sf(wm, e, E, (size_t)I * srow) + (size_t)(i0 + (r & 7)) * srow;
#pragma unroll
        for (int mt = 0; mt < NMT; mt++) xr[mt] = x + (size_t)tix[mt] * H;
        const int nsc = H / 128;
        // one super-chunk per wave and step: a wave holds only that step's codes and token
        // fragments, so more workgroups fit on a CU (4 per step measured 8-10 % slower)
        constexpr int NB = 1;
        for (int s0 = wave; s0 < nsc; s0 += 4 * NB) {
            u32x4 qv[RG][NB], a[NMT][NB][4];
            uint32_t sb[RG][NB];
#pragma unroll
            for (int q = 0; q < RG; q++)
#pragma unroll
                for (int i = 0; i < NB; i++) {
                    const int sc = s0 + 4 * i;
                    if (sc < nsc) {
                        const int kb = sc * 128 + g * 32;
                        qv[q][i] = ld16(Q0 + (size_t)q * 8 * (H / 2) + kb / 2);
                        sb[q][i] = *reinterpret_cast<const uint16_t *>(SF0 + (size_t)q * 8 * srow +
                                                                       (FMT == 1 ? kb / 16 : 2 * sc));
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
                    for (int q = 0; q < RG; q++) {
                        if (FMT == 1) {
#pragma unroll
                            for (int j = 0; j < 4; j++) {
                                bf16x8 bv = as_bf16x8(dequant8(qv[q][i][j], e4m3_to_f32((sb[q][i] >> (8 * (j >> 1))) & 0xffu)));
#pragma unroll
                                for (int mt = 0; mt < NMT; mt++)
                                    if (NMT == 1 || mt < nmt) acc[q][mt] = mfma16x16x32(as_bf16x8(a[mt][i][j]), bv, acc[q][mt]);
                            }
                        } else {
                            // INT4: the super-chunk is one scale group and its 4 MFMAs
                            // contract inside it, so they run on the exact integer codes
                            // and the group scale of the lane's column (its own row)
                            // multiplies their fp32 sum.
                            f32x4 gsum[NMT];
#pragma unroll
                            for (int mt = 0; mt < NMT; mt++) gsum[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int j = 0; j < 4; j++) {
                                bf16x8 bv = as_bf16x8(int4_bf16x8(qv[q][i][j]));
#pragma unroll
                                for (int mt = 0; mt < NMT; mt++)
                                    if (NMT == 1 || mt < nmt) gsum[mt] = mfma16x16x32(as_bf16x8(a[mt][i][j]), bv, gsum[mt]);
                            }
                            const float sv = bf2f(sb[q][i]);
#pragma unroll
                            for (int mt = 0; mt < NMT; mt++)
                                acc[q][mt] = f32x4{acc[q][mt][0] + gsum[mt][0] * sv, acc[q][mt][1] + gsum[mt][1] * sv,
                                                   acc[q][mt][2] + gsum[mt][2] * sv, acc[q][mt][3] + gsum[mt][3] * sv};
                        }
                    }
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < RG; q++)
#pragma unroll
        for (int mt = 0; mt < NMT; mt++)
#pragma unroll
            for (int i = 0; i < 4; i++) red[wave][q][mt][lane][i] = acc[q][mt][i];
    __syncthreads();
    // D[m][n] sits in lane 16 (m / 4) + n, element m % 4; g in columns 0-7, u in 8-15.
    for (int j = tid; j < RG * nmt * 128; j += 256) {
        const int q = j / (nmt * 128), jj = j - q * nmt * 128;
        const int mt = jj >> 7, m = (jj >> 3) & 15, i = jj & 7;
        const int lg = 16 * (m >> 2) + i, el = m & 3;
        float gs = 0.f, us = 0.f;
#pragma unroll
        for (int wv = 0; wv < 4; wv++) {
            gs += red[wv][q][mt][lg][el];
            us += red[wv][q][mt][lg + 8][el];
        }
        const int ti = mt * 16 + m;
        if (ti < cnt) h[(size_t)(base + ti) * I + i0 + 8 * q + i] = (uint16_t)f2bf(silu(gs * tsg) * (us * tsu));
    }
}

// ------------------------------------------------------------------ pass 2: down
// KS = 1: one workgroup per (touched expert, 64 rows of H): wave w multiplies rows 64 nb +
// 16 w ... + 15 (MFMA columns) over all of K = I against the expert's h rows, every load of
// a batch in flight.  KS = 4 (few experts, e.g. a dense layer): one workgroup per (expert,
// RW rows), wave w takes the w-th quarter of K and the quarters are summed through LDS, so
// four times as many waves stream the same rows; RW = 8 (MFMA columns 8-15 repeat 0-7 and
// are not stored) when 16-row workgroups would leave CUs without work.  Per-slot outputs o[slot][n] go to the
// workspace in fp32.  `cls` as for gate/up.  Thousands of small independent workgroups
// keep the weight stream busy the way the gate/up pass does.
template <int FMT, int NMT, int KS, int RW = 16>
__global__ __launch_bounds__(256) void gemv_down_kernel(int H, int I, int E, int cls, int dense_T, WSet w,
                                                        const uint16_t *__restrict__ h, Plan p,
                                                        float *__restrict__ o, uint16_t *__restrict__ y)
{
    static_assert(KS == 1 || KS == 4, "K split over the 4 waves or none");
    static_assert(RW == 16 || RW == 8, "16 or 8 rows per workgroup");
    __shared__ f32x4 red[KS == 4 ? 3 : 1][NMT][64];
    const int nrb = KS == 1 ? H / 64 : H / RW;
    const int u = blockIdx.x / nrb, nb = blockIdx.x - u * nrb;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
    // dense_T > 0: a dense layer of dense_T tokens, unit u = tokens 16 u .. 16 u + 15, outputs y
    const int nT = dense_T ? (dense_T + 15) / 16 : p.meta[0];
    const int e = dense_T ? E : p.touched[u], base = dense_T ? 16 * u : p.tbase[u], cnt = dense_T ? min(16, dense_T - 16 * u) : p.tcount[u];
    if (u >= nT || (cls == 1 && cnt > 16) || (cls == 2 && cnt <= 16)) return;
    const int row = KS == 1 ? nb * 64 + wave * 16 + r : nb * RW + (r % RW);  // MFMA column r of this wave
    const int kw = KS == 1 ? 0 : wave;  // this wave's part of K
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
        const int nch = I / 32, ce = nch * (kw + 1) / KS;
        // KS = 4: 16 (8) chunks per batch, so a dense layer's long rows take two round
        // trips per wave instead of six
        constexpr int NB = KS == 1 ? (NMT == 1 ? 24 : 12) : (NMT == 1 ? 16 : 8);
        int c0 = nch * kw / KS;
        for (; c0 + NB <= ce; c0 += NB) {   // full batches: every load issued, no branches
            u32x4 b[NB], a[NMT][NB];
#pragma unroll
            for (int i = 0; i < NB; i++) b[i] = ld16(Wd + (c0 + i) * 32 + g * 8);
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
        if (c0 < ce) {                         // the last, partial batch: its loads in flight together
            u32x4 b[NB], a[NMT][NB];
#pragma unroll
            for (int i = 0; i < NB; i++) b[i] = c0 + i < ce ? ld16(Wd + (c0 + i) * 32 + g * 8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int mt = 0; mt < NMT; mt++)
#pragma unroll
                for (int i = 0; i < NB; i++)
                    a[mt][i] = (NMT == 1 || mt < nmt) && c0 + i < ce && has_tok[mt] ? ld16(hr[mt] + (c0 + i) * 32 + g * 8)
                                                                                  : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < NB; i++)
                if (c0 + i < ce)
#pragma unroll
                    for (int mt = 0; mt < NMT; mt++)
                        if (NMT == 1 || mt < nmt) acc[mt] = mfma16x16x32(as_bf16x8(a[mt][i]), as_bf16x8(b[i]), acc[mt]);
        }
    } else {
        const size_t srow = scale_row_bytes(FMT, I);
        const uint8_t *Qd = expert_base(w.down, e, E, (size_t)H * I / 2) + (size_t)row * (I / 2);
        const uint8_t *Sd = expert_sf(w.down, e, E, (size_t)H * srow) + (size_t)row * srow;
        if (FMT == 1) ts = expert_ts(w.down, e, E);
        const int nsc = I / 128, se = nsc * (kw + 1) / KS;
        // split-K workgroups take one super-chunk per step (two measured 0.4-2.4 % slower)
        constexpr int NB = KS == 1 ? (NMT == 1 ? 6 : 3) : 1;
        for (int s0 = nsc * kw / KS; s0 < se; s0 += NB) {
            u32x4 q[NB], a[NMT][NB][4];
            uint32_t sb[NB];
#pragma unroll
            for (int i = 0; i < NB; i++) {
                q[i] = u32x4{0u, 0u, 0u, 0u};
                sb[i] = 0u;
                if (s0 + i < se) {
                    const int kb = (s0 + i) * 128 + g * 32;
                    q[i] = ld16(Qd + kb / 2);
                    sb[i] = *reinterpret_cast<const uint16_t *>(Sd + (FMT == 1 ? kb / 16 : 2 * (s0 + i)));
                }
            }
#pragma unroll
            for (int mt = 0; mt < NMT; mt++)
                if (NMT == 1 || mt < nmt)
#pragma unroll
                    for (int i = 0; i < NB; i++)
                        if (s0 + i < se)
#pragma unroll
                            for (int j = 0; j < 4; j++)
                                a[mt][i][j] = has_tok[mt] ? ld16(hr[mt] + (s0 + i) * 128 + g * 32 + 8 * j) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int i = 0; i < NB; i++) {
                if (s0 + i < se) {
                    if (FMT == 1) {
#pragma unroll
                        for (int j = 0; j < 4; j++) {
                            bf16x8 bv = as_bf16x8(dequant8(q[i][j], e4m3_to_f32((sb[i] >> (8 * (j >> 1))) & 0xffu)));
#pragma unroll
                            for (int mt = 0; mt < NMT; mt++)
                                if (NMT == 1 || mt < nmt) acc[mt] = mfma16x16x32(as_bf16x8(a[mt][i][j]), bv, acc[mt]);
                        }
                    } else {  // INT4: integer codes per scale group, then the row's group scale
                        f32x4 gsum[NMT];
#pragma unroll
                        for (int mt = 0; mt < NMT; mt++) gsum[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int j = 0; j < 4; j++) {
                            bf16x8 bv = as_bf16x8(int4_bf16x8(q[i][j]));
#pragma unroll
                            for (int mt = 0; mt < NMT; mt++)
                                if (NMT == 1 || mt < nmt) gsum[mt] = mfma16x16x32(as_bf16x8(a[mt][i][j]), bv, gsum[mt]);
                        }
                        const float sv = bf2f(sb[i]);
#pragma unroll
                        for (int mt = 0; mt < NMT; mt++)
                            acc[mt] = f32x4{acc[mt][0] + gsum[mt][0] * sv, acc[mt][1] + gsum[mt][1] * sv,
                                            acc[mt][2] + gsum[mt][2] * sv, acc[mt][3] + gsum[mt][3] * sv};
                    }
                }
            }
        }
    }
    if (KS == 4) {  // waves 1..3 hand their partial sums to wave 0 (K order: wave 0 first)
        if (wave > 0)
#pragma unroll
            for (int mt = 0; mt < NMT; mt++) red[KS == 4 ? wave - 1 : 0][mt][lane] = acc[mt];
        __syncthreads();
        if (wave > 0) return;
#pragma unroll
        for (int q = 0; q < 3; q++)
#pragma unroll
            for (int mt = 0; mt < NMT; mt++) {
                const f32x4 v = red[KS == 4 ? q : 0][mt][lane];
                acc[mt] = f32x4{acc[mt][0] + v[0], acc[mt][1] + v[1], acc[mt][2] + v[2], acc[mt][3] + v[3]};
            }
    }
    // D[m][n]: lane 16 (m / 4) + n, element m % 4; rows (slots) of this lane: m = 4 g + i.
#pragma unroll
    for (int mt = 0; mt < NMT; mt++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int ti = mt * 16 + 4 * g + i;
            if ((NMT == 1 || mt < nmt) && ti < cnt && (KS == 1 || r < RW)) {
                if (dense_T)  // the combine of a dense layer is y = bf16(o): written here
                    y[(size_t)(base + ti) * H + row] = (uint16_t)f2bf(acc[mt][i] * ts);
                else
                    o[(size_t)(base + ti) * H + row] = acc[mt][i] * ts;
            }
        }
}

// ------------------------------------------------------------------ pass 3: combine
// y[t][n] = bf16(o[T*k + t][n] + sum_j w[t][j] * o[ap[t*k + j]][n]), summed in fp32 in that
// order (shared first, then j ascending); 8 columns per thread.  Slots outside [0, T k)
// (assignments dropped for an out-of-range expert id) are skipped.
__global__ __launch_bounds__(256) void gemv_combine_kernel(int T, int H, int k, int S,
                                                           const float *__restrict__ o,
                                                           const float *__restrict__ topk_w,
                                                           const int32_t *__restrict__ ap,
                                                           uint16_t *__restrict__ y)
{
    const int per_tok = H / 8;
    const int gid = blockIdx.x * 256 + threadIdx.x;
    if (gid >= T * per_tok) return;
    const int t = gid / per_tok, c = (gid - t * per_tok) * 8;
    float wj[8];
    int sl[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
        wj[j] = j < k ? topk_w[t * k + j] : 0.f;
        sl[j] = j < k ? ap[t * k + j] : -1;
    }
    float acc[8];
    if (S) {
        const f32x4 a0 = *reinterpret_cast<const f32x4 *>(o + ((size_t)T * k + t) * H + c);
        const f32x4 a1 = *reinterpret_cast<const f32x4 *>(o + ((size_t)T * k + t) * H + c + 4);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            acc[i] = a0[i];
            acc[4 + i] = a1[i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; i++) acc[i] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; j++) {
        if (sl[j] >= 0 && sl[j] < T * k) {  // a dropped assignment (expert id out of range) has no slot
            const f32x4 a0 = *reinterpret_cast<const f32x4 *>(o + (size_t)sl[j] * H + c);
            const f32x4 a1 = *reinterpret_cast<const f32x4 *>(o + (size_t)sl[j] * H + c + 4);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                acc[i] += wj[j] * a0[i];
                acc[4 + i] += wj[j] * a1[i];
            }
        }
    }
    u32x4 outv;
#pragma unroll
    for (int i = 0; i < 4; i++) outv[i] = f2bf(acc[2 * i]) | (f2bf(acc[2 * i + 1]) << 16);
    *reinterpret_cast<u32x4 *>(y + (size_t)t * H + c) = outv;
}

// Gate/up, row groups per wave: 2 with one token tile, else 1; 4-bit weights with more than
// 16 tokens take 4.  (With 4-bit weights taken one super-chunk per step a wave needs few
// registers: a second NVFP4 group measured 3-5 % faster; four groups measured slower at
// T = 8 and 2-3 % faster at T = 32.)
template <int FMT, int NMT>
static void launch_gateup(const Shape &s, const WSet &w, int64_t T, int maxU, int cls, const uint16_t *x,
                          const int32_t *sa, const Plan &plan, uint16_t *h, hipStream_t st)
{
    constexpr int RG = NMT == 1 ? 2 : 1;
    if (FMT != 0 && NMT == 1 && T > 16) {  // 4-bit, fuller units: four row groups
        const unsigned grid4 = (unsigned)(maxU * (s.I / 32));
        gemv_gateup_kernel<FMT, NMT, 4><<<grid4, 256, 0, st>>>((int)T, s.H, s.I, s.E, s.k, cls, s.E == 0, w, x, sa,
                                                             plan, h);
        return;
    }
    const unsigned grid = (unsigned)(maxU * (s.I / (8 * RG)));
    gemv_gateup_kernel<FMT, NMT, RG><<<grid, 256, 0, st>>>((int)T, s.H, s.I, s.E, s.k, cls, s.E == 0, w, x, sa,
                                                         plan, h);
}

// Split K over the waves when 64-row workgroups would leave most CUs idle, and always for
// 4-bit weights (their short rows make a 64-row workgroup mostly wait: 16-row workgroups
// measured 2-3 % faster per NVFP4 layer at T = 8 and 32), and take 8 rows per workgroup when
// 16-row ones would still number fewer than the CUs.
template <int FMT, int NMT>
static void launch_down(const Shape &s, const WSet &w, int64_t T, int maxU, int cls, const uint16_t *h,
                        const Plan &plan, float *o, uint16_t *y, hipStream_t st)
{
    const int dense_T = s.E == 0 ? (int)T : 0;
    if (FMT == 0 && maxU * (s.H / 64) >= 512)
        gemv_down_kernel<FMT, NMT, 1><<<(unsigned)(maxU * (s.H / 64)), 256, 0, st>>>(s.H, s.I, s.E, cls, dense_T, w, h,
                                                                                  plan, o, y);
    else if (maxU * (s.H / 16) >= 256)
        gemv_down_kernel<FMT, NMT, 4><<<(unsigned)(maxU * (s.H / 16)), 256, 0, st>>>(s.H, s.I, s.E, cls, dense_T, w, h,
                                                                                  plan, o, y);
    else
        gemv_down_kernel<FMT, NMT, 4, 8><<<(unsigned)(maxU * (s.H / 8)), 256, 0, st>>>(s.H, s.I, s.E, cls, dense_T, w,
                                                                                    h, plan, o, y);
}

// With routed experts the plan lists units of at most 16 tokens (an expert with more is
// split; in practice the shared expert once T > 16), so one launch of the one-tile
// kernels covers every unit.  A dense layer (E = 0) is split the same way, so for T > 16
// its weights are read once per unit; one unit of two token tiles measured slower (its
// workgroups read twice the activations with twice the registers).  Its plan is implicit
// (no plan launch) and its down pass writes y (no combine launch).
template <int FMT>
static void launch_stream(const Shape &s, const WSet &w, int64_t T, const uint16_t *x,
                          const float *topk_w, const int32_t *sa, const int32_t *ap,
                          const Plan &plan, uint16_t *h, float *o, uint16_t *y, hipStream_t st)
{
    const int maxU = (int)(std::min<int64_t>(T * s.k, s.E) + (T * s.k + kUnitRows - 1) / kUnitRows +
                           (int64_t)s.S * ((T + kUnitRows - 1) / kUnitRows));
    launch_gateup<FMT, 1>(s, w, T, maxU, 0, x, sa, plan, h, st);
    launch_down<FMT, 1>(s, w, T, maxU, 0, h, plan, o, y, st);
    if (s.E == 0) return;
    const int nthreads = (int)T * (s.H / 8);
    gemv_combine_kernel<<<(unsigned)((nthreads + 255) / 256), 256, 0, st>>>((int)T, s.H, s.k, s.S, o, topk_w, ap, y);
}

hipError_t launch_gemv_forward(const Shape &s, const WSet &w, int64_t T, const uint16_t *x,
                               const float *topk_w, const int32_t *sa, const int32_t *ap,
                               const Plan &plan, uint16_t *h, float *o, uint16_t *y, hipStream_t st)
{
    if (w.fmt == 0)
        launch_stream<0>(s, w, T, x, topk_w, sa, ap, plan, h, o, y, st);
    else if (w.fmt == 1)
        launch_stream<1>(s, w, T, x, topk_w, sa, ap, plan, h, o, y, st);
    else
        launch_stream<2>(s, w, T, x, topk_w, sa, ap, plan, h, o, y, st);
    return hipGetLastError();
}

}  // namespace flint
