// decode_few.hip -- a small decode batch (2 <= T <= 16 tokens): the whole MoE layer in one
// persistent launch.
//
// The pages' GB200 runtime keeps a low-latency decode path for batches of up to 8 requests
// (recipes.vllm.ai "RecursiveSI/flint", Overview), and decode reads only the touched
// experts' weights (qantcore.space review, section 01).  As separate launches (router and
// selection, gate/up, down, combine) a batch of 8 pays each launch's ramp and drain and a
// single-workgroup selection between them; here one launch of one workgroup per CU (8
// waves) runs the layer, its workgroups trading data through tagged words (xchg.h):
//
//   route    workgroup b < E: logit b of every token (router row b in fp32), published as
//            words; every workgroup waits for all T E of them.
//   select   wave w selects for tokens w and w + 8 (one token per wave, as in the
//            small-batch router launch).  Every workgroup then builds the same plan in LDS:
//            the units (the shared expert, then the touched experts in ascending order),
//            each unit's tokens and their slots -- routed slots grouped by expert with the
//            assignments ascending, shared slots T k + t: the routing tensors of the other
//            paths.
//   gate/up  the units' (gate row i, up row i) pairs in blocks of 8, each block one MFMA
//            tile: B = its 8 gate rows (columns 0-7) and the same 8 up rows (columns 8-15),
//            A = all T tokens, whichever unit the block belongs to.  The tokens are the same
//            for every expert (a token's rows for an expert it did not pick are computed and
//            not stored), so the token fragments are loaded once per wave and the blocks of
//            all units form one even list, dealt out round-robin (workgroup b takes blocks
//            b, b + 256, ...).
//            Seven waves split K; their partial tiles meet in LDS, where the eighth wave
//            forms h = silu(g) u of the unit's tokens, rounded to bf16, and writes it out as
//            words of two values.  (The streaming waves issue no stores: a wave's memory
//            operations complete in order, so a write-through store would delay the wait
//            for the next weight load by the store's round trip, once per block.)
//   down     the units' 16-row blocks of H in contiguous ranges (workgroup b takes blocks
//            [b n / 256, (b+1) n / 256), mostly of one unit).  A = the unit's h rows
//            (polled; with the gate/up blocks dealt round-robin a unit's h is written by
//            many workgroups, most units' long before the down phase), B = 16 down rows;
//            the eighth wave writes the per-slot outputs as fp32 words.
//   combine  workgroup b owns elements [b T H / 256, (b+1) T H / 256) of y: it polls the
//            k + 1 slot words of each and sums them in fp32, shared first, then j
//            ascending (news.ditty.ir, third paragraph: one shared expert always active).
//
// Weights stream straight from HBM into MFMA B operands, several blocks in flight per
// wave.  A wait depends only on an earlier phase of other workgroups (gate/up on the
// logits, down on gate/up, combine on down), so with every workgroup resident (checked by
// the host) the launch completes; every wait is bounded in any case and a timeout is
// reported through the workspace head's error flags.
#include "xchg.h"

namespace flint {

namespace {

constexpr int kFG = kPersistentGrid;  // workgroups
constexpr int kFWaves = 8, kFComp = kFWaves - 1;  // waves; those that stream weights
constexpr int kFMaxT = 16, kFMaxK = 8, kFMaxE = 256, kFMaxH = 2048, kFMaxI = 1024;
constexpr int kFMaxSlots = kFMaxT * (kFMaxK + 1);
constexpr int kFMaxU = 1 + kFMaxT * kFMaxK;  // the shared expert and up to T k touched experts

// Exchange words in the workspace head, from kHeadFewXchg: logits [T][E], h [slots][I / 2]
// (word q of a slot: bf16 h[2q] low, h[2q + 1] high), per-slot outputs [slots][H] (fp32);
// then a chain's two token buffers, bf16 [T][H] each: layer l of a chain reads buffer l % 2
// and writes the next layer's tokens to the other (a workgroup that owns no logit may still
// be reading its tokens while others already write the next ones).
constexpr size_t kFLogOff = kHeadFewXchg;
constexpr size_t kFHOff = kFLogOff + 8 * (size_t)kFMaxT * kFMaxE;
constexpr size_t kFOOff = kFHOff + 8 * (size_t)kFMaxSlots * (kFMaxI / 2);
constexpr size_t kFXOff = kFOOff + 8 * (size_t)kFMaxSlots * kFMaxH;
constexpr size_t kFEnd = kFXOff + 2 * 2 * (size_t)kFMaxT * kFMaxH;
static_assert(kFEnd <= kSyncBytes, "small-batch exchange words exceed the head");
static_assert(kFG == 256 && kFMaxE <= kFG, "workgroup b computes logit b");

struct FArgs {
    int T, H, I, E, k, S, renorm;
    WSet w;
    const uint16_t *x;
    const float *Wr, *bias;
    uint16_t *y;
    uint16_t *xnext;  // null, or receives the next layer's tokens: y, or bf16(x + y) with `residual`
    int residual;
    float *logits;
    int32_t *ids;
    float *tw;
    int32_t *counts, *offsets, *sa, *ap;
    uint8_t *head;
    uint64_t *xlog, *xh, *xo;
};

struct FShared {
    f32x4 red[2][kFWaves][64];       // the waves' partial MFMA tiles, two blocks in turn
    float lg[kFMaxT * kFMaxE];       // logits [t][e]
    int32_t ids[kFMaxT * kFMaxK];
    float wt[kFMaxT * kFMaxK];
    int32_t pos[kFMaxT * kFMaxK];    // slot of assignment a
    int32_t cnt_e[kFMaxE], below_e[kFMaxE], unit_e[kFMaxE];
    uint32_t tmask[kFMaxE];          // tokens that picked expert e (bit t)
    int32_t u_e[kFMaxU], u_cnt[kFMaxU];
    int16_t u_slot[kFMaxU][kFMaxT];  // slot of the unit's m-th token, m < u_cnt
    int16_t u_tslot[kFMaxU][kFMaxT]; // slot of token t in the unit, -1 when t is not in it
    float u_ts[3][kFMaxU];           // NVFP4 tensor scales of gate, up, down
    int32_t wtouch[4], wsum[4];
    int32_t nunits;
    uint32_t tag, giveup;
};

__device__ __forceinline__ u32x4 ldg16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

__device__ __forceinline__ const uint8_t *wbase(const WMat &m, int e, int E, size_t bytes)
{
    return e == E ? m.shared : m.routed + (size_t)e * bytes;
}
__device__ __forceinline__ const uint8_t *wsf(const WMat &m, int e, int E, size_t bytes)
{
    return e == E ? m.sf_shared : m.sf_routed + (size_t)e * bytes;
}
__device__ __forceinline__ float wts(const WMat &m, int e, int E)
{
    return e == E ? *m.ts_shared : m.ts_routed[e];
}

// A workgroup barrier that waits for this wave's LDS accesses only: the weight loads in
// flight stay in flight.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt untouched
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// One MFMA tile's K part against B fragments: bf16 chunks of 32 columns, or 4-bit
// super-chunks of 128 (a lane's 32 codes of its row, MFMA j taking columns 8 j .. 8 j + 7 of
// the lane's 32, with the block scales (NVFP4) or the group scale (INT4) in sc).
template <int FMT, int NC>
__device__ __forceinline__ f32x4 tile_mma(const u32x4 *a, const u32x4 *v, const uint32_t *sc, int nc)
{
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; c++) {
        if (c < nc) {
            if (FMT == 0) {
                acc = mfma16x16x32(as_bf16x8(a[c]), as_bf16x8(v[c]), acc);
            } else if (FMT == 1) {
                const u32x4 q = v[c];
                const uint32_t q0 = q[0], q1 = q[1], q2 = q[2], q3 = q[3];
                const float s0 = e4m3_to_f32(sc[c] & 0xffu), s1 = e4m3_to_f32((sc[c] >> 8) & 0xffu);
                acc = mfma16x16x32(as_bf16x8(a[4 * c]), as_bf16x8(dequant8_stream(q0, s0)), acc);
                acc = mfma16x16x32(as_bf16x8(a[4 * c + 1]), as_bf16x8(dequant8_stream(q1, s0)), acc);
                acc = mfma16x16x32(as_bf16x8(a[4 * c + 2]), as_bf16x8(dequant8_stream(q2, s1)), acc);
                acc = mfma16x16x32(as_bf16x8(a[4 * c + 3]), as_bf16x8(dequant8_stream(q3, s1)), acc);
            } else {  // INT4: exact integer codes within the group, then its scale
                const u32x4 q = v[c];
                const uint32_t q0 = q[0], q1 = q[1], q2 = q[2], q3 = q[3];
                f32x4 gs = f32x4{0.f, 0.f, 0.f, 0.f};
                gs = mfma16x16x32(as_bf16x8(a[4 * c]), as_bf16x8(int4_bf16x8(q0)), gs);
                gs = mfma16x16x32(as_bf16x8(a[4 * c + 1]), as_bf16x8(int4_bf16x8(q1)), gs);
                gs = mfma16x16x32(as_bf16x8(a[4 * c + 2]), as_bf16x8(int4_bf16x8(q2)), gs);
                gs = mfma16x16x32(as_bf16x8(a[4 * c + 3]), as_bf16x8(int4_bf16x8(q3)), gs);
                const float sv = bf2f(sc[c] & 0xffffu);
                acc = f32x4{acc[0] + gs[0] * sv, acc[1] + gs[1] * sv, acc[2] + gs[2] * sv, acc[3] + gs[3] * sv};
            }
        }
    }
    return acc;
}

template <int FMT>
__global__ __launch_bounds__(512) void decode_few_kernel(FArgs a)
{
    __shared__ FShared sh;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
    const int b = blockIdx.x;
    const int T = a.T, H = a.H, I = a.I, E = a.E, k = a.k, S = a.S, TK = T * k;
    // bf16 moves in 16-byte chunks of 32 columns, 4-bit weights in super-chunks of 128; a
    // streaming wave's part of K: at most NCG chunks of a gate/up row (H <= kFMaxH), NCD of a
    // down row (I <= kFMaxI)
    constexpr int NCG = FMT == 0 ? (kFMaxH / 32 + kFComp - 1) / kFComp : (kFMaxH / 128 + kFComp - 1) / kFComp;
    constexpr int NCD = FMT == 0 ? (kFMaxI / 32 + kFComp - 1) / kFComp : (kFMaxI / 128 + kFComp - 1) / kFComp;
    constexpr int NAG = FMT == 0 ? NCG : 4 * NCG, NAD = FMT == 0 ? NCD : 4 * NCD;
    constexpr int GD = FMT == 0 ? 3 : 6;   // gate/up blocks in flight
    constexpr int DD = FMT == 0 ? 3 : 6;   // down blocks in flight
    const bool comp = wave < kFComp;

    uint32_t launches = 0;
    if (tid == 0) {
        launches = read_launches(a.head);
        sh.tag = launch_tag(launches);
        sh.giveup = diag_word(a.head);
    }

    // ---------------- route
    // The token fragments of the gate/up tiles (rows = tokens, this wave's part of K) go
    // out first; they are used only after the plan.
    const int nkg = FMT == 0 ? H / 32 : (H + 127) / 128;
    const int kg0 = comp ? nkg * wave / kFComp : 0, ng = comp ? nkg * (wave + 1) / kFComp - kg0 : 0;
    u32x4 ax[NAG];
    {
        const bool tok = r < T;
        const uint16_t *xr = a.x + (size_t)(tok ? r : 0) * H;
#pragma unroll
        for (int c = 0; c < NCG; c++) {
            if (FMT == 0) {
                ax[c] = tok && c < ng ? ldg16(xr + (kg0 + c) * 32 + g * 8) : u32x4{0u, 0u, 0u, 0u};
            } else {
                const int kb = (kg0 + c) * 128 + g * 32;
                const bool in = tok && c < ng && kb < H;
#pragma unroll
                for (int j = 0; j < 4; j++) ax[4 * c + j] = in ? ldg16(xr + kb + 8 * j) : u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
    float lv[2] = {0.f, 0.f};
    if (b < E) router_dot_wave<2>(T, H, b, wave, kFWaves, a.x, a.Wr, lv);
    __syncthreads();
    const uint32_t tag = sh.tag;
    const bool giveup = sh.giveup != 0;
    if (b < E && lane == 0) {
        const float bias = a.bias ? a.bias[b] : 0.f;
#pragma unroll
        for (int q = 0; q < 2; q++) {
            const int t = wave + kFWaves * q;
            if (t < T) {
                const float l = lv[q] + bias;
                if (a.logits) a.logits[(size_t)t * E + b] = l;
                put_word(a.xlog + (size_t)t * E + b, tag, l);
            }
        }
    }
    {
        const int nl = T * E, nq = tid < nl ? (nl - tid + 511) / 512 : 0;
        uint64_t lw[8];
#pragma unroll
        for (int q = 0; q < 8; q++) lw[q] = q < nq ? get_word(a.xlog + tid + 512 * q) : 0ull;
        await_words<8>(a.xlog + tid, 512, nq, lw, tag, a.head, giveup);
#pragma unroll
        for (int q = 0; q < 8; q++)
            if (q < nq) sh.lg[tid + 512 * q] = __uint_as_float((uint32_t)lw[q]);
    }
    for (int i = tid; i < kFMaxU * kFMaxT; i += 512) (&sh.u_tslot[0][0])[i] = -1;
    if (tid < kFMaxE) {
        sh.cnt_e[tid] = 0;
        sh.tmask[tid] = 0u;
    }
    __syncthreads();

    // ---------------- select, plan
    // Each selecting wave also counts its token's experts and marks the token in each
    // expert's token mask (LDS atomics: the results do not depend on their order).
    for (int t = wave; t < T; t += kFWaves) {
        topk_wave(sh.lg + t * E, E, k, a.renorm, sh.ids + t * k, sh.wt + t * k);
        if (lane < k) {
            const int e = sh.ids[t * k + lane];
            atomicAdd(&sh.cnt_e[e], 1);
            atomicOr(&sh.tmask[e], 1u << t);
        }
    }
    __syncthreads();
    // Expert e = tid: the assignments below it (a scan of the counts over the experts, in
    // waves of 64 and then across the 4 waves) and its unit (S + its rank among the touched).
    int cnt = 0, incl = 0, trank = 0;
    if (tid < kFMaxE) {
        cnt = sh.cnt_e[tid];
        incl = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int n = __shfl_up(incl, d);
            if (lane >= d) incl += n;
        }
        const uint64_t bal = __ballot(cnt > 0);
        trank = __popcll(bal & ((1ull << lane) - 1ull));
        if (lane == 63) {
            sh.wsum[wave] = incl;
            sh.wtouch[wave] = __popcll(bal);
        }
    }
    __syncthreads();
    if (tid < kFMaxE) {
        const int e = tid;
        int below = incl - cnt, u = S + trank;
        for (int w2 = 0; w2 < wave; w2++) {
            below += sh.wsum[w2];
            u += sh.wtouch[w2];
        }
        sh.below_e[e] = below;
        if (cnt > 0) {
            sh.unit_e[e] = u;
            sh.u_e[u] = e;
            sh.u_cnt[u] = cnt;
            if (FMT == 1) {
                sh.u_ts[0][u] = a.w.gate.ts_routed[e];
                sh.u_ts[1][u] = a.w.up.ts_routed[e];
                sh.u_ts[2][u] = a.w.down.ts_routed[e];
            }
        }
    } else if (tid == 256) {
        sh.nunits = S + sh.wtouch[0] + sh.wtouch[1] + sh.wtouch[2] + sh.wtouch[3];
        if (S) {
            sh.u_e[0] = E;
            sh.u_cnt[0] = T;
            if (FMT == 1) {
                sh.u_ts[0][0] = *a.w.gate.ts_shared;
                sh.u_ts[1][0] = *a.w.up.ts_shared;
                sh.u_ts[2][0] = *a.w.down.ts_shared;
            }
        }
    }
    __syncthreads();
    if (tid < TK) {  // assignment tid = t k + j: its rank among the expert's tokens gives its slot
        const int e = sh.ids[tid], u = sh.unit_e[e], t = tid / k;
        const int rank = __popc(sh.tmask[e] & ((1u << t) - 1u)), p = sh.below_e[e] + rank;
        sh.pos[tid] = p;
        sh.u_slot[u][rank] = (int16_t)p;
        sh.u_tslot[u][t] = (int16_t)p;
        if (b == 0) {  // the routing tensors (workgroup 0)
            a.ids[tid] = e;
            a.tw[tid] = sh.wt[tid];
            if (a.sa) {
                a.sa[p] = tid;
                a.ap[tid] = p;
            }
        }
    } else if (tid >= 256 && tid - 256 < T && S) {
        const int t = tid - 256;
        sh.u_slot[0][t] = (int16_t)(TK + t);
        sh.u_tslot[0][t] = (int16_t)(TK + t);
    }
    if (b == 0 && a.counts) {
        if (tid >= 256 && tid - 256 < E) {
            a.counts[tid - 256] = sh.cnt_e[tid - 256];
            a.offsets[tid - 256] = sh.below_e[tid - 256];
        }
        if (tid == 255) a.offsets[E] = TK;
    }
    __syncthreads();
    const int nunits = sh.nunits;
    int par = 0;  // which half of red the next block uses: blocks alternate across both phases

    // ---------------- gate / up
    // Waves 0 .. kFComp - 1 stream the weights and multiply; the last wave sums their partial
    // tiles and writes the exchange words.  The streaming waves issue no stores: a wave's
    // memory operations complete in order, so a write-through store ahead of a weight load
    // would hold up the wait for that load by the store's round trip, every block.
    {
        // Workgroup b takes blocks b, b + 256, b + 512, ...: the units' blocks are dealt out in
        // unit order, so most units' h is complete long before the down phase needs it
        // (contiguous ranges had every unit finish with its workgroups' last blocks).
        const int bpu = I / 8, nbk = nunits * bpu;
        const int b0 = 0, b1 = nbk > b ? (nbk - b + kFG - 1) / kFG : 0;  // this workgroup's blocks, counted
        const size_t srow = scale_row_bytes(FMT, H);
        u32x4 wv[GD][NCG];
        uint32_t ws[GD][NCG];
        auto issue = [&](int jb, u32x4 *v, uint32_t *sc) {  // this workgroup's block jb
            const int blk = b + kFG * jb;
            const int u = blk / bpu, i = (blk - u * bpu) * 8 + (r & 7), e = sh.u_e[u];
            const WMat &m = r < 8 ? a.w.gate : a.w.up;
            if (FMT == 0) {
                const uint16_t *row = reinterpret_cast<const uint16_t *>(wbase(m, e, E, (size_t)I * H * 2)) + (size_t)i * H + g * 8;
#pragma unroll
                for (int c = 0; c < NCG; c++) v[c] = c < ng ? ldg16(row + (kg0 + c) * 32) : u32x4{0u, 0u, 0u, 0u};
            } else {
                const uint8_t *row = wbase(m, e, E, (size_t)I * H / 2) + (size_t)i * (H / 2);
                const uint8_t *sf = wsf(m, e, E, (size_t)I * srow) + (size_t)i * srow;
#pragma unroll
                for (int c = 0; c < NCG; c++) {
                    const int kb = (kg0 + c) * 128 + g * 32;
                    const bool in = c < ng && kb < H;
                    v[c] = in ? ldg16(row + kb / 2) : u32x4{0u, 0u, 0u, 0u};
                    sc[c] = in ? *reinterpret_cast<const uint16_t *>(sf + (FMT == 1 ? kb / 16 : 2 * (kg0 + c))) : 0u;
                }
            }
        };
        // the last wave: lane = (token m, pairs q0 and q0 + 1 of the block)
        auto epilogue = [&](int jb) {
            const int blk = b + kFG * jb;
            const int u = blk / bpu, i0 = (blk - u * bpu) * 8;
            const int m = lane >> 2, q0 = 2 * (lane & 3);
            const int slot = m < T ? sh.u_tslot[u][m] : -1;
            if (slot >= 0) {
                const float tg = FMT == 1 ? sh.u_ts[0][u] : 1.f, tu = FMT == 1 ? sh.u_ts[1][u] : 1.f;
                float hv[2];
#pragma unroll
                for (int qq = 0; qq < 2; qq++) {
                    // D[m][n] sits in lane 16 (m / 4) + n, element m % 4: g in n < 8, u in n + 8
                    const int l = 16 * (m >> 2) + q0 + qq, el = m & 3;
                    float gs = 0.f, us = 0.f;
#pragma unroll
                    for (int w2 = 0; w2 < kFComp; w2++) {
                        gs += sh.red[par][w2][l][el];
                        us += sh.red[par][w2][l + 8][el];
                    }
                    hv[qq] = silu(gs * tg) * (us * tu);
                }
                put_h2(a.xh + (size_t)slot * (I / 2) + (i0 + q0) / 2, tag, hv[0], hv[1]);
            }
        };
        if (comp)
#pragma unroll
            for (int s = 0; s < GD; s++)
                if (b0 + s < b1) issue(b0 + s, wv[s], ws[s]);
        for (int base = b0; base < b1; base += GD) {
#pragma unroll
            for (int s = 0; s < GD; s++) {
                const int blk = base + s;
                if (blk < b1) {
                    if (comp) {
                        const f32x4 acc = tile_mma<FMT, NCG>(ax, wv[s], ws[s], ng);
                        if (blk + GD < b1) issue(blk + GD, wv[s], ws[s]);
                        sh.red[par][wave][lane] = acc;
                    }
                    lds_barrier();
                    if (!comp) epilogue(blk);
                    par ^= 1;
                }
            }
        }
    }

    // ---------------- down
    {
        const int rpu = H / 16, ndb = nunits * rpu;
        const int d0 = (int)((int64_t)ndb * b / kFG), d1 = (int)((int64_t)ndb * (b + 1) / kFG);
        const int nkd = FMT == 0 ? I / 32 : (I + 127) / 128;
        const int kd0 = comp ? nkd * wave / kFComp : 0, nd = comp ? nkd * (wave + 1) / kFComp - kd0 : 0;
        const size_t srow = scale_row_bytes(FMT, I);
        u32x4 wv[DD][NCD];
        uint32_t ws[DD][NCD];
        u32x4 ah[NAD];  // the current unit's h fragments (A rows = the unit's tokens)
        int au = -1;
        auto issue = [&](int blk, u32x4 *v, uint32_t *sc) {
            const int u = blk / rpu, n = (blk - u * rpu) * 16 + r, e = sh.u_e[u];
            if (FMT == 0) {
                const uint16_t *row = reinterpret_cast<const uint16_t *>(wbase(a.w.down, e, E, (size_t)H * I * 2)) + (size_t)n * I + g * 8;
#pragma unroll
                for (int c = 0; c < NCD; c++) v[c] = c < nd ? ldg16(row + (kd0 + c) * 32) : u32x4{0u, 0u, 0u, 0u};
            } else {
                const uint8_t *row = wbase(a.w.down, e, E, (size_t)H * I / 2) + (size_t)n * (I / 2);
                const uint8_t *sf = wsf(a.w.down, e, E, (size_t)H * srow) + (size_t)n * srow;
#pragma unroll
                for (int c = 0; c < NCD; c++) {
                    const int kb = (kd0 + c) * 128 + g * 32;
                    const bool in = c < nd && kb < I;
                    v[c] = in ? ldg16(row + kb / 2) : u32x4{0u, 0u, 0u, 0u};
                    sc[c] = in ? *reinterpret_cast<const uint16_t *>(sf + (FMT == 1 ? kb / 16 : 2 * (kd0 + c))) : 0u;
                }
            }
        };
        // Lane (g, r): token r of unit u; word j of its fragment list: bf16 chunk c = j / 4
        // holds columns 32 c + 8 g .. + 7 (words j % 4 of them); 4-bit super-chunk c = j / 16,
        // part jj = j / 4 % 4 holds columns 128 c + 32 g + 8 jj .. + 7.
        auto load_h = [&](int u) {
            constexpr int NW = 4 * NAD;
            const int cnt = sh.u_cnt[u];
            const bool has = r < cnt;
            const uint64_t *hp = a.xh + (size_t)(has ? sh.u_slot[u][r] : 0) * (I / 2);
            int off[NW];
            bool need[NW];
            uint64_t hw[NW];
#pragma unroll
            for (int j = 0; j < NW; j++) {
                int col;
                if (FMT == 0) {
                    col = (kd0 + j / 4) * 32 + g * 8;
                    need[j] = has && j / 4 < nd;
                } else {
                    const int kb = (kd0 + j / 16) * 128 + g * 32;
                    col = kb + 8 * ((j / 4) % 4);
                    need[j] = has && j / 16 < nd && kb < I;
                }
                off[j] = col / 2 + (j & 3);
                hw[j] = need[j] ? get_word(hp + off[j]) : 0ull;
            }
            for (int n = 0;; n++) {
                bool miss = false;
#pragma unroll
                for (int j = 0; j < NW; j++) miss |= need[j] && (uint32_t)(hw[j] >> 32) != tag;
                if (!miss) break;
                if (giveup || n >= kSpin) {
                    __hip_atomic_fetch_or(reinterpret_cast<uint32_t *>(a.head + kHeadError), kWsWaitTimeout,
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
#pragma unroll
                for (int j = 0; j < NW; j++)
                    if (need[j] && (uint32_t)(hw[j] >> 32) != tag) hw[j] = get_word(hp + off[j]);
            }
#pragma unroll
            for (int j = 0; j < NAD; j++)
                ah[j] = u32x4{(uint32_t)hw[4 * j], (uint32_t)hw[4 * j + 1], (uint32_t)hw[4 * j + 2], (uint32_t)hw[4 * j + 3]};
        };
        // the last wave: items (token m of the unit, row n0 + n), four per lane
        auto epilogue = [&](int blk) {
            const int u = blk / rpu, n0 = (blk - u * rpu) * 16, cnt = sh.u_cnt[u];
            const float ts = FMT == 1 ? sh.u_ts[2][u] : 1.f;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int item = lane + 64 * q, m = item >> 4, n = item & 15;
                if (m < cnt) {
                    const int l = 16 * (m >> 2) + n, el = m & 3;
                    float o = 0.f;
#pragma unroll
                    for (int w2 = 0; w2 < kFComp; w2++) o += sh.red[par][w2][l][el];
                    put_word(a.xo + (size_t)sh.u_slot[u][m] * H + n0 + n, tag, o * ts);
                }
            }
        };
        if (comp)
#pragma unroll
            for (int s = 0; s < DD; s++)
                if (d0 + s < d1) issue(d0 + s, wv[s], ws[s]);
        for (int base = d0; base < d1; base += DD) {
#pragma unroll
            for (int s = 0; s < DD; s++) {
                const int blk = base + s;
                if (blk < d1) {
                    if (comp) {
                        const int u = blk / rpu;
                        if (u != au) {
                            load_h(u);
                            au = u;
                        }
                        const f32x4 acc = tile_mma<FMT, NCD>(ah, wv[s], ws[s], nd);
                        if (blk + DD < d1) issue(blk + DD, wv[s], ws[s]);
                        sh.red[par][wave][lane] = acc;
                    }
                    lds_barrier();
                    if (!comp) epilogue(blk);
                    par ^= 1;
                }
            }
        }
    }

    // ---------------- combine
    {
        const int ne = T * H;
        const int e0 = (int)((int64_t)ne * b / kFG), e1 = (int)((int64_t)ne * (b + 1) / kFG);
        for (int el = e0 + tid; el < e1; el += 512) {
            const int t = el / H, n = el - t * H, nw = k + S;
            uint64_t ow[kFMaxK + 1];
            size_t off[kFMaxK + 1];
#pragma unroll
            for (int q = 0; q <= kFMaxK; q++) {
                const int slot = q < k ? sh.pos[t * k + q] : TK + t;  // q = k: the shared slot
                off[q] = (size_t)slot * H + n;
                ow[q] = q < nw ? get_word(a.xo + off[q]) : 0ull;
            }
            for (int it = 0;; it++) {
                bool miss = false;
#pragma unroll
                for (int q = 0; q <= kFMaxK; q++) miss |= q < nw && (uint32_t)(ow[q] >> 32) != tag;
                if (!miss) break;
                if (giveup || it >= kSpin) {
                    __hip_atomic_fetch_or(reinterpret_cast<uint32_t *>(a.head + kHeadError), kWsWaitTimeout,
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
#pragma unroll
                for (int q = 0; q <= kFMaxK; q++)
                    if (q < nw && (uint32_t)(ow[q] >> 32) != tag) ow[q] = get_word(a.xo + off[q]);
            }
            float acc = 0.f;
#pragma unroll
            for (int q = 0; q <= kFMaxK; q++)  // shared first (word k), then j ascending
                if (S && q == k) acc = __uint_as_float((uint32_t)ow[q]);
#pragma unroll
            for (int q = 0; q < kFMaxK; q++)
                if (q < k) acc += sh.wt[t * k + q] * __uint_as_float((uint32_t)ow[q]);
            const uint32_t yv = f2bf(acc);
            a.y[(size_t)t * H + n] = (uint16_t)yv;
            if (a.xnext)
                a.xnext[(size_t)t * H + n] =
                    (uint16_t)(a.residual ? f2bf(bf2f(a.x[(size_t)t * H + n]) + bf2f(yv)) : yv);
        }
    }
    if (tid == 0) bump_launches(a.head, launches);  // last, as in decode1_kernel
}

}  // namespace

static const void *few_entry(int fmt)
{
    return fmt == 0 ? reinterpret_cast<const void *>(&decode_few_kernel<0>)
         : fmt == 1 ? reinterpret_cast<const void *>(&decode_few_kernel<1>)
                    : reinterpret_cast<const void *>(&decode_few_kernel<2>);
}

bool decode_few_supported(const Shape &s, int fmt, int64_t T)
{
    return T >= 2 && T <= kFMaxT && s.E >= 1 && s.E <= kFMaxE && s.k >= 1 && s.k <= kFMaxK && s.k <= s.E &&
           s.S <= 1 && s.H % 64 == 0 && s.H <= kFMaxH && s.I % 32 == 0 && s.I <= kFMaxI &&
           persistent_fits(few_entry(fmt), 64 * kFWaves, 0);
}

static void launch_few(const FArgs &a, int fmt, hipStream_t st)
{
    if (fmt == 0) decode_few_kernel<0><<<kFG, 64 * kFWaves, 0, st>>>(a);
    else if (fmt == 1) decode_few_kernel<1><<<kFG, 64 * kFWaves, 0, st>>>(a);
    else decode_few_kernel<2><<<kFG, 64 * kFWaves, 0, st>>>(a);
}

static FArgs few_args(const Shape &s, const WSet &w, int64_t T, void *head)
{
    char *hb = static_cast<char *>(head);
    FArgs a{};
    a.T = (int)T;
    a.H = s.H;
    a.I = s.I;
    a.E = s.E;
    a.k = s.k;
    a.S = s.S;
    a.renorm = s.renorm;
    a.w = w;
    a.head = reinterpret_cast<uint8_t *>(hb);
    a.xlog = reinterpret_cast<uint64_t *>(hb + kFLogOff);
    a.xh = reinterpret_cast<uint64_t *>(hb + kFHOff);
    a.xo = reinterpret_cast<uint64_t *>(hb + kFOOff);
    return a;
}

hipError_t launch_decode_few(const Shape &s, const WSet &w, int64_t T, const uint16_t *x, const float *Wr,
                             const float *bias, uint16_t *y, float *logits, int32_t *ids, float *tw,
                             int32_t *counts, int32_t *offsets, int32_t *sa, int32_t *ap, void *head,
                             hipStream_t st)
{
    FArgs a = few_args(s, w, T, head);
    a.x = x;
    a.Wr = Wr;
    a.bias = bias;
    a.y = y;
    a.logits = logits;
    a.ids = ids;
    a.tw = tw;
    a.counts = counts;
    a.offsets = offsets;
    a.sa = sa;
    a.ap = ap;
    launch_few(a, w.fmt, st);
    return hipGetLastError();
}

hipError_t launch_decode_few_chain(const Shape &s, const WSet *w, const float *const *Wr,
                                   const float *const *bias, int L, int l0, bool residual, int64_t T,
                                   const uint16_t *x, bool hand_on, uint16_t *y, int32_t *ids, float *tw,
                                   float *logits, int32_t *ids_scratch, float *tw_scratch, void *head,
                                   hipStream_t st)
{
    uint16_t *buf = reinterpret_cast<uint16_t *>(static_cast<char *>(head) + kFXOff);
    const size_t tb = (size_t)kFMaxT * kFMaxH;  // elements per token buffer
    for (int l = 0; l < L; l++) {
        const int g = l0 + l;  // layer index within the whole chain: its tokens are in buffer g % 2
        FArgs a = few_args(s, w[l], T, head);
        a.x = g == 0 && x ? x : buf + (size_t)(g & 1) * tb;
        a.Wr = Wr[l];
        a.bias = bias[l];
        a.y = y + (size_t)l * T * s.H;
        a.xnext = l + 1 < L || hand_on ? buf + (size_t)((g + 1) & 1) * tb : nullptr;
        a.residual = residual ? 1 : 0;
        a.logits = logits ? logits + (size_t)l * T * s.E : nullptr;
        a.ids = ids ? ids + (size_t)l * T * s.k : ids_scratch;
        a.tw = tw ? tw + (size_t)l * T * s.k : tw_scratch;
        launch_few(a, w[l].fmt, st);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace flint
