// decode1.hip -- the whole MoE layer for one token in a single persistent launch.
//
// Decode of one token reads only the active weights (qantcore.space review, section 01),
// 68 MB per layer at H=2048, I=768, so a layer is ~11 us of HBM streaming.  On this GPU
// every kernel launch costs ~1.6 us and every dependent global round trip ~1.5-2 us, so
// the layer runs as one launch of one workgroup per CU in three phases:
//
//   phase 1  router row e = workgroup id (fp32, one wave); the shared expert's gate/up rows
//            of this workgroup's I-slice (known before routing: news.ditty.ir, third
//            paragraph, one shared expert always active) -> h of the shared slot; the
//            shared expert's down rows of this workgroup's H-slice go straight into LDS.
//   wait     for the 256 logit words.
//   phase 2  every wave selects the top-k of the 256 logits itself (same code, same bits,
//            so every copy agrees).  Right after round j it issues its gate/up row of
//            that expert (workgroup b owns rows [b I/256, (b+1) I/256) of every selected
//            expert: the single token is the same for every expert); the later selection
//            rounds run while the first slots stream.  The selected experts' down rows of
//            the H-slice are copied HBM -> LDS (no registers): bf16 by the last two waves
//            after every gate/up row, so they land during the h exchange; 4-bit by every
//            wave with each slot.
//   wait     for the words of h: one per (pair of slots, row of I), two bf16 values each,
//            polled by the waves with no copies in flight.
//   phase 3  down rows from LDS against h (bf16, as on every path), one slot per wave and
//            8 lanes per row; combine (shared first, then j ascending) -> y.
//
// Cross-workgroup data (logits, h) moves as 64-bit exchange words {launch tag, payload}
// written with agent-scope stores and polled with agent-scope loads: one aligned 64-bit
// access carries the payload and its readiness together, so there are no grid barriers,
// fences or cache-wide write-backs, and a reader waits one round trip after the word it
// needs lands.  The launch's tag comes from the workspace head's launch counters: workgroup
// b reads counter b when it starts and writes it back plus one, and every persistent launch
// has exactly 256 workgroups, so every counter holds the number of earlier launches and all
// workgroups of a launch compute the same tag.  A workgroup that starts late still reads its
// own launch's count (only workgroup b of the next launch could change counter b, and the
// next launch on the stream starts after this one has ended), so a word it publishes never
// carries a later launch's tag.  No two workgroups touch one counter, so nothing contends
// for it.  Every wait is bounded: on timeout the kernel sets the head's error flag (read and
// cleared by flint_moe_workspace_status) and carries on with the values it has.  All 256
// workgroups must be resident together (one per CU): the host checks the CU count and the
// kernel's occupancy before choosing this launch.
#include "xchg.h"

#include <map>
#include <mutex>
#include <tuple>

namespace flint {

namespace {

constexpr int kG = 256;        // workgroups (one per CU)
constexpr int kWaves = 8;
constexpr int kMaxK = 8;
constexpr int kMaxXC = 4;      // 16-byte x chunks per lane: H <= 2048

// Exchange words in the workspace head (see common.h for the head's control words): u64
// words for the logits at kXLogOff (one per workgroup: the fp32 logit) and for h at kXHOff
// ([(k + S + 1) / 2][I]: word (q, i) holds bf16 h of slots 2 q (low half) and 2 q + 1 (high
// half) at row i; slot k = shared expert).  Every workgroup reads all of h, so two values per
// word halve the polling traffic, and h is rounded to bf16 before the down rows on every path
// anyway.  A chain of layers hands each token to the next launch through the bf16 [2048]
// buffer at kXNextOff.
constexpr size_t kXLogOff = kHeadXchg, kXHOff = kXLogOff + 8 * kG;
constexpr size_t kXNextOff = kXHOff + 8 * (size_t)(kMaxK + 1) * 1024;
static_assert(kXNextOff + 2 * 2048 <= kHeadFewXchg, "exchange words exceed their part of the head");
static_assert(kG == kPersistentGrid, "one launch counter per workgroup of a persistent launch");

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

// 16 bytes per lane from HBM straight into LDS: lane l writes lds + 16 l (lds is uniform).
__device__ __forceinline__ void lds_load16(const void *g, uint8_t *lds)
{
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

// 8 bf16 products summed into acc.  The elements go through named scalars: a bit cast
// taken directly of an indexed vector element in an unrolled loop reads element 0 every
// time with this compiler.
__device__ __forceinline__ float dot8_bf16(u32x4 w, u32x4 x, float acc)
{
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t wi = w[i], xi = x[i];
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, wi), __builtin_bit_cast(bf16x2, xi), acc, false);
    }
    return acc;
}

// One 16-byte NVFP4 chunk (32 codes = 2 blocks of 16) against 32 fp32 x values:
// sum over each block of e2m1 * x, times the block's E4M3 scale.
__device__ __forceinline__ float dot32_nvfp4(u32x4 q, uint32_t sb2, const float *xv)
{
    float blk[2] = {0.f, 0.f};
#pragma unroll
    for (int wd = 0; wd < 4; wd++) {
        const uint32_t qw = q[wd];
        const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(qw, 1.0f, 0);
        const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(qw, 1.0f, 1);
        const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(qw, 1.0f, 2);
        const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(qw, 1.0f, 3);
        const float *xp = xv + 8 * wd;
        float s = blk[wd >> 1];
        s += v0[0] * xp[0];
        s += v0[1] * xp[1];
        s += v1[0] * xp[2];
        s += v1[1] * xp[3];
        s += v2[0] * xp[4];
        s += v2[1] * xp[5];
        s += v3[0] * xp[6];
        s += v3[1] * xp[7];
        blk[wd >> 1] = s;
    }
    return blk[0] * e4m3_to_f32(sb2 & 0xffu) + blk[1] * e4m3_to_f32((sb2 >> 8) & 0xffu);
}

// One 16-byte INT4 chunk (32 signed nibbles of one 128-column group) against 32 fp32 x
// values, times the group's bf16 scale.
__device__ __forceinline__ float dot32_int4(u32x4 q, uint32_t sbits, const float *xv)
{
    float acc = 0.f;
#pragma unroll
    for (int wd = 0; wd < 4; wd++) {
        const uint32_t qw = q[wd];
#pragma unroll
        for (int i = 0; i < 8; i++) acc += (float)int4_at(qw, i) * xv[8 * wd + i];
    }
    return acc * bf2f(sbits & 0xffffu);
}

// Eight INT4 nibbles (one word) against 8 bf16 h values, in fp32.
__device__ __forceinline__ float dot8_int4_bf16(uint32_t q, u32x4 h, float acc)
{
    const uint32_t h0 = h[0], h1 = h[1], h2 = h[2], h3 = h[3];
    const uint32_t hv[4] = {h0, h1, h2, h3};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        acc += (float)int4_at(q, 2 * i) * bf2f(hv[i] & 0xffffu);
        acc += (float)int4_at(q, 2 * i + 1) * bf2f(hv[i] >> 16);
    }
    return acc;
}

// Eight E2M1 codes (one word, low nibble first) against 8 bf16 h values: exact e2m1
// values as bf16 pairs, then bf16 dot products.
__device__ __forceinline__ float dot8_fp4_bf16(uint32_t q, u32x4 h, float acc)
{
    const uint32_t h0 = h[0], h1 = h[1], h2 = h[2], h3 = h[3];
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 0), __builtin_bit_cast(bf16x2, h0), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 1), __builtin_bit_cast(bf16x2, h1), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 2), __builtin_bit_cast(bf16x2, h2), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, 1.0f, 3), __builtin_bit_cast(bf16x2, h3), acc, false);
    return acc;
}

struct D1Args {
    int H, I, E, k, S, renorm;
    WSet w;
    const uint16_t *x;
    const float *Wr, *bias;
    uint16_t *y;
    uint16_t *xnext;  // null, or receives the next layer's token: y, or bf16(x + y) with `residual`
    int residual;
    float *logits;
    int32_t *ids;
    float *tw;
    int32_t *counts, *offsets, *sa, *ap;  // null in a chain
    uint8_t *head;   // workspace head: launch counters, error flags, diagnostic switch
    uint64_t *xlog;  // [256] exchange words: logit of expert b (workgroup b)
    uint64_t *xh;    // [(k + S + 1) / 2][I] exchange words, two slots each: slot j < k = j-th
                     // selected expert, slot k = shared
};

__device__ __forceinline__ const uint8_t *mat_base(const WMat &m, int e, int E, size_t bytes)
{
    return e == E ? m.shared : m.routed + (size_t)e * bytes;
}
__device__ __forceinline__ const uint8_t *mat_sf(const WMat &m, int e, int E, size_t bytes)
{
    return e == E ? m.sf_shared : m.sf_routed + (size_t)e * bytes;
}
__device__ __forceinline__ float mat_ts(const WMat &m, int e, int E)
{
    return e == E ? *m.ts_shared : m.ts_routed[e];
}

// One gate or up row (expert e, row i) of a wave in flight: bf16 lane chunks lane + 64 c,
// or the lane's NVFP4 chunk with its two block scales and the tensor scale.
template <int FMT>
struct RowLoad {
    u32x4 v[FMT == 0 ? kMaxXC : 1];
    uint32_t sb;
    float ts;
};

template <int FMT>
__device__ __forceinline__ void row_issue(const D1Args &a, const WMat &m, int e, int i, RowLoad<FMT> &r)
{
    const int lane = threadIdx.x & 63, H = a.H, I = a.I, E = a.E;
    if (FMT == 0) {
        const uint16_t *row = reinterpret_cast<const uint16_t *>(mat_base(m, e, E, (size_t)I * H * 2)) + (size_t)i * H;
#pragma unroll
        for (int c = 0; c < kMaxXC; c++)
            if (lane + 64 * c < H / 8) r.v[c] = ld16(row + 8 * (lane + 64 * c));
    } else {  // NVFP4: the lane's 32 k = 2 blocks; INT4: a quarter of one 128-column group
        const size_t srow = scale_row_bytes(FMT, H);
        const uint8_t *row = mat_base(m, e, E, (size_t)I * H / 2) + (size_t)i * (H / 2);
        const uint8_t *sf = mat_sf(m, e, E, (size_t)I * srow) + (size_t)i * srow;
        if (lane < H / 32) {
            r.v[0] = ld16(row + 16 * lane);
            r.sb = *reinterpret_cast<const uint16_t *>(sf + (FMT == 1 ? 2 * lane : 2 * (lane >> 2)));
        }
        r.ts = FMT == 1 ? mat_ts(m, e, E) : 1.f;
    }
}

template <int FMT>
__device__ __forceinline__ float row_dot(const D1Args &a, const RowLoad<FMT> &r, const u32x4 *xb, const float *xf)
{
    const int lane = threadIdx.x & 63, H = a.H;
    float acc = 0.f;
    if (FMT == 0) {
#pragma unroll
        for (int c = 0; c < kMaxXC; c++)
            if (lane + 64 * c < H / 8) acc = dot8_bf16(r.v[c], xb[c], acc);
        return wave_sum(acc);
    }
    if (lane < H / 32) acc = FMT == 1 ? dot32_nvfp4(r.v[0], r.sb, xf) : dot32_int4(r.v[0], r.sb, xf);
    return wave_sum(acc) * r.ts;
}

struct D1Shared {
    float lg[kG];                 // the logits, for every wave's selection
    float gs[4], us[4];           // shared expert gate / up of this workgroup's pairs
    float g[kMaxK][4], u[kMaxK][4];
    int32_t ids[kMaxK];
    float wt[kMaxK];
    float dts[kMaxK + 1];         // NVFP4 down tensor scale of every slot
    float o[kMaxK + 1][8];        // per-slot down outputs of this workgroup's rows_h columns
    uint32_t tag, giveup;         // this launch's tag and the diagnostic switch (from wave 0)
    __attribute__((aligned(16))) uint16_t hb[(kMaxK + 1) * 1024];  // h of every slot, bf16 [slot][I]
};

template <int FMT>
__global__ __launch_bounds__(512) void decode1_kernel(D1Args a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];  // down rows of this H-slice
    __shared__ D1Shared sh;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int b = blockIdx.x;
    const int H = a.H, I = a.I, E = a.E, k = a.k, S = a.S, ns = k + S;
    const int rows_h = H / kG;                        // down rows (columns of y) per workgroup
    const int n0 = b * rows_h;
    const int i0 = b * I / kG, npair = (b + 1) * I / kG - i0;  // gate/up rows of every expert
    // The launch counter is read before anything else; wave 0 needs the tag only once its
    // router row is in (its loads return in order), the other waves read it from LDS after
    // phase 1.
    uint32_t launches = 0, diag = 0;
    if (tid == 0) {
        launches = read_launches(a.head);
        diag = diag_word(a.head);
    }
    const size_t drow_bytes = FMT == 0 ? (size_t)I * 2 : (size_t)I / 2 + scale_row_bytes(FMT, I);
    const int cpb = (int)(rows_h * drow_bytes / 16);  // 16-byte chunks per slot block
    const int ngrp = (cpb + 63) / 64;                 // 64-chunk groups per slot block

    // Token in registers: bf16 chunks for the bf16 dot, fp32 for the NVFP4 dot.
    u32x4 xb[kMaxXC];
    float xf[32];
    if (FMT == 0) {
#pragma unroll
        for (int c = 0; c < kMaxXC; c++) xb[c] = (lane + 64 * c < H / 8) ? ld16(a.x + 8 * (lane + 64 * c)) : u32x4{0, 0, 0, 0};
    } else {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            u32x4 v = (lane < H / 32) ? ld16(a.x + 32 * lane + 8 * i) : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const uint32_t vj = v[j];
                xf[8 * i + 2 * j] = bf2f(vj & 0xffffu);
                xf[8 * i + 2 * j + 1] = bf2f(vj >> 16);
            }
        }
    }

    // Down rows of this H-slice, slot block j at dyn + j * cpb * 16: chunk c (16 bytes).
    // For NVFP4 a block is the rows' codes followed by their block scales (each contiguous
    // in HBM for a run of rows).  Waves w0 .. w0 + nw - 1 copy chunk groups w - w0,
    // w - w0 + nw, ...
    auto load_down = [&](int j, int e, int w0, int nw) {
        const int ncq = rows_h * I / 32;
        for (int g = wave - w0; g < ngrp; g += nw) {
            const int c = 64 * g + lane;
            if (c < cpb) {
                const uint8_t *src;
                if (FMT == 0) src = mat_base(a.w.down, e, E, (size_t)H * I * 2) + (size_t)n0 * I * 2 + 16 * c;
                else if (c < ncq) src = mat_base(a.w.down, e, E, (size_t)H * I / 2) + (size_t)n0 * (I / 2) + 16 * c;
                else src = mat_sf(a.w.down, e, E, (size_t)H * scale_row_bytes(FMT, I)) +
                           (size_t)n0 * scale_row_bytes(FMT, I) + 16 * (c - ncq);
                lds_load16(src, dyn + ((size_t)j * cpb + 64 * g) * 16);
            }
        }
    };

    // ---------------- phase 1
    // bf16: the router row goes out first: every workgroup's other copies wait for the
    // barrier below, so the 2 MB of router rows are ahead of the shared expert's 9 MB in the
    // memory queues and the logits, on which everything after depends, come back sooner
    // (with 4-bit weights the shared expert is 2.6 MB and holding it back measured slower).
    if (FMT != 0 && S) load_down(k, E, 0, kWaves);
    float4 wv[8];
    u32x2 xv[8];
    if (wave == 0 && b < E) {  // E <= 256: workgroup b computes logit b, if there is one
        const float4 *w4 = reinterpret_cast<const float4 *>(a.Wr + (size_t)b * H);
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int c = lane + 64 * i;
            wv[i] = c < H / 4 ? w4[c] : float4{0.f, 0.f, 0.f, 0.f};
            xv[i] = c < H / 4 ? *reinterpret_cast<const u32x2 *>(a.x + 4 * c) : u32x2{0u, 0u};
        }
    }
    if (FMT == 0) {
        __syncthreads();
        if (S) load_down(k, E, 0, kWaves);
    }
    if (wave == 0) {
        const uint32_t tag0 = __builtin_amdgcn_readlane(launch_tag(launches), 0);
        if (lane == 0) {
            sh.tag = tag0;
            sh.giveup = diag;
        }
        const int e = b;
        if (e < E) {      // router row: one logit
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const uint32_t x0 = xv[i][0], x1 = xv[i][1];
                acc += bf2f(x0 & 0xffffu) * wv[i].x;
                acc += bf2f(x0 >> 16) * wv[i].y;
                acc += bf2f(x1 & 0xffffu) * wv[i].z;
                acc += bf2f(x1 >> 16) * wv[i].w;
            }
            const float l = wave_sum(acc) + (a.bias ? a.bias[e] : 0.f);
            if (lane == 0) {
                if (a.logits) a.logits[e] = l;
                put_word(a.xlog + b, tag0, l);
            }
        } else if (lane == 0) {
            put_word(a.xlog + b, tag0, 0.f);  // no expert: the word only says "workgroup started"
        }
    } else if (S) {
        // shared expert rows r = 2 (i - i0) + {0 gate, 1 up}, r < 2 npair: wave 1 + r % 7
        RowLoad<FMT> r0, r1;
        const int ra = wave - 1, rb = wave + 6;
        if (ra < 2 * npair) row_issue<FMT>(a, (ra & 1) ? a.w.up : a.w.gate, E, i0 + (ra >> 1), r0);
        if (rb < 2 * npair) row_issue<FMT>(a, (rb & 1) ? a.w.up : a.w.gate, E, i0 + (rb >> 1), r1);
        if (ra < 2 * npair) {
            const float v = row_dot<FMT>(a, r0, xb, xf);
            if (lane == 0) ((ra & 1) ? sh.us : sh.gs)[ra >> 1] = v;
        }
        if (rb < 2 * npair) {
            const float v = row_dot<FMT>(a, r1, xb, xf);
            if (lane == 0) ((rb & 1) ? sh.us : sh.gs)[rb >> 1] = v;
        }
    }
    __syncthreads();
    const uint32_t tag = sh.tag;
    const bool giveup = sh.giveup != 0;
    // the shared slot k has a word of its own when k is even; otherwise it shares one with
    // slot k - 1 and goes out in phase 2
    if (S && (k & 1) == 0 && tid < npair)
        put_h2(a.xh + (size_t)(k / 2) * I + i0 + tid, tag, silu(sh.gs[tid]) * sh.us[tid], 0.f);

    // ---------------- phase 2: selection (every wave), routed gate/up rows, down rows
    if (wave == 0) {
        uint64_t lw[4];
#pragma unroll
        for (int i = 0; i < 4; i++) lw[i] = get_word(a.xlog + lane + 64 * i);
        await_words<4>(a.xlog + lane, 64, 4, lw, tag, a.head, giveup);
#pragma unroll
        for (int i = 0; i < 4; i++) sh.lg[lane + 64 * i] = __uint_as_float((uint32_t)lw[i]);
    }
    __syncthreads();
    // Lane holds experts lane + 64 i.  Key = order of the logit (select_key's high word)
    // plus one, 0 = no expert or already taken, so a NaN logit (order 0) still ranks above
    // those.  Each round takes the largest key; among equal keys the lowest expert, found
    // as the first i with a match and the lowest lane in it.
    uint32_t key[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const int e = lane + 64 * i;
        key[i] = e < E ? (uint32_t)(select_key(sh.lg[e], e) >> 32) + 1u : 0u;
    }
    const bool has_row = wave < 2 * npair;  // this wave's row: pair i0 + wave / 2, gate if even
    const WMat &my_mat = (wave & 1) ? a.w.up : a.w.gate;
    int sel[kMaxK];
    uint32_t ordv[kMaxK];
    RowLoad<FMT> rl[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; j++) {
        if (j < k) {
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
            const int e = wl + 64 * i;
            sel[j] = e;
            ordv[j] = m - 1u;
            if (has_row) row_issue<FMT>(a, my_mat, e, i0 + (wave >> 1), rl[j]);
            if (FMT != 0) load_down(j, e, 0, kWaves);
        }
    }
    // bf16: the routed down rows are needed only after the h exchange: the last two waves
    // copy them once every gate/up row has been asked for, so the gate/up rows, on which h
    // and everything after it wait, are ahead of them in the memory queues; the copies then
    // land while h is exchanged.  (These waves' own loads return in order, so they take no
    // part in polling for h.)  With 4-bit weights the down rows are a few KB per slot and
    // go out with each slot, by every wave (deferring them measured slower).
    if (FMT == 0 && wave >= kWaves - 2) {
#pragma unroll
        for (int j = 0; j < kMaxK; j++)
            if (j < k) load_down(j, sel[j], kWaves - 2, 2);
    }
    if (wave == 0 && lane == 0) {
        float sum = 0.f;
        for (int j = 0; j < k; j++) {
            // the logit from its order (inverse of select_key; -0 comes back as +0)
            const uint32_t o = ordv[j];
            const float l = __uint_as_float((o & 0x80000000u) ? (o ^ 0x80000000u) : ~o);
            const float sg = 1.0f / (1.0f + expf(-l));
            sh.ids[j] = sel[j];
            sh.wt[j] = sg;
            sum += sg;
        }
        if (a.renorm)
            for (int j = 0; j < k; j++) sh.wt[j] = sh.wt[j] / sum;
    }
    float dts = 1.f;
    if (FMT == 1 && wave == 0 && lane < ns) {
        int e = E;
#pragma unroll
        for (int j = 0; j < kMaxK; j++)
            if (j < k && lane == j) e = sel[j];
        dts = mat_ts(a.w.down, e, E);
    }
    if (has_row) {
#pragma unroll
        for (int j = 0; j < kMaxK; j++) {
            if (j < k) {
                const float v = row_dot<FMT>(a, rl[j], xb, xf);
                if (lane == 0) ((wave & 1) ? sh.u : sh.g)[j][wave >> 1] = v;
            }
        }
    }
    if (FMT == 1 && wave == 0 && lane < ns) sh.dts[lane] = dts;
    if (FMT == 0) {
        // LDS writes done, then a barrier that does not wait for the down-row copies in flight
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt untouched
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    } else {
        __syncthreads();  // also completes this workgroup's HBM -> LDS copies
    }
    for (int q = tid; q < (k + 1) / 2 * npair; q += 512) {
        const int jp = q / npair, p = q - jp * npair, j = 2 * jp;
        const float lo = silu(sh.g[j][p]) * sh.u[j][p];
        const float hi = j + 1 < k ? silu(sh.g[j + 1][p]) * sh.u[j + 1][p]
                                   : (S ? silu(sh.gs[p]) * sh.us[p] : 0.f);  // slot k: shared
        put_h2(a.xh + (size_t)jp * I + i0 + p, tag, lo, hi);
    }
    if (b == 0 && tid < 64) {  // publish the routing tensors (the single token: t = 0)
        if (tid < k) {
            if (a.ids) a.ids[tid] = sh.ids[tid];
            if (a.tw) a.tw[tid] = sh.wt[tid];
        }
        if (a.counts) {
            for (int e = tid; e <= E; e += 64) {
                int below = 0, eq = 0;
                for (int j = 0; j < k; j++) {
                    below += sh.ids[j] < e;
                    eq += sh.ids[j] == e;
                }
                a.offsets[e] = below;
                if (e < E) a.counts[e] = eq;
            }
            if (tid < k) {
                int pos = 0;
                for (int j = 0; j < k; j++) pos += sh.ids[j] < sh.ids[tid];
                a.sa[pos] = tid;
                a.ap[tid] = pos;
            }
        }
    }

    // ---------------- phase 3: down rows from LDS against h, combine
    // bf16: first one word of each workgroup's phase-2 words (slot pair 0, its first row):
    // they go out together, so this waits for every workgroup's h with a twelfth of the
    // polling traffic; then every word (any still missing awaited).  (Measured: bf16 layer
    // 21.4 -> 21.2 us, chain 21.6 -> 20.9 us; NVFP4 17.4 -> 17.9 us, so not with 4-bit
    // weights.)
    if (FMT == 0) {
        if (tid < kG && (tid + 1) * I / kG > tid * I / kG) {
            uint64_t sw = get_word(a.xh + tid * I / kG);
            await_words<1>(a.xh + tid * I / kG, 0, 1, &sw, tag, a.head, giveup);
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // a barrier that waits for no copy in flight
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    {
        constexpr int kPollT = 64 * (FMT == 0 ? kWaves - 2 : kWaves);  // waves with no down-row copies in flight
        constexpr int NH = ((kMaxK + 2) / 2 * 1024 + kPollT - 1) / kPollT;
        const int nh = (ns + 1) / 2 * I, nq = tid < kPollT && tid < nh ? (nh - tid + kPollT - 1) / kPollT : 0;
        uint64_t hw[NH];
#pragma unroll
        for (int q = 0; q < NH; q++) hw[q] = q < nq ? get_word(a.xh + tid + kPollT * q) : 0ull;
        await_words<NH>(a.xh + tid, kPollT, nq, hw, tag, a.head, giveup);
#pragma unroll
        for (int q = 0; q < NH; q++) {
            if (q < nq) {
                const int wdx = tid + kPollT * q, jp = wdx / I, i = wdx - jp * I;
                sh.hb[(size_t)(2 * jp) * I + i] = (uint16_t)(hw[q] & 0xffffu);
                if (2 * jp + 1 < ns) sh.hb[(size_t)(2 * jp + 1) * I + i] = (uint16_t)((hw[q] >> 16) & 0xffffu);
            }
        }
    }
    __syncthreads();
    // Wave w takes slot j = w (and j + 8); lane = (row n = lane / 8, part s = lane % 8):
    // the 8 lanes of row n0 + n take 16-byte units s, s + 8, ... so that every group of
    // 8 lanes reads 128 contiguous bytes of LDS.
    {
        const int n = lane >> 3, s = lane & 7;
        for (int j = wave; j < ns; j += kWaves) {
            float acc = 0.f;
            if (n < rows_h) {
                const uint8_t *blk = dyn + (size_t)j * cpb * 16;
                const uint16_t *hj = sh.hb + (size_t)j * I;
                if (FMT == 0) {
                    const uint8_t *row = blk + (size_t)n * drow_bytes;
                    for (int c = s; c < I / 8; c += 8)
                        acc = dot8_bf16(*reinterpret_cast<const u32x4 *>(row + 16 * c),
                                        *reinterpret_cast<const u32x4 *>(hj + 8 * c), acc);
                } else if (FMT == 1) {
                    const uint8_t *qrow = blk + (size_t)n * (I / 2);
                    const uint8_t *sf = blk + (size_t)rows_h * (I / 2) + (size_t)n * (I / 16);
                    for (int c = s; c < I / 16; c += 8) {  // 16-element blocks: 8 code bytes, one scale
                        const u32x2 q = *reinterpret_cast<const u32x2 *>(qrow + 8 * c);
                        const uint32_t q0 = q[0], q1 = q[1];
                        float p = dot8_fp4_bf16(q0, *reinterpret_cast<const u32x4 *>(hj + 16 * c), 0.f);
                        p = dot8_fp4_bf16(q1, *reinterpret_cast<const u32x4 *>(hj + 16 * c + 8), p);
                        acc += p * e4m3_to_f32(sf[c]);
                    }
                } else {
                    const uint8_t *qrow = blk + (size_t)n * (I / 2);
                    const uint16_t *sf = reinterpret_cast<const uint16_t *>(blk + (size_t)rows_h * (I / 2) + (size_t)n * (I / 64));
                    for (int c = s; c < I / 16; c += 8) {  // 16-element pieces; scale of group c / 8
                        const u32x2 q = *reinterpret_cast<const u32x2 *>(qrow + 8 * c);
                        const uint32_t q0 = q[0], q1 = q[1];
                        float p = dot8_int4_bf16(q0, *reinterpret_cast<const u32x4 *>(hj + 16 * c), 0.f);
                        p = dot8_int4_bf16(q1, *reinterpret_cast<const u32x4 *>(hj + 16 * c + 8), p);
                        acc += p * bf2f(sf[c >> 3]);
                    }
                }
            }
            // sum over the row's 8 lanes: xor 1, xor 2, then the mirror within 8 lanes
            acc += __int_as_float(FLINT_DPP(__float_as_int(acc), 0xB1));
            acc += __int_as_float(FLINT_DPP(__float_as_int(acc), 0x4E));
            acc += __int_as_float(FLINT_DPP(__float_as_int(acc), 0x141));
            if (s == 0 && n < rows_h) sh.o[j][n] = FMT == 1 ? acc * sh.dts[j] : acc;
        }
    }
    __syncthreads();
    for (int n = tid; n < rows_h; n += 512) {
        float acc = S ? sh.o[k][n] : 0.f;
        for (int j = 0; j < k; j++) acc += sh.wt[j] * sh.o[j][n];
        const uint32_t yv = f2bf(acc);
        a.y[n0 + n] = (uint16_t)yv;
        // The next layer's token (a chain): this launch read all of x in phase 1, before any
        // workgroup got here, so x and xnext may be the same buffer.
        if (a.xnext)
            a.xnext[n0 + n] = (uint16_t)(a.residual ? f2bf(bf2f(a.x[n0 + n]) + bf2f(yv)) : yv);
    }
    // last: a write-through store in flight holds up the next barrier's wait (measured
    // 1.2 us per layer when this store went out in phase 1)
    if (tid == 0) bump_launches(a.head, launches);
}

// ---------------------------------------------------------------- dense layer, one token
// A dense SwiGLU layer (no router, the one expert held as the shared expert: the dense
// layers of the same model, qantcore.space review, section 01) for one token, in one
// launch of one workgroup per CU.  h travels as W = I / 2 exchange words, word q holding
// bf16 h[2q] (low half) and h[2q + 1]; workgroup b owns words [b W / 256, (b + 1) W / 256)
// (1 to 8 of them) and the down rows of its H-slice.
//   waves 0-7   one word each: the gate and up rows 2q and 2q + 1 (4 rows of H in flight
//               per lane), then the word; then they poll all W words and write h to LDS.
//   waves 8-11  copy the down rows of the slice HBM -> LDS behind the row loads (4-bit:
//               the rows' codes, then their scales), and take no part in polling (a
//               wave's loads return in order).
//   all         down row n = wave of the slice against h from LDS -> y.
// The launch tag comes from the workgroup's launch counter, as in decode1_kernel.
constexpr int kDenseRowWaves = 8, kDenseWaves = kDenseRowWaves + 4, kDenseMaxI = 4096;

template <int FMT>
__global__ __launch_bounds__(64 * kDenseWaves) void dense1_kernel(D1Args a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];  // down rows of the slice
    __shared__ __attribute__((aligned(16))) uint16_t hb[kDenseMaxI];
    __shared__ uint32_t s_tag[2];  // this launch's tag, the diagnostic switch
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, b = blockIdx.x;
    const int H = a.H, I = a.I, W = I / 2;
    const int rows_h = H / kG, n0 = b * rows_h;
    const int q0 = b * W / kG, nq = (b + 1) * W / kG - q0;
    const size_t srow = scale_row_bytes(FMT, I);  // down row scale bytes (4-bit)

    // The row waves' loads go out first; the copy waves start after a barrier that waits
    // for no load, so the gate/up rows, on which h and the exchange wait, are ahead of the
    // down rows in the memory queues and the down rows land while h is exchanged.
    const bool rows = wave < kDenseRowWaves && wave < nq;
    uint32_t launches = 0, diag = 0;  // read first; needed only once the rows' products are done
    if (tid == 0) {
        launches = read_launches(a.head);
        diag = diag_word(a.head);
    }
    const int i = 2 * (q0 + wave);
    RowLoad<FMT> rl[4];  // gate i, up i, gate i + 1, up i + 1
    u32x4 xb[kMaxXC];
    float xf[32];
    if (rows) {
#pragma unroll
        for (int r = 0; r < 4; r++) row_issue<FMT>(a, (r & 1) ? a.w.up : a.w.gate, 0, i + (r >> 1), rl[r]);
        if (FMT == 0) {
#pragma unroll
            for (int c = 0; c < kMaxXC; c++)
                xb[c] = lane + 64 * c < H / 8 ? ld16(a.x + 8 * (lane + 64 * c)) : u32x4{0, 0, 0, 0};
        } else {
#pragma unroll
            for (int q = 0; q < 4; q++) {
                u32x4 v = (lane < H / 32) ? ld16(a.x + 32 * lane + 8 * q) : u32x4{0, 0, 0, 0};
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const uint32_t vj = v[j];
                    xf[8 * q + 2 * j] = bf2f(vj & 0xffffu);
                    xf[8 * q + 2 * j + 1] = bf2f(vj >> 16);
                }
            }
        }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    float d[4];
    if (wave >= kDenseRowWaves) {
        const size_t drow = FMT == 0 ? (size_t)I * 2 : (size_t)I / 2;  // code (or bf16) bytes per row
        const int ncq = (int)(rows_h * drow / 16);                      // 16-byte chunks of them
        const int cpb = ncq + (int)(rows_h * srow / 16);
        const uint8_t *src = a.w.down.shared + (size_t)n0 * drow;
        const uint8_t *ssrc = FMT == 0 ? nullptr : a.w.down.sf_shared + (size_t)n0 * srow;
        for (int g = wave - kDenseRowWaves; 64 * g < cpb; g += kDenseWaves - kDenseRowWaves) {
            const int c = 64 * g + lane;
            if (c < cpb) lds_load16(c < ncq ? src + 16 * c : ssrc + 16 * (c - ncq), dyn + (size_t)64 * g * 16);
        }
    } else if (rows) {
#pragma unroll
        for (int r = 0; r < 4; r++) d[r] = row_dot<FMT>(a, rl[r], xb, xf);
    }
    // The tag reaches every wave through LDS behind a barrier that waits for LDS writes
    // only (the copy waves' copies stay in flight).
    if (tid == 0) {
        s_tag[0] = launch_tag(launches);
        s_tag[1] = diag;
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt untouched
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const uint32_t tag = s_tag[0];
    const bool giveup = s_tag[1] != 0;
    if (rows && lane == 0) put_h2(a.xh + q0 + wave, tag, silu(d[0]) * d[1], silu(d[2]) * d[3]);
    if (wave < kDenseRowWaves) {
        constexpr int kPollT = 64 * kDenseRowWaves, NH = kDenseMaxI / 2 / kPollT;
        const int nw = tid < W ? (W - tid + kPollT - 1) / kPollT : 0;
        uint64_t hw[NH];
#pragma unroll
        for (int q = 0; q < NH; q++) hw[q] = q < nw ? get_word(a.xh + tid + kPollT * q) : 0ull;
        await_words<NH>(a.xh + tid, kPollT, nw, hw, tag, a.head, giveup);
#pragma unroll
        for (int q = 0; q < NH; q++)
            if (q < nw) reinterpret_cast<uint32_t *>(hb)[tid + kPollT * q] = (uint32_t)hw[q];
    }
    __syncthreads();  // h in LDS; the copy waves' down rows have landed
    if (wave < rows_h) {
        float acc = 0.f;
        if (FMT == 0) {
            const uint8_t *row = dyn + (size_t)wave * I * 2;
            for (int c = lane; c < I / 8; c += 64)
                acc = dot8_bf16(*reinterpret_cast<const u32x4 *>(row + 16 * c), *reinterpret_cast<const u32x4 *>(hb + 8 * c), acc);
        } else {
            // 16-element blocks c: 8 code bytes against 16 bf16 h values, times the block's
            // E4M3 scale (NVFP4) or the bf16 scale of its 128-column group (INT4)
            const uint8_t *qrow = dyn + (size_t)wave * (I / 2);
            const uint8_t *sf = dyn + (size_t)rows_h * (I / 2) + (size_t)wave * srow;
            for (int c = lane; c < I / 16; c += 64) {
                const u32x2 q = *reinterpret_cast<const u32x2 *>(qrow + 8 * c);
                const uint32_t q0w = q[0], q1w = q[1];
                const u32x4 h0 = *reinterpret_cast<const u32x4 *>(hb + 16 * c);
                const u32x4 h1 = *reinterpret_cast<const u32x4 *>(hb + 16 * c + 8);
                if (FMT == 1) {
                    const float p = dot8_fp4_bf16(q1w, h1, dot8_fp4_bf16(q0w, h0, 0.f));
                    acc += p * e4m3_to_f32(sf[c]);
                } else {
                    const float p = dot8_int4_bf16(q1w, h1, dot8_int4_bf16(q0w, h0, 0.f));
                    acc += p * bf2f(reinterpret_cast<const uint16_t *>(sf)[c >> 3]);
                }
            }
        }
        acc = wave_sum(acc);
        if (FMT == 1) acc *= *a.w.down.ts_shared;
        if (lane == 0) a.y[n0 + wave] = (uint16_t)f2bf(acc);
    }
    if (tid == 0) bump_launches(a.head, launches);  // last, as in decode1_kernel
}

}  // namespace

// LDS for the down rows of one workgroup's H-slice, all k + S experts.
static size_t d1_dyn_bytes(const Shape &s, int fmt)
{
    const size_t row = fmt == 0 ? (size_t)s.I * 2 : (size_t)s.I / 2 + scale_row_bytes(fmt, s.I);
    return (size_t)(s.k + s.S) * (s.H / kG) * row;
}

// A persistent launch needs every one of its kG workgroups resident at once: a device with
// at least kG CUs, and room on a CU for one workgroup of the kernel (registers and LDS,
// hipOccupancyMaxActiveBlocksPerMultiprocessor).  Asked once per (device, kernel, LDS bytes).
// It cannot see other work on the GPU: a launch that shares the CUs with other kernels may
// find its waits running out, which the workspace's error flags report.
bool persistent_fits(const void *kernel, int threads, size_t dyn)
{
    static std::mutex mu;
    static std::map<std::tuple<int, const void *, size_t>, bool> known;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    const auto key = std::make_tuple(dev, kernel, dyn);
    std::lock_guard<std::mutex> lock(mu);
    const auto it = known.find(key);
    if (it != known.end()) return it->second;
    int cus = 0, blocks = 0;
    const bool ok = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                    cus >= kG &&
                    hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, threads, dyn) == hipSuccess &&
                    blocks >= 1;
    known[key] = ok;
    return ok;
}

static const void *decode1_entry(int fmt)
{
    return fmt == 0 ? reinterpret_cast<const void *>(&decode1_kernel<0>)
         : fmt == 1 ? reinterpret_cast<const void *>(&decode1_kernel<1>)
                    : reinterpret_cast<const void *>(&decode1_kernel<2>);
}

bool decode1_supported(const Shape &s, int fmt)
{
    const size_t row = fmt == 0 ? (size_t)s.I * 2 : (size_t)s.I / 2 + scale_row_bytes(fmt, s.I);
    const int rows_h = s.H / kG;
    return s.E >= 1 && s.H % kG == 0 && s.H <= 2048 &&                   // rows_h <= 8, x in 4 chunks per lane
           s.I % 32 == 0 && s.I <= 1024 && s.k <= kMaxK &&    // <= 4 gate/up pairs: one row per wave
           (size_t)rows_h * row % 16 == 0 &&                  // whole 16-byte chunks per block
           d1_dyn_bytes(s, fmt) + sizeof(D1Shared) <= 160 * 1024 &&
           persistent_fits(decode1_entry(fmt), 512, d1_dyn_bytes(s, fmt));
}

static hipError_t launch_d1(const Shape &s, int fmt, const D1Args &a, hipStream_t st)
{
    const size_t dyn = d1_dyn_bytes(s, fmt);
    // HIP on gfx950 takes up to the CU's 160 KB of LDS per workgroup without an opt-in.
    if (fmt == 0) decode1_kernel<0><<<kG, 512, dyn, st>>>(a);
    else if (fmt == 1) decode1_kernel<1><<<kG, 512, dyn, st>>>(a);
    else decode1_kernel<2><<<kG, 512, dyn, st>>>(a);
    return hipGetLastError();
}

hipError_t launch_decode1(const Shape &s, const WSet &w, const uint16_t *x, const float *Wr,
                          const float *bias, uint16_t *y, float *logits, int32_t *ids, float *tw,
                          int32_t *counts, int32_t *offsets, int32_t *sa, int32_t *ap, void *head,
                          hipStream_t st)
{
    char *hb = static_cast<char *>(head);
    D1Args a{s.H, s.I, s.E, s.k, s.S, s.renorm, w, x, Wr, bias, y, nullptr, 0, logits, ids, tw,
             counts, offsets, sa, ap, reinterpret_cast<uint8_t *>(hb),
             reinterpret_cast<uint64_t *>(hb + kXLogOff), reinterpret_cast<uint64_t *>(hb + kXHOff)};
    return launch_d1(s, w.fmt, a, st);
}

hipError_t launch_decode_chain(const Shape &s, const WSet *w, const float *const *Wr,
                               const float *const *bias, int L, bool residual, const uint16_t *x,
                               bool hand_on, uint16_t *y, int32_t *ids, float *tw, float *logits,
                               void *head, hipStream_t st)
{
    char *hb = static_cast<char *>(head);
    uint16_t *xnext = reinterpret_cast<uint16_t *>(hb + kXNextOff);
    for (int l = 0; l < L; l++) {
        D1Args a{s.H, s.I, s.E, s.k, s.S, s.renorm, w[l], l == 0 && x ? x : xnext, Wr[l], bias[l],
                 y + (size_t)l * s.H, l + 1 < L || hand_on ? xnext : nullptr, residual ? 1 : 0,
                 logits ? logits + (size_t)l * s.E : nullptr, ids ? ids + (size_t)l * s.k : nullptr,
                 tw ? tw + (size_t)l * s.k : nullptr, nullptr, nullptr, nullptr, nullptr,
                 reinterpret_cast<uint8_t *>(hb), reinterpret_cast<uint64_t *>(hb + kXLogOff),
                 reinterpret_cast<uint64_t *>(hb + kXHOff)};
        const hipError_t e = launch_d1(s, w[l].fmt, a, st);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

bool dense1_supported(const Shape &s, int fmt)
{
    const size_t row = fmt == 0 ? (size_t)s.I * 2 : (size_t)s.I / 2 + scale_row_bytes(fmt, s.I);
    const int rows_h = s.H / kG;
    const void *entry = fmt == 0 ? reinterpret_cast<const void *>(&dense1_kernel<0>)
                      : fmt == 1 ? reinterpret_cast<const void *>(&dense1_kernel<1>)
                                 : reinterpret_cast<const void *>(&dense1_kernel<2>);
    return s.E == 0 && s.S == 1 && s.H % kG == 0 && s.H <= 2048 &&  // <= 8 down rows per workgroup
           s.I % 128 == 0 && s.I >= 2 * kG && s.I <= kDenseMaxI &&  // 1..8 h words per workgroup
           (size_t)rows_h * s.I / 2 % 16 == 0 && (size_t)rows_h * row % 16 == 0 &&  // whole chunks
           (size_t)rows_h * row <= 128 * 1024 && persistent_fits(entry, 64 * kDenseWaves, (size_t)rows_h * row);
}

hipError_t launch_dense1(const Shape &s, const WSet &w, const uint16_t *x, uint16_t *y, void *head,
                         hipStream_t st)
{
    char *hb = static_cast<char *>(head);
    D1Args a{};
    a.H = s.H;
    a.I = s.I;
    a.S = 1;
    a.w = w;
    a.x = x;
    a.y = y;
    a.head = reinterpret_cast<uint8_t *>(hb);
    a.xh = reinterpret_cast<uint64_t *>(hb + kXHOff);
    const size_t row = w.fmt == 0 ? (size_t)s.I * 2 : (size_t)s.I / 2 + scale_row_bytes(w.fmt, s.I);
    const size_t dyn = (size_t)(s.H / kG) * row;
    if (w.fmt == 0) dense1_kernel<0><<<kG, 64 * kDenseWaves, dyn, st>>>(a);
    else if (w.fmt == 1) dense1_kernel<1><<<kG, 64 * kDenseWaves, dyn, st>>>(a);
    else dense1_kernel<2><<<kG, 64 * kDenseWaves, dyn, st>>>(a);
    return hipGetLastError();
}

}  // namespace flint

namespace flint {

__global__ void ws_status_kernel(uint32_t *flags, int32_t *out)
{
    *out = (int32_t)__hip_atomic_exchange(flags, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_ws_status(void *head, int32_t *out, hipStream_t st)
{
    ws_status_kernel<<<1, 1, 0, st>>>(reinterpret_cast<uint32_t *>(static_cast<char *>(head) + kHeadError), out);
    return hipGetLastError();
}

}  // namespace flint
