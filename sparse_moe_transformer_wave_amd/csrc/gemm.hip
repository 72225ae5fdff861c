// gemm.hip -- grouped expert GEMMs for larger batches (T > 32 tokens) and the combine.
//
// Prefill is compute-heavy rather than weight-bound (recipes.vllm.ai "RecursiveSI/flint",
// Benchmarking: the NVFP4 checkpoint barely changes the 8K-token prefill time), so the
// expert FFNs run on bf16 MFMA with fp32 accumulation and LDS-staged tiles: bf16 weights
// through a ring of K stages filled HBM -> LDS directly (gemm_bf16k64_kernel, 64-wide
// stages; gemm_bf16_down_kernel, 32-wide, for a down pass with I % 64 == 32); 4-bit weights as
// their codes through a register ring, dequantised once into a bf16 LDS stage
// (gemm_q4_kernel, K a multiple of 128); NVFP4 weights whose K is not a multiple of 128
// through registers into a padded double buffer, dequantised on the way, with a prefetch of
// the next K step and zeros past K (grouped_gemm_kernel).
//
// Work items come from the device plan: one item = (touched expert, 256-row tile of its
// slots), so an expert of up to 256 rows streams its weights once.  Gate/up: A = the
// expert's tokens gathered from x, B = gate rows and the same up rows per wave column,
// epilogue h = bf16(silu(g) * u).  Down: A = h rows of the expert's slots (contiguous),
// epilogue o = bf16(acc).  N tiles past the matrix (I not a multiple of 128 for gate/up, H
// not a multiple of 256 for down) read a repeat of the last row and store nothing.  The
// combine then forms y = o_shared + sum_j w_j o_j per token, in that fixed order.
#include "common.h"

namespace flint {

namespace {

constexpr int BM = kGemmBM;  // rows (slots) per tile: a uniform expert fits in one tile
constexpr int BN = 256;      // B rows per tile
constexpr int BK = 64;       // K per stage
constexpr int LDP = BK + 8;  // padded LDS row (bf16 elements): 144 bytes
constexpr int NT = 1024;     // 16 waves: 4 (M) x 4 (N), 64 x 64 per wave
constexpr int NP = BM * (BK / 8) / NT;  // 16-byte chunks of A (and of B) staged per thread
constexpr int kXcds = 8;     // workgroup b runs on XCD b % 8
constexpr int kRingStages = 4;  // bf16 K-stage ring depth (32 KB per stage)

__device__ __forceinline__ u32x4 ld16g(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

// Workgroup b -> (item, N-tile): all N-tiles of an item go to one XCD, back to back, so
// the item's A tile is fetched into that XCD's L2 once and reused.
__device__ __forceinline__ void xcd_map(int b, int n_tiles, int &item, int &nb)
{
    const int x = b % kXcds, q = b / kXcds;
    nb = q % n_tiles;
    item = x + kXcds * (q / n_tiles);
}

// NVFP4 weights with K not a multiple of 128 (K a multiple of 16): the same 256 x 256 tiles
// and work items as the kernels below, A and B staged through registers into a padded
// double buffer, 64-wide K steps, the next step's loads in flight while the MFMAs run.
template <int MODE>
__global__ __launch_bounds__(NT) void grouped_gemm_kernel(int T, int H, int I, int E, int k,
                                                          WSet w,
                                                          const uint16_t *__restrict__ asrc,
                                                          const int32_t *__restrict__ sa,
                                                          Plan p, uint16_t *__restrict__ out)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM][LDP];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN][LDP];
    const int N = MODE == 0 ? 2 * I : H;  // B rows of the whole problem
    const int n_tiles = (N + BN - 1) / BN;
    int item, nb;
    xcd_map(blockIdx.x, n_tiles, item, nb);
    if (item >= p.meta[1]) return;
    const int code = p.items[item];
    const int u = code >> 16, mtile = code & 0xffff;
    const int e = p.touched[u], base = p.tbase[u], cnt = p.tcount[u];
    const bool sh = (e == E);
    const int m0 = mtile * BM;
    const int valid = min(BM, cnt - m0);
    const int K = MODE == 0 ? H : I;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
    const int wm = wave >> 2, wn = wave & 3;

    // Staging: thread tid copies chunk tid + NT j (row = chunk / 8, 16-byte column chunk % 8).
    const uint16_t *arow[NP];
    const uint8_t *brow[NP];
    const uint8_t *bsf[NP];
#pragma unroll
    for (int j = 0; j < NP; j++) {
        const int rr = (tid + NT * j) >> 3;
        const int ri = min(rr, valid - 1);
        if (MODE == 0) {
            const int tok = sh ? base - T * k + m0 + ri : sa[base + m0 + ri] / k;
            arow[j] = asrc + (size_t)tok * H;
        } else {
            arow[j] = asrc + (size_t)(base + m0 + ri) * I;
        }
        // B row rr of the tile.  Gate/up: each 64-row wave column holds 32 gate rows and the
        // same 32 up rows, so g and u of one column meet in the same lane.
        const WMat *mat;
        int n;
        if (MODE == 0) {
            const int wcol = rr >> 6, within = rr & 63;
            mat = (within >> 5) ? &w.up : &w.gate;
            n = min(nb * (BN / 2) + wcol * 32 + (within & 31), I - 1);
        } else {
            mat = &w.down;
            n = min(nb * BN + rr, H - 1);
        }
        const size_t mb = (size_t)H * I / 2, srow = scale_row_bytes(1, K), sb = (size_t)(H * I / K) * srow;
        brow[j] = (sh ? mat->shared : mat->routed + (size_t)e * mb) + (size_t)n * (K / 2);
        bsf[j] = (sh ? mat->sf_shared : mat->sf_routed + (size_t)e * sb) + (size_t)n * srow;
    }
    const int schunk = tid & 7;

    u32x4 ra[NP], rb[NP];
    auto gload = [&](int k0) {  // columns past K (the last stage when K % 64 != 0) are zeros
        const int kk = k0 + schunk * 8;
        const bool in = kk < K;
#pragma unroll
        for (int j = 0; j < NP; j++) {
            ra[j] = u32x4{0u, 0u, 0u, 0u};
            rb[j] = u32x4{0u, 0u, 0u, 0u};
            if (!in) continue;
            ra[j] = ld16g(arow[j] + kk);
            const uint32_t q = *reinterpret_cast<const uint32_t *>(brow[j] + kk / 2);
            rb[j] = dequant8(q, e4m3_to_f32(bsf[j][kk / 16]));
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int j = 0; j < NP; j++) {
            const int rr = (tid + NT * j) >> 3;
            *reinterpret_cast<u32x4 *>(&As[buf][rr][schunk * 8]) = ra[j];
            *reinterpret_cast<u32x4 *>(&Bs[buf][rr][schunk * 8]) = rb[j];
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (K + BK - 1) / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt++) {
        const int buf = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
        for (int kk = 0; kk < BK / 32; kk++) {
            bf16x8 af[4], bfr[4];
#pragma unroll
            for (int ms = 0; ms < 4; ms++)
                af[ms] = as_bf16x8(*reinterpret_cast<const u32x4 *>(&As[buf][wm * 64 + ms * 16 + r][kk * 32 + g * 8]));
#pragma unroll
            for (int ns = 0; ns < 4; ns++)
                bfr[ns] = as_bf16x8(*reinterpret_cast<const u32x4 *>(&Bs[buf][wn * 64 + ns * 16 + r][kk * 32 + g * 8]));
#pragma unroll
            for (int ms = 0; ms < 4; ms++)
#pragma unroll
                for (int ns = 0; ns < 4; ns++) acc[ms][ns] = mfma16x16x32(af[ms], bfr[ns], acc[ms][ns]);
        }
        if (kt + 1 < nk) lstore(buf ^ 1);
        __syncthreads();
    }

    // Epilogue.  acc[ms][ns][i] = D[row = wm*64 + ms*16 + 4g + i][brow = wn*64 + ns*16 + r].
    const float tsg = sh ? *w.gate.ts_shared : w.gate.ts_routed[e];
    const float tsu = sh ? *w.up.ts_shared : w.up.ts_routed[e];
    const float tsd = sh ? *w.down.ts_shared : w.down.ts_routed[e];
#pragma unroll
    for (int ms = 0; ms < 4; ms++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int row = wm * 64 + ms * 16 + 4 * g + i;
            if (row >= valid) continue;
            const size_t slot = (size_t)(base + m0 + row);
            if (MODE == 0) {
#pragma unroll
                for (int ns = 0; ns < 2; ns++) {
                    const int col = nb * (BN / 2) + wn * 32 + ns * 16 + r;
                    const float gv = acc[ms][ns][i] * tsg, uv = acc[ms][ns + 2][i] * tsu;
                    if (col < I) out[slot * I + col] = (uint16_t)f2bf(silu(gv) * uv);
                }
            } else {
#pragma unroll
                for (int ns = 0; ns < 4; ns++) {
                    const int col = nb * BN + wn * 64 + ns * 16 + r;
                    if (col < H) out[slot * H + col] = (uint16_t)f2bf(acc[ms][ns][i] * tsd);
                }
            }
        }
    }
}

// ---------------------------------------------------------------- bf16: 32-wide LDS ring
// The down pass when I % 64 == 32 (K = I not a whole number of 64-wide stages; the
// 64-wide kernel below takes every other bf16 pass).  The same tiles and work items as
// the other grouped GEMMs, with the K loop built around the
// CU's LDS: K runs in stages of 32 through a ring of NS stages (32 KB each: 256 A rows and
// 256 B rows of 64 bytes), filled HBM -> LDS by global_load_lds_dwordx4 (no registers)
// NS - 1 stages ahead, so three or four stages of loads are in flight per CU while the
// MFMAs consume the oldest one, and each stage costs one barrier.  Row R keeps its
// 16-byte chunk c at slot c ^ ((R >> 1) & 3).  A fragment read (lane (g, r): row r of a
// 16-row group, chunk g) then runs at the LDS's full 256 bytes per clock; measured on
// gfx950, the same read with c ^ ((R >> 2) & 3) or unswizzled 64-byte rows takes twice as
// long (two-way bank conflicts).  A copy instruction writes 1 KB of LDS contiguously (16
// whole rows), so the swizzle only decides which global chunk each lane fetches.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    // gfx9 s_waitcnt: vmcnt in bits 3:0 and 15:14; expcnt (6:4) and lgkmcnt (11:8) at their maxima
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ void lds_copy16(const void *g, uint8_t *lds)
{
    __builtin_amdgcn_global_load_lds(g, (__attribute__((address_space(3))) void *)lds, 16, 0, 0);
}

template <int NS>
__global__ __launch_bounds__(NT) void gemm_bf16_down_kernel(int H, int I, int E, WSet w,
                                                            const uint16_t *__restrict__ asrc, Plan p,
                                                            uint16_t *__restrict__ out)
{
    constexpr int kRow = 64, kTile = 256 * kRow, kStage = 2 * kTile;  // bytes
    extern __shared__ __attribute__((aligned(16))) uint8_t ring[];     // NS * kStage
    const int n_tiles = (H + BN - 1) / BN;
    int item, nb;
    xcd_map(blockIdx.x, n_tiles, item, nb);
    if (item >= p.meta[1]) return;
    const int code = p.items[item];
    const int u = code >> 16, mtile = code & 0xffff;
    const int e = p.touched[u], base = p.tbase[u], cnt = p.tcount[u];
    const bool sh = (e == E);
    const int m0 = mtile * BM;
    const int valid = min(BM, cnt - m0);
    const int K = I;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
    const int wm = wave >> 2, wn = wave & 3;

    // Copies: wave w fills A rows (h rows of the item's slots) and B rows (down rows)
    // 16 w .. 16 w + 15 of every stage; lane l takes
    // row 16 w + l / 4, slot l % 4, i.e. logical chunk (l % 4) ^ ((row >> 1) & 3).
    const int crow = 16 * wave + (lane >> 2);
    const int cchunk = (lane & 3) ^ ((crow >> 1) & 3);
    const uint16_t *ap_;
    const uint16_t *bp_;
    {
        const int ri = min(crow, valid - 1);
        ap_ = asrc + (size_t)(base + m0 + ri) * I + 8 * cchunk;
        const int n = min(nb * BN + crow, H - 1);
        const size_t mb = (size_t)H * I;
        bp_ = reinterpret_cast<const uint16_t *>(sh ? w.down.shared : w.down.routed) + (sh ? 0 : (size_t)e * mb) +
              (size_t)n * K + 8 * cchunk;
    }
    uint8_t *const cdst = ring + 1024 * wave;  // + stage * kStage (+ kTile for B)
    auto issue = [&](int kt) {
        uint8_t *st = cdst + (size_t)(kt % NS) * kStage;
        lds_copy16(ap_ + 32 * kt, st);
        lds_copy16(bp_ + 32 * kt, st + kTile);
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Fragment reads: A row wm*64 + 16 ms + r and B row wn*64 + 16 ns + r, logical chunk g.
    const int fslot = 16 * (g ^ ((r >> 1) & 3));
    const int aoff = (wm * 64 + r) * kRow + fslot, boff = kTile + (wn * 64 + r) * kRow + fslot;
    const int nk = K / 32;  // >= 4
#pragma unroll
    for (int s = 0; s < NS - 1; s++)
        if (s < nk) issue(s);
    for (int kt = 0; kt < nk; kt++) {
        // Stage kt has landed for this wave once at most min(NS - 2, nk - 1 - kt) later
        // stages (two copies each) are still in flight; the barrier makes it true for every
        // wave and frees the slot read in iteration kt - 1, which stage kt + NS - 1 refills.
        const int later = nk - 1 - kt;
        if (later >= NS - 2) wait_vmcnt<2 * (NS - 2)>();
        else if (NS > 4 && later == 2) wait_vmcnt<4>();
        else if (later == 1) wait_vmcnt<2>();
        else wait_vmcnt<0>();
        // the barrier orders LDS accesses for the hardware; the signal fences keep the
        // compiler from moving fragment reads or ring copies across it
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (kt + NS - 1 < nk) issue(kt + NS - 1);
        const uint8_t *st = ring + (size_t)(kt % NS) * kStage;
        bf16x8 af[4], bfr[4];
#pragma unroll
        for (int ms = 0; ms < 4; ms++) af[ms] = as_bf16x8(*reinterpret_cast<const u32x4 *>(st + aoff + ms * 16 * kRow));
#pragma unroll
        for (int ns = 0; ns < 4; ns++) bfr[ns] = as_bf16x8(*reinterpret_cast<const u32x4 *>(st + boff + ns * 16 * kRow));
#pragma unroll
        for (int ms = 0; ms < 4; ms++)
#pragma unroll
            for (int ns = 0; ns < 4; ns++) acc[ms][ns] = mfma16x16x32(af[ms], bfr[ns], acc[ms][ns]);
    }

    // Epilogue.  acc[ms][ns][i] = D[row = wm*64 + ms*16 + 4g + i][brow = wn*64 + ns*16 + r].
#pragma unroll
    for (int ms = 0; ms < 4; ms++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int row = wm * 64 + ms * 16 + 4 * g + i;
            if (row >= valid) continue;
            const size_t slot = (size_t)(base + m0 + row);
#pragma unroll
            for (int ns = 0; ns < 4; ns++) {
                const int col = nb * BN + wn * 64 + ns * 16 + r;
                if (col < H) out[slot * H + col] = (uint16_t)f2bf(acc[ms][ns][i]);
            }
        }
    }
}

// ---------------------------------------------------------------- bf16: 64-wide K stages
// The 16-wave kernel with K stages of 64 (128-byte row pieces, whole cache lines): a copy
// instruction fetches 8 rows x 128 B, so the same bytes take half as many L2 requests as
// with 64-byte pieces, whose kernel spent 61 % of its cycles with the CU's L1 stalled on
// pending requests (counters); this one measured 5 % faster.  Two stages of 64 KB: the
// copies of stage kt + 1 fly while stage kt is multiplied.
// Row R keeps its 16-byte chunk c at slot c ^ (R & 7), conflict-free for the fragment reads
// (lane (g, r): row r, chunk 4 j + g in K half j).  K must be a multiple of 64.
template <int MODE>
__global__ __launch_bounds__(NT) void gemm_bf16k64_kernel(int T, int H, int I, int E, int k, WSet w,
                                                          const uint16_t *__restrict__ asrc,
                                                          const int32_t *__restrict__ sa, Plan p,
                                                          uint16_t *__restrict__ out)
{
    constexpr int kRow = 128, kTile = 256 * kRow, kStage = 2 * kTile;  // bytes
    extern __shared__ __attribute__((aligned(16))) uint8_t ring[];      // 2 * kStage
    const int N = MODE == 0 ? 2 * I : H;
    const int n_tiles = (N + BN - 1) / BN;
    int item, nb;
    xcd_map(blockIdx.x, n_tiles, item, nb);
    if (item >= p.meta[1]) return;
    const int code = p.items[item];
    const int u = code >> 16, mtile = code & 0xffff;
    const int e = p.touched[u], base = p.tbase[u], cnt = p.tcount[u];
    const bool sh = (e == E);
    const int m0 = mtile * BM;
    const int valid = min(BM, cnt - m0);
    const int K = MODE == 0 ? H : I;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
    const int wm = wave >> 2, wn = wave & 3;

    // Copies: wave w fills A rows and B rows 16 w + 8 c + l / 8 (c < 2) of every stage,
    // slot l % 8, i.e. logical chunk (l % 8) ^ (row & 7).
    const uint16_t *ap_[2];
    const uint16_t *bp_[2];
#pragma unroll
    for (int c = 0; c < 2; c++) {
        const int crow = 16 * wave + 8 * c + (lane >> 3);
        const int cchunk = (lane & 7) ^ (crow & 7);
        const int ri = min(crow, valid - 1);
        if (MODE == 0) {
            const int tok = sh ? base - T * k + m0 + ri : sa[base + m0 + ri] / k;
            ap_[c] = asrc + (size_t)tok * H + 8 * cchunk;
        } else {
            ap_[c] = asrc + (size_t)(base + m0 + ri) * I + 8 * cchunk;
        }
        const WMat *mat;
        int n;
        if (MODE == 0) {  // each 64-row wave column: 32 gate rows, then the same 32 up rows
            const int wcol = crow >> 6, within = crow & 63;
            mat = (within >> 5) ? &w.up : &w.gate;
            n = min(nb * (BN / 2) + wcol * 32 + (within & 31), I - 1);
        } else {
            mat = &w.down;
            n = min(nb * BN + crow, H - 1);
        }
        const size_t mb = (size_t)H * I;
        bp_[c] = reinterpret_cast<const uint16_t *>(sh ? mat->shared : mat->routed) + (sh ? 0 : (size_t)e * mb) +
                 (size_t)n * K + 8 * cchunk;
    }
    uint8_t *const cdst = ring + 2048 * wave;  // + stage * kStage (+ kTile for B)
    auto issue = [&](int kt) {
        uint8_t *st = cdst + (size_t)(kt & 1) * kStage;
        lds_copy16(ap_[0] + 64 * kt, st);
        lds_copy16(ap_[1] + 64 * kt, st + 1024);
        lds_copy16(bp_[0] + 64 * kt, st + kTile);
        lds_copy16(bp_[1] + 64 * kt, st + kTile + 1024);
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Fragment reads: A row wm*64 + 16 ms + r and B row wn*64 + 16 ns + r, logical chunk
    // 4 j + g for the K half j of the stage.
    const int aoff = (wm * 64 + r) * kRow, boff = kTile + (wn * 64 + r) * kRow;
    const int fs0 = 16 * (g ^ (r & 7)), fs1 = 16 * ((4 + g) ^ (r & 7));
    const int nk = K / 64;
    issue(0);
    for (int kt = 0; kt < nk; kt++) {
        // stage kt is the only one in flight: once it has landed for every wave, the slot
        // read in iteration kt - 1 is free for stage kt + 1
        wait_vmcnt<0>();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (kt + 1 < nk) issue(kt + 1);
        const uint8_t *st = ring + (size_t)(kt & 1) * kStage;
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int fs = j ? fs1 : fs0;
            bf16x8 af[4], bfr[4];
#pragma unroll
            for (int ms = 0; ms < 4; ms++) af[ms] = as_bf16x8(*reinterpret_cast<const u32x4 *>(st + aoff + ms * 16 * kRow + fs));
#pragma unroll
            for (int ns = 0; ns < 4; ns++) bfr[ns] = as_bf16x8(*reinterpret_cast<const u32x4 *>(st + boff + ns * 16 * kRow + fs));
#pragma unroll
            for (int ms = 0; ms < 4; ms++)
#pragma unroll
                for (int ns = 0; ns < 4; ns++) acc[ms][ns] = mfma16x16x32(af[ms], bfr[ns], acc[ms][ns]);
        }
    }

    // Epilogue.  acc[ms][ns][i] = D[row = wm*64 + ms*16 + 4g + i][brow = wn*64 + ns*16 + r].
#pragma unroll
    for (int ms = 0; ms < 4; ms++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int row = wm * 64 + ms * 16 + 4 * g + i;
            if (row >= valid) continue;
            const size_t slot = (size_t)(base + m0 + row);
            if (MODE == 0) {
#pragma unroll
                for (int ns = 0; ns < 2; ns++) {
                    const int col = nb * (BN / 2) + wn * 32 + ns * 16 + r;
                    if (col < I) out[slot * I + col] = (uint16_t)f2bf(silu(acc[ms][ns][i]) * acc[ms][ns + 2][i]);
                }
            } else {
#pragma unroll
                for (int ns = 0; ns < 4; ns++) {
                    const int col = nb * BN + wn * 64 + ns * 16 + r;
                    if (col < H) out[slot * H + col] = (uint16_t)f2bf(acc[ms][ns][i]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------- NVFP4 / INT4: codes to LDS once
// The same 256 x 256 tiles as the bf16 kernels, here with 8 waves (two per SIMD) of
// 64 slots x 128 B rows each, so the registers hold what the 4-bit path adds.  The tokens
// (A) come through a 5-stage ring of 32-wide K stages filled HBM -> LDS by
// global_load_lds_dwordx4, four stages ahead.  The weights arrive as their 4-bit codes:
// per stage a thread loads 16 codes of one row (8 bytes) and their scale into a 4-slot
// register ring, four stages ahead as well, so the weight bytes in flight are a quarter of
// bf16's; when the stage comes up it turns them into 16 exact bf16 values (NVFP4: e2m1
// times the E4M3 block scale; INT4: q times the bf16 group scale, rounded once, as in
// grouped_gemm_kernel's staging) and writes them to a double-buffered bf16 B stage in the
// ring's swizzled layout, where every wave reads its fragments.  Copies and loads go out
// per stage s as A(s) (two per wave), codes(s), scale(s), so with stage s + 4 issued in
// iteration s, stage s has landed once at most twelve are in flight.  The loop runs four
// stages per trip (the register slots stay fixed) and its steady state has no branches.
constexpr int NTQ = 512;
template <int MODE, int FMT>
__global__ __launch_bounds__(NTQ) void gemm_q4_kernel(int T, int H, int I, int E, int k, WSet w,
                                                      const uint16_t *__restrict__ asrc,
                                                      const int32_t *__restrict__ sa, Plan p,
                                                      uint16_t *__restrict__ out)
{
    constexpr int kRow = 64, kStage = 256 * kRow;  // bytes: one A stage, one B stage
    constexpr int NSA = 5;                         // A ring stages
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // NSA A stages + 2 B stages
    uint8_t *const bbuf = lds + NSA * kStage;
    const int N = MODE == 0 ? 2 * I : H;
    const int n_tiles = (N + BN - 1) / BN;
    int item, nb;
    xcd_map(blockIdx.x, n_tiles, item, nb);
    if (item >= p.meta[1]) return;
    const int code = p.items[item];
    const int u = code >> 16, mtile = code & 0xffff;
    const int e = p.touched[u], base = p.tbase[u], cnt = p.tcount[u];
    const bool sh = (e == E);
    const int m0 = mtile * BM;
    const int valid = min(BM, cnt - m0);
    const int K = MODE == 0 ? H : I;
    const int nk = K / 32;  // a multiple of 4
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
    const int wm = wave >> 1, wn = wave & 1;

    // A copies: wave w fills rows 32 w + 16 c + l / 4 (c < 2) of every stage, slot l % 4,
    // i.e. logical chunk (l % 4) ^ ((row >> 1) & 3).  Rows past the tile repeat the last.
    const uint16_t *ap_[2];
#pragma unroll
    for (int c = 0; c < 2; c++) {
        const int crow = 32 * wave + 16 * c + (lane >> 2);
        const int cchunk = (lane & 3) ^ ((crow >> 1) & 3);
        const int ri = min(crow, valid - 1);
        if (MODE == 0) {
            const int tok = sh ? base - T * k + m0 + ri : sa[base + m0 + ri] / k;
            ap_[c] = asrc + (size_t)tok * H + 8 * cchunk;
        } else {
            ap_[c] = asrc + (size_t)(base + m0 + ri) * I + 8 * cchunk;
        }
    }
    uint8_t *const cdst = lds + 2048 * wave;  // + slot * kStage
    auto issue_a = [&](int kt, int slot) {
        lds_copy16(ap_[0] + 32 * kt, cdst + slot * kStage);
        lds_copy16(ap_[1] + 32 * kt, cdst + slot * kStage + 1024);
    };

    // Codes: thread tid takes B row bro = tid / 2 of the tile and k 16 hq .. 16 hq + 15 of
    // every stage (hq = tid % 2): logical chunks 2 hq and 2 hq + 1 of row bro.  Gate/up:
    // each 128-row wave column holds 64 gate rows, then the same 64 up rows.
    const int bro = tid >> 1, hq = tid & 1;
    const uint8_t *qp;
    const uint8_t *sp;
    {
        const WMat *mat;
        int n;
        if (MODE == 0) {
            const int wcol = bro >> 7, within = bro & 127;
            mat = (within >> 6) ? &w.up : &w.gate;
            n = min(nb * (BN / 2) + wcol * 64 + (within & 63), I - 1);
        } else {
            mat = &w.down;
            n = min(nb * BN + bro, H - 1);
        }
        const size_t mb = (size_t)H * I / 2, srow = scale_row_bytes(FMT, K), sb = (size_t)(H * I / K) * srow;
        qp = (sh ? mat->shared : mat->routed + (size_t)e * mb) + (size_t)n * (K / 2) + 8 * hq;
        // NVFP4: block 2 s + hq of the row (16 codes); INT4: group s / 4 (bf16)
        sp = (sh ? mat->sf_shared : mat->sf_routed + (size_t)e * sb) + (size_t)n * srow + (FMT == 1 ? hq : 0);
    }
    u32x2 cq[4];
    uint32_t cs[4];
    auto issue_b = [&](int kt, int slot) {
        cq[slot] = *reinterpret_cast<const u32x2 *>(qp + 16 * kt);
        cs[slot] = FMT == 1 ? (uint32_t)sp[2 * kt] : (uint32_t)reinterpret_cast<const uint16_t *>(sp)[kt >> 2];
    };
    auto dequant_b = [&](int kt, int slot) {  // stage kt's codes -> bf16 B buffer kt % 2
        const float sc = FMT == 1 ? e4m3_to_f32(cs[slot]) : bf2f(cs[slot]);
        uint8_t *row = bbuf + (kt & 1) * kStage + bro * kRow;
        const int sw = (bro >> 1) & 3;
#pragma unroll
        for (int h2 = 0; h2 < 2; h2++) {
            const uint32_t qw = cq[slot][h2];
            const u32x4 v = FMT == 1 ? dequant8(qw, sc) : dequant8_int4(qw, sc);
            *reinterpret_cast<u32x4 *>(row + 16 * ((2 * hq + h2) ^ sw)) = v;
        }
    };

    f32x4 acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 8; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Fragment reads: A row wm*64 + 16 ms + r and B row wn*128 + 16 ns + r, logical chunk g.
    const int fslot = 16 * (g ^ ((r >> 1) & 3));
    const int aoff = (wm * 64 + r) * kRow + fslot, boff = (wn * 128 + r) * kRow + fslot;
    auto compute = [&](int kt) {
        const uint8_t *as = lds + (kt % NSA) * kStage + aoff;
        const uint8_t *bs = bbuf + (kt & 1) * kStage + boff;
        bf16x8 af[4];
#pragma unroll
        for (int ms = 0; ms < 4; ms++) af[ms] = as_bf16x8(*reinterpret_cast<const u32x4 *>(as + ms * 16 * kRow));
#pragma unroll
        for (int ns = 0; ns < 8; ns++) {
            const bf16x8 bfr = as_bf16x8(*reinterpret_cast<const u32x4 *>(bs + ns * 16 * kRow));
#pragma unroll
            for (int ms = 0; ms < 4; ms++) acc[ms][ns] = mfma16x16x32(af[ms], bfr, acc[ms][ns]);
        }
    };
    // Iteration kt: stage kt landed (A in its ring slot, codes in register slot kt % 4);
    // its codes become bf16 in B buffer kt % 2 (last read in iteration kt - 2, before the
    // previous barrier); the barrier makes A and B of stage kt visible and frees A slot
    // (kt + 4) % 5 (read in kt - 1), which stage kt + 4 refills together with the codes
    // slot just used; then the MFMAs.
    auto step = [&](int kt, int cslot, bool more) {
        dequant_b(kt, cslot);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (more) {
            issue_a(kt + 4, (kt + 4) % NSA);
            issue_b(kt + 4, cslot);
        }
        compute(kt);
    };

#pragma unroll
    for (int s0 = 0; s0 < 4; s0++) {
        issue_a(s0, s0);
        issue_b(s0, s0);
    }
    int kt = 0;
    for (; kt + 8 <= nk; kt += 4) {  // every stage of this trip issues stage + 4
        wait_vmcnt<12>();
        step(kt, 0, true);
        wait_vmcnt<12>();
        step(kt + 1, 1, true);
        wait_vmcnt<12>();
        step(kt + 2, 2, true);
        wait_vmcnt<12>();
        step(kt + 3, 3, true);
    }
    // last four stages: nothing more to issue, so fewer copies are in flight at each wait
    wait_vmcnt<12>();
    step(kt, 0, false);
    wait_vmcnt<8>();
    step(kt + 1, 1, false);
    wait_vmcnt<4>();
    step(kt + 2, 2, false);
    wait_vmcnt<0>();
    step(kt + 3, 3, false);

    // Epilogue.  acc[ms][ns][i] = D[row = wm*64 + ms*16 + 4g + i][brow = wn*128 + ns*16 + r].
    float tsg = 1.f, tsu = 1.f, tsd = 1.f;  // NVFP4 tensor scales
    if (FMT == 1) {
        tsg = sh ? *w.gate.ts_shared : w.gate.ts_routed[e];
        tsu = sh ? *w.up.ts_shared : w.up.ts_routed[e];
        tsd = sh ? *w.down.ts_shared : w.down.ts_routed[e];
    }
#pragma unroll
    for (int ms = 0; ms < 4; ms++) {
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int row = wm * 64 + ms * 16 + 4 * g + i;
            if (row >= valid) continue;
            const size_t slot = (size_t)(base + m0 + row);
            if (MODE == 0) {
#pragma unroll
                for (int ns = 0; ns < 4; ns++) {
                    const int col = nb * (BN / 2) + wn * 64 + ns * 16 + r;
                    const float gv = acc[ms][ns][i] * tsg, uv = acc[ms][ns + 4][i] * tsu;
                    if (col < I) out[slot * I + col] = (uint16_t)f2bf(silu(gv) * uv);
                }
            } else {
#pragma unroll
                for (int ns = 0; ns < 8; ns++) {
                    const int col = nb * BN + wn * 128 + ns * 16 + r;
                    if (col < H) out[slot * H + col] = (uint16_t)f2bf(acc[ms][ns][i] * tsd);
                }
            }
        }
    }
}

// y[t][n] = bf16(o[T*k + t][n] + sum_j w[t][j] * o[ap[t*k + j]][n]); 8 columns per thread.
// Slots outside [0, T k) (assignments dropped for an out-of-range expert id) are skipped.
__global__ __launch_bounds__(256) void combine_kernel(int T, int H, int k, int S,
                                                      const uint16_t *__restrict__ o,
                                                      const float *__restrict__ topk_w,
                                                      const int32_t *__restrict__ ap,
                                                      uint16_t *__restrict__ y)
{
    const int per_tok = H / 8;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= (int64_t)T * per_tok) return;
    const int t = (int)(gid / per_tok), c = (int)(gid % per_tok) * 8;
    float acc[8];
    if (S) {
        u32x4 v = ld16g(o + ((size_t)T * k + t) * H + c);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            acc[2 * i] = bf2f(v[i] & 0xffffu);
            acc[2 * i + 1] = bf2f(v[i] >> 16);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; i++) acc[i] = 0.f;
    }
    for (int j = 0; j < k; j++) {
        const int sl = ap[t * k + j];
        if (sl < 0 || sl >= T * k) continue;  // a dropped assignment (expert id out of range) has no slot
        const float wj = topk_w[t * k + j];
        u32x4 v = ld16g(o + (size_t)sl * H + c);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            acc[2 * i] += wj * bf2f(v[i] & 0xffffu);
            acc[2 * i + 1] += wj * bf2f(v[i] >> 16);
        }
    }
    u32x4 outv;
#pragma unroll
    for (int i = 0; i < 4; i++) outv[i] = f2bf(acc[2 * i]) | (f2bf(acc[2 * i + 1]) << 16);
    *reinterpret_cast<u32x4 *>(y + (size_t)t * H + c) = outv;
}

}  // namespace

hipError_t launch_gemm_forward(const Shape &s, const WSet &w, int64_t T, const uint16_t *x,
                               const float *topk_w, const int32_t *sa, const int32_t *ap,
                               const Plan &plan, uint16_t *h, uint16_t *o, uint16_t *y,
                               hipStream_t st)
{
    const int64_t slots = T * s.k + T * s.S;
    const int64_t max_items = (slots + kGemmBM - 1) / kGemmBM + s.E + s.S;
    const int64_t item_slots = (max_items + kXcds - 1) / kXcds * kXcds;
    const unsigned g1 = (unsigned)(item_slots * ((2 * s.I + BN - 1) / BN));
    const unsigned g2 = (unsigned)(item_slots * ((s.H + BN - 1) / BN));
    if (w.fmt == 0) {
        // 64-wide K stages (H is a multiple of 64); the down pass with I % 64 == 32 takes the
        // 32-wide ring
        constexpr size_t lds32 = (size_t)kRingStages * 2 * 256 * 64, lds64 = (size_t)2 * 2 * 256 * 128;
        gemm_bf16k64_kernel<0><<<g1, NT, lds64, st>>>((int)T, s.H, s.I, s.E, s.k, w, x, sa, plan, h);
        if (s.I % 64 == 0)
            gemm_bf16k64_kernel<1><<<g2, NT, lds64, st>>>((int)T, s.H, s.I, s.E, s.k, w, h, sa, plan, o);
        else
            gemm_bf16_down_kernel<kRingStages><<<g2, NT, lds32, st>>>(s.H, s.I, s.E, w, h, plan, o);
    } else {
        // 4-bit weights: the code ring needs K in whole trips of four 32-wide stages (INT4
        // always has them: its scale groups are 128 columns); NVFP4 with K % 128 != 0 takes
        // the register-staged kernel
        constexpr size_t qlds = (size_t)(5 + 2) * 256 * 64;
        const bool ring_gu = s.H % 128 == 0, ring_dn = s.I % 128 == 0;
        if (w.fmt == 1) {
            if (ring_gu) gemm_q4_kernel<0, 1><<<g1, NTQ, qlds, st>>>((int)T, s.H, s.I, s.E, s.k, w, x, sa, plan, h);
            else grouped_gemm_kernel<0><<<g1, NT, 0, st>>>((int)T, s.H, s.I, s.E, s.k, w, x, sa, plan, h);
            if (ring_dn) gemm_q4_kernel<1, 1><<<g2, NTQ, qlds, st>>>((int)T, s.H, s.I, s.E, s.k, w, h, sa, plan, o);
            else grouped_gemm_kernel<1><<<g2, NT, 0, st>>>((int)T, s.H, s.I, s.E, s.k, w, h, sa, plan, o);
        } else {
            gemm_q4_kernel<0, 2><<<g1, NTQ, qlds, st>>>((int)T, s.H, s.I, s.E, s.k, w, x, sa, plan, h);
            gemm_q4_kernel<1, 2><<<g2, NTQ, qlds, st>>>((int)T, s.H, s.I, s.E, s.k, w, h, sa, plan, o);
        }
    }
    const int64_t nthreads = T * (s.H / 8);
    combine_kernel<<<(unsigned)((nthreads + 255) / 256), 256, 0, st>>>((int)T, s.H, s.k, s.S, o,
                                                                       topk_w, ap, y);
    return hipGetLastError();
}

}  // namespace flint
