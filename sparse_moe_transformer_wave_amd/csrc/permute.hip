// permute.hip -- grouping of the T*k (token, slot) assignments by expert, and the
// per-expert work plan the expert kernels consume.
//
// The grouping is the data movement a fused MoE kernel needs (recipes.vllm.ai
// "RecursiveSI/flint", Overview, "fused MoE"): counts, exclusive offsets, the stable
// order (ascending assignment index inside each expert) and its inverse.  All integer.
#include "common.h"

namespace flint {

// Exclusive scan of in[0..n) into out[0..n], out[n] = total; n <= 320; wave 0 only.
__device__ void wave0_exclusive_scan(const int *in, int *out, int n)
{
    const int lane = threadIdx.x & 63;
    int loc[5];
    int s = 0;
#pragma unroll
    for (int i = 0; i < 5; i++) {
        int idx = lane * 5 + i;
        loc[i] = idx < n ? in[idx] : 0;
        s += loc[i];
    }
    int inc = s;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int o = __shfl_up(inc, off, 64);
        if (lane >= off) inc += o;
    }
    int ex = inc - s;
#pragma unroll
    for (int i = 0; i < 5; i++) {
        int idx = lane * 5 + i;
        if (idx < n) out[idx] = ex;
        ex += loc[i];
    }
    if (lane == 63) out[n] = inc;
}

struct PlanScratch {
    int flag[320], idx[321], nt[320], base[321];
};

// Build the plan from per-expert counts and offsets held in LDS.  Touched experts are
// listed in ascending id, the shared expert (id E, all T tokens) last.
__device__ void build_plan(int T, int E, int k, int S, int H, const int *cnt, const int *off,
                           const Plan &p, PlanScratch &ps)
{
    const int tid = threadIdx.x, bd = blockDim.x;
    const int n = E + S;
    for (int e = tid; e < n; e += bd) ps.flag[e] = (e < E) ? (cnt[e] > 0) : (T > 0);
    __syncthreads();
    if (tid < 64) wave0_exclusive_scan(ps.flag, ps.idx, n);
    __syncthreads();
    const int nT = ps.idx[n];
    for (int e = tid; e < n; e += bd) {
        if (!ps.flag[e]) continue;
        int u = ps.idx[e];
        int rows = (e < E) ? cnt[e] : T;
        p.touched[u] = e;
        p.tbase[u] = (e < E) ? off[e] : T * k;
        p.tcount[u] = rows;
        ps.nt[u] = (rows + kGemmBM - 1) / kGemmBM;
    }
    __syncthreads();
    if (tid < 64) wave0_exclusive_scan(ps.nt, ps.base, nT);
    __syncthreads();
    for (int u = tid; u < nT; u += bd)
        for (int m = 0; m < ps.nt[u]; m++) p.items[ps.base[u] + m] = (u << 16) | m;
    if (tid == 0) {
        p.meta[0] = nT;
        p.meta[1] = ps.base[nT];
    }
    for (int i = tid; i < H / 16; i += bd) p.counters[i] = 0;
}

// Grouping of n assignments by expert, by one workgroup of 1024 threads.  Assignments are
// processed in chunks of 1024 in ascending order; inside a chunk, a lane's rank among
// equal experts of lower lanes comes from eight ballots over the expert id bits, and
// per-wave counts in LDS give the offsets of earlier waves.  `cursor` carries each
// expert's fill level across chunks, which makes the order stable.  Leaves counts and
// exclusive offsets in cnt/off (LDS).
struct GroupScratch {
    int cnt[256];
    int off[257];
    int cursor[256];
    int wave_cnt[16][256];
};

__device__ void group_by_expert(int n, int E, const int32_t *ids, GroupScratch &g,
                                int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                int32_t *__restrict__ sa, int32_t *__restrict__ ap)
{
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    if (tid < 256) g.cnt[tid] = 0;
    __syncthreads();
    for (int a = tid; a < n; a += 1024) {
        int e = ids[a];
        if (e >= 0 && e < E) atomicAdd(&g.cnt[e], 1);
    }
    __syncthreads();
    if (tid < 64) wave0_exclusive_scan(g.cnt, g.off, E);
    __syncthreads();
    for (int e = tid; e < E; e += 1024) {
        counts[e] = g.cnt[e];
        offsets[e] = g.off[e];
        g.cursor[e] = g.off[e];
    }
    if (tid == 0) offsets[E] = g.off[E];
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = 0; base < n; base += 1024) {
        const int a = base + tid;
        int e = (a < n) ? ids[a] : -1;
        const bool valid = (e >= 0 && e < E);
        for (int i = tid; i < 16 * 256; i += 1024) (&g.wave_cnt[0][0])[i] = 0;
        __syncthreads();
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; b++) {
            bool bit = valid && ((e >> b) & 1);
            uint64_t vote = __ballot(bit);
            peers &= bit ? vote : ~vote;
        }
        const int rank = __popcll(peers & lt_mask);
        if (valid && rank == 0) g.wave_cnt[wv][e] = __popcll(peers);
        __syncthreads();
        if (valid) {
            int before = 0;
            for (int w = 0; w < wv; w++) before += g.wave_cnt[w][e];
            int pos = g.cursor[e] + before + rank;
            sa[pos] = a;
            ap[a] = pos;
        }
        __syncthreads();
        for (int x = tid; x < E; x += 1024) {
            int tot = 0;
            for (int w = 0; w < 16; w++) tot += g.wave_cnt[w][x];
            g.cursor[x] += tot;
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(1024) void permute_kernel(int T, int E, int k, int S, int H,
                                                       const int32_t *__restrict__ ids,
                                                       int32_t *__restrict__ counts,
                                                       int32_t *__restrict__ offsets,
                                                       int32_t *__restrict__ sa,
                                                       int32_t *__restrict__ ap, Plan plan,
                                                       int with_plan)
{
    __shared__ GroupScratch g;
    __shared__ PlanScratch ps;
    group_by_expert(T * k, E, ids, g, counts, offsets, sa, ap);
    if (with_plan) build_plan(T, E, k, S, H, g.cnt, g.off, plan, ps);
}

// Small batches (T <= 32): top-k of every token (one wave per token), the grouping and
// the plan in a single workgroup, so routing costs one launch after the router.
__global__ __launch_bounds__(1024) void select_permute_kernel(
    int T, int E, int k, int S, int H, int renorm, const float *__restrict__ logits,
    int32_t *__restrict__ ids, float *__restrict__ wout, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sa, int32_t *__restrict__ ap, Plan plan)
{
    __shared__ GroupScratch g;
    __shared__ PlanScratch ps;
    __shared__ int32_t s_ids[kGemvMaxT * 8];
    __shared__ float s_w[kGemvMaxT * 8];
    const int wv = threadIdx.x >> 6;
    for (int t = wv; t < T; t += 16)
        topk_token(logits + (size_t)t * E, E, k, renorm, s_ids + t * k, s_w + t * k);
    __syncthreads();
    for (int a = threadIdx.x; a < T * k; a += 1024) {
        ids[a] = s_ids[a];
        wout[a] = s_w[a];
    }
    group_by_expert(T * k, E, s_ids, g, counts, offsets, sa, ap);
    build_plan(T, E, k, S, H, g.cnt, g.off, plan, ps);
}

hipError_t launch_select_permute(const Shape &s, int64_t T, const float *logits, int32_t *ids,
                                 float *w, int32_t *counts, int32_t *offsets, int32_t *sa,
                                 int32_t *ap, const Plan &plan, hipStream_t st)
{
    select_permute_kernel<<<1, 1024, 0, st>>>((int)T, s.E, s.k, s.S, s.H, s.renorm, logits, ids,
                                              w, counts, offsets, sa, ap, plan);
    return hipGetLastError();
}

// ---- many assignments (prefill): three launches instead of one serial workgroup ----
// (1) per-block histograms of 1024 assignments, (2) one workgroup turns them into expert
// offsets and per-(block, expert) bases, (3) each block places its assignments: base of
// its (block, expert) + rank among equal experts of lower lanes in the block.  Blocks
// are ordered like the assignments, so the grouping stays stable.
__global__ __launch_bounds__(1024) void perm_hist_kernel(int n, int E, const int32_t *__restrict__ ids,
                                                         int32_t *__restrict__ hist)
{
    __shared__ int cnt[256];
    const int tid = threadIdx.x;
    if (tid < 256) cnt[tid] = 0;
    __syncthreads();
    const int a = blockIdx.x * 1024 + tid;
    if (a < n) {
        const int e = ids[a];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    if (tid < E) hist[(size_t)blockIdx.x * E + tid] = cnt[tid];
}

__global__ __launch_bounds__(256) void perm_scan_kernel(int T, int E, int k, int S, int H, int nb,
                                                        int32_t *__restrict__ hist,
                                                        int32_t *__restrict__ counts,
                                                        int32_t *__restrict__ offsets, Plan plan,
                                                        int with_plan)
{
    __shared__ int cnt[256];
    __shared__ int off[257];
    __shared__ PlanScratch ps;
    const int e = threadIdx.x;
    int tot = 0;
    if (e < E)
        for (int b = 0; b < nb; b++) {
            const int c = hist[(size_t)b * E + e];
            hist[(size_t)b * E + e] = tot;  // exclusive prefix over blocks
            tot += c;
        }
    if (e < 256) cnt[e] = (e < E) ? tot : 0;
    __syncthreads();
    if (threadIdx.x < 64) wave0_exclusive_scan(cnt, off, E);
    __syncthreads();
    if (e < E) {
        counts[e] = cnt[e];
        offsets[e] = off[e];
        for (int b = 0; b < nb; b++) hist[(size_t)b * E + e] += off[e];
    }
    if (e == 0) offsets[E] = off[E];
    if (with_plan) build_plan(T, E, k, S, H, cnt, off, plan, ps);
}

__global__ __launch_bounds__(1024) void perm_scatter_kernel(int n, int E, const int32_t *__restrict__ ids,
                                                            const int32_t *__restrict__ base,
                                                            int32_t *__restrict__ sa,
                                                            int32_t *__restrict__ ap)
{
    __shared__ int wave_cnt[16][256];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int a = blockIdx.x * 1024 + tid;
    const int e = (a < n) ? ids[a] : -1;
    const bool valid = (e >= 0 && e < E);
    for (int i = tid; i < 16 * 256; i += 1024) (&wave_cnt[0][0])[i] = 0;
    __syncthreads();
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; b++) {
        const bool bit = valid && ((e >> b) & 1);
        const uint64_t vote = __ballot(bit);
        peers &= bit ? vote : ~vote;
    }
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(peers & lt);
    if (valid && rank == 0) wave_cnt[wv][e] = __popcll(peers);
    __syncthreads();
    if (valid) {
        int before = 0;
        for (int w = 0; w < wv; w++) before += wave_cnt[w][e];
        const int pos = base[(size_t)blockIdx.x * E + e] + before + rank;
        sa[pos] = a;
        ap[a] = pos;
    }
}

constexpr int kSingleBlockPermuteMax = 4096;

hipError_t launch_permute(const Shape &s, int64_t T, const int32_t *ids, int32_t *counts,
                          int32_t *offsets, int32_t *sa, int32_t *ap, const Plan *plan,
                          int32_t *hist, hipStream_t st)
{
    Plan p = plan ? *plan : Plan{};
    const int n = (int)(T * s.k);
    if (n <= kSingleBlockPermuteMax || hist == nullptr) {
        permute_kernel<<<1, 1024, 0, st>>>((int)T, s.E, s.k, s.S, s.H, ids, counts, offsets, sa, ap,
                                           p, plan ? 1 : 0);
        return hipGetLastError();
    }
    const int nb = (n + 1023) / 1024;
    perm_hist_kernel<<<nb, 1024, 0, st>>>(n, s.E, ids, hist);
    perm_scan_kernel<<<1, 256, 0, st>>>((int)T, s.E, s.k, s.S, s.H, nb, hist, counts, offsets, p,
                                        plan ? 1 : 0);
    perm_scatter_kernel<<<nb, 1024, 0, st>>>(n, s.E, ids, hist, sa, ap);
    return hipGetLastError();
}

// Plan from caller-provided offsets (forward called on its own).
__global__ __launch_bounds__(256) void plan_kernel(int T, int E, int k, int S, int H,
                                                   const int32_t *__restrict__ offsets, Plan plan)
{
    __shared__ int cnt[256];
    __shared__ int off[257];
    __shared__ PlanScratch ps;
    for (int e = threadIdx.x; e <= E; e += blockDim.x) off[e] = offsets[e];
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = off[e + 1] - off[e];
    __syncthreads();
    build_plan(T, E, k, S, H, cnt, off, plan, ps);
}

hipError_t launch_plan(const Shape &s, int64_t T, const int32_t *offsets, const Plan &plan,
                       hipStream_t st)
{
    plan_kernel<<<1, 256, 0, st>>>((int)T, s.E, s.k, s.S, s.H, offsets, plan);
    return hipGetLastError();
}

}  // namespace flint
