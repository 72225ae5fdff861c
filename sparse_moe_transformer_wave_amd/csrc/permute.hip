// permute.hip -- grouping of the T*k (token, slot) assignments by expert, and the
// per-expert work plan the expert kernels consume.
//
// The grouping is the data movement a fused MoE kernel needs (recipes.vllm.ai
// "RecursiveSI/flint", Overview, "fused MoE"): counts, exclusive offsets, the stable
// order (ascending assignment index inside each expert) and its inverse.  All integer.
// An assignment whose id lies outside [0, E) is dropped: it is in no count, its
// assign_pos is -1, and sorted_assign holds -1 past offsets[E] (every path below).
#include "common.h"
#include "xchg.h"

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
// listed in ascending id, the shared expert (id E, all T tokens) last.  For the streaming
// path (T <= kGemvMaxT, routed experts present) an expert with more than kUnitRows rows
// is listed as several units of at most kUnitRows rows, so one token-tile width serves
// every unit (the shared expert's weights are then read once per unit).
__device__ void build_plan(int T, int E, int k, int S, int H, const int *cnt, const int *off,
                           const Plan &p, PlanScratch &ps)
{
    const int tid = threadIdx.x, bd = blockDim.x;
    const int n = E + S;
    const bool split = T <= kGemvMaxT && E > 0;
    for (int e = tid; e < n; e += bd) {
        const int rows = (e < E) ? cnt[e] : T;
        ps.flag[e] = rows <= 0 ? 0 : split ? (rows + kUnitRows - 1) / kUnitRows : 1;
    }
    __syncthreads();
    if (tid < 64) wave0_exclusive_scan(ps.flag, ps.idx, n);
    __syncthreads();
    const int nT = ps.idx[n];
    for (int e = tid; e < n; e += bd) {
        const int rows = (e < E) ? cnt[e] : T, base = (e < E) ? off[e] : T * k;
        for (int c = 0; c < ps.flag[e]; c++) {
            const int u = ps.idx[e] + c;
            const int r = split ? min(kUnitRows, rows - kUnitRows * c) : rows;
            p.touched[u] = e;
            p.tbase[u] = base + (split ? kUnitRows * c : 0);
            p.tcount[u] = r;
            ps.nt[u] = (r + kGemmBM - 1) / kGemmBM;
        }
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
    for (int p = g.off[E] + tid; p < n; p += 1024) sa[p] = -1;  // past the valid assignments
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = 0; base < n; base += 1024) {
        const int a = base + tid;
        int e = (a < n) ? ids[a] : -1;
        const bool valid = (e >= 0 && e < E);
        if (!valid && a < n) ap[a] = -1;
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

// Grouping and plan for n = T * k <= 256 assignments by one 1024-thread workgroup, all in
// LDS: per-expert counts (LDS atomics), exclusive offsets, and the stable position of
// assignment a = the offset of its expert plus the number of earlier assignments of the
// same expert.  Plan: touched experts ascending, the shared expert (all T tokens) last,
// one work item each (no expert holds more than kGemvMaxT * 8 rows).
struct SmallGroup {
    int cnt[257], off[258], flag[257], idx[258];
    int wcnt[4][256];  // per wave of assignments: how many of them went to each expert
};

__device__ void group_plan_small(int T, int E, int k, int S, const int32_t *s_ids, SmallGroup &g,
                                 int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
                                 int32_t *__restrict__ sa, int32_t *__restrict__ ap, const Plan &p)
{
    const int tid = threadIdx.x, n = T * k, lane = tid & 63, wv = tid >> 6;
    if (tid < E) g.cnt[tid] = 0;
    (&g.wcnt[0][0])[tid] = 0;  // 1024 entries, one per thread
    __syncthreads();
    const int e = tid < n ? s_ids[tid] : -1;
    const bool valid = e >= 0 && e < E;
    if (valid) atomicAdd(&g.cnt[e], 1);
    // lanes of this wave with the same expert (one ballot per id bit) and the rank among them
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; b++) {
        const bool bit = valid && ((e >> b) & 1);
        const uint64_t vote = __ballot(bit);
        peers &= bit ? vote : ~vote;
    }
    const uint64_t lt_mask = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(peers & lt_mask);
    if (valid && rank == 0) g.wcnt[wv][e] = __popcll(peers);
    __syncthreads();
    if (tid < 64) wave0_exclusive_scan(g.cnt, g.off, E);
    __syncthreads();
    if (tid < E) {
        counts[tid] = g.cnt[tid];
        offsets[tid] = g.off[tid];
    }
    if (tid == 0) offsets[E] = g.off[E];
    if (valid) {  // stable: earlier waves' assignments of e, then this wave's lower lanes
        int before = rank;
        for (int w = 0; w < wv; w++) before += g.wcnt[w][e];
        const int pos = g.off[e] + before;
        sa[pos] = tid;
        ap[tid] = pos;
    } else if (tid < n) {
        ap[tid] = -1;
    }
    if (tid >= g.off[E] && tid < n) sa[tid] = -1;
    // units of at most kUnitRows rows (as in build_plan's streaming case)
    const int nf = E + S;
    if (tid < nf) {
        const int rows = tid < E ? g.cnt[tid] : T;
        g.flag[tid] = (rows + kUnitRows - 1) / kUnitRows;
    }
    __syncthreads();
    if (tid < 64) wave0_exclusive_scan(g.flag, g.idx, nf);
    __syncthreads();
    if (tid < nf) {
        const int rows = tid < E ? g.cnt[tid] : T, base = tid < E ? g.off[tid] : T * k;
        for (int c = 0; c < g.flag[tid]; c++) {
            const int u = g.idx[tid] + c;
            p.touched[u] = tid;
            p.tbase[u] = base + kUnitRows * c;
            p.tcount[u] = min(kUnitRows, rows - kUnitRows * c);
            p.items[u] = u << 16;
        }
    }
    if (tid == 0) {
        p.meta[0] = g.idx[nf];
        p.meta[1] = g.idx[nf];
    }
}

// Small batches (T <= 32, unless the single-token launch takes T = 1): router, selection,
// grouping and plan in one persistent launch of kPersistentGrid workgroups (one per CU), so
// the expert kernels that follow need no routing step of their own.  Workgroup e < E
// (16 waves, wave w takes tokens w and w + 16) computes the logits of expert e and publishes
// each as a tagged exchange word (xchg.h: the launch tag and the fp32 value in one 64-bit
// agent-scope store).  Workgroups 0 and, for more than 16 tokens, 1 then select: wave w of
// workgroup b polls the E words of token 16 b + w and picks its top-k (`topk_wave`).
// Workgroup 1 publishes its tokens' selections as words too; workgroup 0 waits for them,
// groups the assignments by expert and writes the plan.  Every other workgroup ends after
// publishing its logits.
//
// An arrival counter instead of tagged words (each workgroup storing its logits, waiting
// for the stores and incrementing one agent-scope counter, the last to arrive selecting for
// every token) measured 11.9 / 18.7 µs per launch at T = 8 / 32 against 8.7 / 12.2 µs here:
// the store wait, the 256 serialised increments, and 32 tokens on one CU's 4 SIMDs.
// Every wait is bounded (kSpin tries); one that runs out sets the workspace head's error
// flag, as in the other persistent launches.
__global__ __launch_bounds__(1024) void router_select_kernel(
    int T, int H, int E, int k, int S, int renorm, const uint16_t *__restrict__ x,
    const float *__restrict__ Wr, const float *__restrict__ bias, float *__restrict__ logits,
    int32_t *__restrict__ ids, float *__restrict__ wout, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sa, int32_t *__restrict__ ap, Plan plan,
    uint8_t *head)
{
    static_assert(kGemvMaxT <= 32, "two selecting workgroups of 16 waves");
    __shared__ SmallGroup g;
    __shared__ float s_lg[16][256];  // the logits of this wave's token
    __shared__ int32_t s_ids[kGemvMaxT * 8];
    __shared__ float s_w[kGemvMaxT * 8];
    __shared__ uint32_t s_tag, s_giveup;
    const int b = blockIdx.x, tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
    uint32_t launches = 0;
    if (tid == 0) {
        launches = read_launches(head);
        s_tag = launch_tag(launches);
        s_giveup = diag_word(head);
    }
    float sums[2] = {0.f, 0.f};
    if (b < E) router_dot_wave<2>(T, H, b, wv, 16, x, Wr, sums);
    __syncthreads();
    const uint32_t tag = s_tag;
    const bool giveup = s_giveup != 0;
    // logit words [T][E], then the second selecting workgroup's {id, weight} word pairs
    uint64_t *xl = reinterpret_cast<uint64_t *>(head + kHeadFewXchg);
    uint64_t *xs = xl + (size_t)T * E;
    if (b < E && lane == 0) {
        const float bv = bias ? bias[b] : 0.f;
#pragma unroll
        for (int q = 0; q < 2; q++) {
            const int t = wv + 16 * q;
            if (t < T) {
                const float l = sums[q] + bv;
                logits[(size_t)t * E + b] = l;
                put_word(xl + (size_t)t * E + b, tag, l);
            }
        }
    }
    if (b >= (T + 15) / 16) {
        if (tid == 0) bump_launches(head, launches);
        return;
    }
    const int t = 16 * b + wv;  // this wave's token
    if (t < T) {
        uint64_t lw[4];
        const int nq = (E - lane + 63) / 64;  // words of experts lane, lane + 64, ... below E
#pragma unroll
        for (int i = 0; i < 4; i++) lw[i] = i < nq ? get_word(xl + (size_t)t * E + lane + 64 * i) : 0ull;
        await_words<4>(xl + (size_t)t * E + lane, 64, nq, lw, tag, head, giveup);
#pragma unroll
        for (int i = 0; i < 4; i++)
            if (i < nq) s_lg[wv][lane + 64 * i] = __uint_as_float((uint32_t)lw[i]);
    }
    __syncthreads();
    if (t < T) {
        topk_wave(s_lg[wv], E, k, renorm, s_ids + t * k, s_w + t * k);
        if (b > 0 && lane < k) {
            const int a = (t - 16) * k + lane;
            put_word(xs + 2 * a, tag, __int_as_float(s_ids[t * k + lane]));
            put_word(xs + 2 * a + 1, tag, s_w[t * k + lane]);
        }
    }
    if (b > 0) {
        if (tid == 0) bump_launches(head, launches);
        return;
    }
    if (T > 16 && tid < (T - 16) * k) {  // assignment 16 k + tid, selected by workgroup 1
        uint64_t sw[2] = {get_word(xs + 2 * tid), get_word(xs + 2 * tid + 1)};
        await_words<2>(xs + 2 * tid, 1, 2, sw, tag, head, giveup);
        s_ids[16 * k + tid] = (int32_t)(uint32_t)sw[0];
        s_w[16 * k + tid] = __uint_as_float((uint32_t)sw[1]);
    }
    __syncthreads();
    for (int a = tid; a < T * k; a += 1024) {
        ids[a] = s_ids[a];
        wout[a] = s_w[a];
    }
    group_plan_small(T, E, k, S, s_ids, g, counts, offsets, sa, ap, plan);
    if (tid == 0) bump_launches(head, launches);
}

bool router_select_supported(const Shape &s, int64_t T)
{
    return T >= 1 && T <= kGemvMaxT && s.E >= 1 && s.E <= 256 && s.k >= 1 && s.k <= 8 && s.S <= 1 &&
           persistent_fits(reinterpret_cast<const void *>(&router_select_kernel), 1024, 0);
}

hipError_t launch_router_select(const Shape &s, int64_t T, const uint16_t *x, const float *Wr,
                                const float *bias, float *logits, int32_t *ids, float *w,
                                int32_t *counts, int32_t *offsets, int32_t *sa, int32_t *ap,
                                const Plan &plan, uint8_t *head, hipStream_t st)
{
    router_select_kernel<<<kPersistentGrid, 1024, 0, st>>>((int)T, s.H, s.E, s.k, s.S, s.renorm, x, Wr, bias,
                                                           logits, ids, w, counts, offsets, sa, ap, plan, head);
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
                                                        int32_t *__restrict__ offsets,
                                                        int32_t *__restrict__ sa, Plan plan,
                                                        int with_plan)
{
    __shared__ int cnt[256];
    __shared__ int off[257];
    __shared__ PlanScratch ps;
    // Thread e: expert e's count over the blocks, then (once the offsets are known) its
    // base in every block = offset of e + the counts of e in earlier blocks.  The block
    // counts are read 16 at a time, every read of a batch in flight together.
    constexpr int B = 16;
    const int e = threadIdx.x;
    int tot = 0;
    if (e < E)
        for (int b0 = 0; b0 < nb; b0 += B) {
            int c[B];
#pragma unroll
            for (int i = 0; i < B; i++) c[i] = b0 + i < nb ? hist[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < B; i++) tot += c[i];
        }
    if (e < 256) cnt[e] = (e < E) ? tot : 0;
    __syncthreads();
    if (threadIdx.x < 64) wave0_exclusive_scan(cnt, off, E);
    __syncthreads();
    if (e < E) {
        counts[e] = cnt[e];
        offsets[e] = off[e];
        int run = off[e];
        for (int b0 = 0; b0 < nb; b0 += B) {
            int c[B];
#pragma unroll
            for (int i = 0; i < B; i++) c[i] = b0 + i < nb ? hist[(size_t)(b0 + i) * E + e] : 0;
#pragma unroll
            for (int i = 0; i < B; i++) {
                if (b0 + i < nb) hist[(size_t)(b0 + i) * E + e] = run;
                run += c[i];
            }
        }
    }
    if (e == 0) offsets[E] = off[E];
    for (int p = off[E] + (int)threadIdx.x; p < T * k; p += 256) sa[p] = -1;  // past the valid assignments
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
    } else if (a < n) {
        ap[a] = -1;
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
    perm_scan_kernel<<<1, 256, 0, st>>>((int)T, s.E, s.k, s.S, s.H, nb, hist, counts, offsets, sa, p,
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
    for (int e = threadIdx.x; e <= E; e += blockDim.x) off[e] = E ? offsets[e] : 0;  // E = 0: dense
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
