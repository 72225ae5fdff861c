// api.hip -- the C ABI declared in include/flint_moe.h: argument validation, workspace
// layout and dispatch to the kernels.  Validation runs before any HIP call, so invalid
// arguments are reported without touching the device.
#include "../../include/flint_moe.h"
#include "common.h"

#include <mutex>
#include <stdio.h>
#include <string.h>

using namespace flint;

namespace {

constexpr int64_t kMaxT = 65536;
constexpr int32_t kMaxChainLayers = 4096;
thread_local char g_msg[256];
thread_local hipError_t g_last_hip = hipSuccess;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

int check_desc(const flint_moe_desc *d)
{
    if (!d) return FLINT_ERR_NULL;
    if (d->n_experts == 0) {  // dense SwiGLU layer: the shared expert alone, no routing
        if (d->top_k != 0 || d->n_shared != 1) return FLINT_ERR_SHAPE;
    } else {
        if (d->n_experts < 1 || d->n_experts > 256) return FLINT_ERR_SHAPE;
        if (d->top_k < 1 || d->top_k > 8 || d->top_k > d->n_experts) return FLINT_ERR_SHAPE;
        if (d->n_shared != 0 && d->n_shared != 1) return FLINT_ERR_SHAPE;
    }
    if (d->hidden < 64 || d->hidden > 8192 || d->hidden % 64) return FLINT_ERR_SHAPE;
    if (d->inter < 32 || d->inter > 4096 || d->inter % 32) return FLINT_ERR_SHAPE;
    if (d->renormalize != 0 && d->renormalize != 1) return FLINT_ERR_SHAPE;
    return FLINT_OK;
}

Shape shape_of(const flint_moe_desc *d)
{
    return Shape{d->hidden, d->inter, d->n_experts, d->top_k, d->n_shared, d->renormalize};
}

int hip_status(hipError_t e)
{
    if (e == hipSuccess) return FLINT_OK;
    g_last_hip = e;
    return FLINT_ERR_HIP;
}

// INT4 scale groups are 128 columns of K (H for gate/up, I for down).
bool format_fits(const flint_moe_desc *d, int32_t format)
{
    return format != FLINT_WFMT_INT4 || (d->hidden % 128 == 0 && d->inter % 128 == 0);
}

int check_weights(const flint_moe_desc *d, const flint_moe_weights *w)
{
    if (!w) return FLINT_ERR_NULL;
    if (w->format != FLINT_WFMT_BF16 && w->format != FLINT_WFMT_NVFP4 && w->format != FLINT_WFMT_INT4)
        return FLINT_ERR_FORMAT;
    if (!format_fits(d, w->format)) return FLINT_ERR_SHAPE;
    const bool dense = d->n_experts == 0;
    if (dense) {  // no routed experts: their pointers must be NULL
        const void *rp[] = {w->gate, w->up, w->down, w->gate_sf, w->up_sf, w->down_sf,
                            w->gate_ts, w->up_ts, w->down_ts};
        for (const void *p : rp)
            if (p) return FLINT_ERR_FORMAT;
    } else if (!w->gate || !w->up || !w->down) {
        return FLINT_ERR_NULL;
    }
    const bool has_sh = w->sh_gate && w->sh_up && w->sh_down;
    const bool any_sh = w->sh_gate || w->sh_up || w->sh_down;
    if (d->n_shared && !has_sh) return FLINT_ERR_NULL;
    if (!d->n_shared && any_sh) return FLINT_ERR_FORMAT;
    const void *ptrs[] = {w->gate, w->up, w->down, w->sh_gate, w->sh_up, w->sh_down};
    for (const void *p : ptrs)
        if (!aligned16(p)) return FLINT_ERR_ALIGN;
    const void *sc[] = {w->gate_sf, w->up_sf, w->down_sf, w->gate_ts, w->up_ts, w->down_ts};
    const void *shsc[] = {w->sh_gate_sf, w->sh_up_sf, w->sh_down_sf, w->sh_ts};
    if (w->format == FLINT_WFMT_BF16) {
        for (const void *p : sc)
            if (p) return FLINT_ERR_FORMAT;
        for (const void *p : shsc)
            if (p) return FLINT_ERR_FORMAT;
    } else if (w->format == FLINT_WFMT_INT4) {  // group scales; no tensor scales
        const void *gs[] = {w->gate_sf, w->up_sf, w->down_sf};
        const void *shgs[] = {w->sh_gate_sf, w->sh_up_sf, w->sh_down_sf};
        if (w->gate_ts || w->up_ts || w->down_ts || w->sh_ts) return FLINT_ERR_FORMAT;
        for (const void *p : gs) {
            if (!dense && !p) return FLINT_ERR_FORMAT;
            if (!aligned16(p)) return FLINT_ERR_ALIGN;
        }
        for (const void *p : shgs) {
            if (d->n_shared && !p) return FLINT_ERR_FORMAT;
            if (!d->n_shared && p) return FLINT_ERR_FORMAT;
            if (!aligned16(p)) return FLINT_ERR_ALIGN;
        }
    } else {
        for (const void *p : sc)
            if (!dense && !p) return FLINT_ERR_FORMAT;
        for (const void *p : sc)
            if (!aligned16(p)) return FLINT_ERR_ALIGN;
        for (const void *p : shsc) {
            if (d->n_shared && !p) return FLINT_ERR_FORMAT;
            if (!d->n_shared && p) return FLINT_ERR_FORMAT;
            if (!aligned16(p)) return FLINT_ERR_ALIGN;
        }
    }
    return FLINT_OK;
}

WSet wset_of(const flint_moe_weights *w)
{
    WSet s;
    s.fmt = w->format;
    auto mk = [&](const void *r, const void *sh, const uint8_t *sf, const uint8_t *shsf,
                  const float *ts, int idx) {
        WMat m;
        m.routed = (const uint8_t *)r;
        m.shared = (const uint8_t *)sh;
        m.sf_routed = sf;
        m.sf_shared = shsf;
        m.ts_routed = ts;
        m.ts_shared = w->sh_ts ? w->sh_ts + idx : nullptr;
        return m;
    };
    s.gate = mk(w->gate, w->sh_gate, w->gate_sf, w->sh_gate_sf, w->gate_ts, 0);
    s.up = mk(w->up, w->sh_up, w->up_sf, w->sh_up_sf, w->up_ts, 1);
    s.down = mk(w->down, w->sh_down, w->down_sf, w->sh_down_sf, w->down_ts, 2);
    return s;
}

}  // namespace

// Workspace of flint_moe_layer_noalloc: one copy per GPU, zero when the library's code object
// is loaded on that device and kept for the life of the process.  Host code never uses this
// name as an address: it asks hipGetSymbolAddress for the device's copy (noalloc_scratch).
constexpr size_t kNoallocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {

// Device address of the current device's `scratch`, looked up once per device.
int noalloc_scratch(void **out)
{
    static std::mutex mu;
    static void *addr[64];
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= 64) return hip_status(hipErrorInvalidDevice);
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        const hipError_t es = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (es != hipSuccess) return hip_status(es);
        addr[dev] = p;
    }
    *out = addr[dev];
    return FLINT_OK;
}

}  // namespace

namespace flint {

WsLayout ws_layout(const Shape &s, int64_t T)
{
    WsLayout L{};
    const size_t TK = (size_t)T * s.k, slots = TK + (size_t)T * s.S;
    L.max_items = (int)((slots + kGemmBM - 1) / kGemmBM + s.E + s.S);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t o = off;
        off = align_up(off + bytes, 256);
        return o;
    };
    L.sync = take(kSyncBytes);  // always at offset 0, whatever T
    L.logits = take((size_t)T * s.E * 4);
    L.ids = take(TK * 4);
    L.w = take(TK * 4);
    L.counts = take((size_t)s.E * 4);
    L.offsets = take((size_t)(s.E + 1) * 4);
    L.sa = take(TK * 4);
    L.ap = take(TK * 4);
    L.plan = take((size_t)(4 + 3 * plan_unit_capacity(s.E, s.k, s.S, T) + L.max_items) * 4);
    L.plan_units = (int)plan_unit_capacity(s.E, s.k, s.S, T);
    L.hist = take(((TK + 1023) / 1024) * (size_t)s.E * 4);
    L.h = take(slots * s.I * 4);
    L.o = take(slots * s.H * 4);
    L.total = off;
    return L;
}

Plan plan_view(void *ws, const WsLayout &L, const Shape &s)
{
    (void)s;
    int *b = (int *)((char *)ws + L.plan);
    Plan p;
    p.meta = b;
    p.touched = b + 4;
    p.tbase = p.touched + L.plan_units;
    p.tcount = p.tbase + L.plan_units;
    p.items = p.tcount + L.plan_units;
    return p;
}

__global__ void zero_words_kernel(uint32_t *p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

}  // namespace flint

extern "C" {

int flint_moe_workspace_init(void *ws, size_t ws_bytes, void *stream)
{
    if (!ws) return FLINT_ERR_NULL;
    if (!aligned16(ws)) return FLINT_ERR_ALIGN;
    if (ws_bytes < kSyncBytes) return FLINT_ERR_WORKSPACE;
    const int n = (int)(kSyncBytes / 4);
    flint::zero_words_kernel<<<(n + 255) / 256, 256, 0, (hipStream_t)stream>>>((uint32_t *)ws, n);
    return hip_status(hipGetLastError());
}

size_t flint_moe_workspace_bytes(const flint_moe_desc *desc, int64_t T_max, int32_t format)
{
    if (check_desc(desc) != FLINT_OK || T_max < 0 || T_max > kMaxT) return 0;
    if (format != FLINT_WFMT_BF16 && format != FLINT_WFMT_NVFP4 && format != FLINT_WFMT_INT4) return 0;
    if (!format_fits(desc, format)) return 0;
    return ws_layout(shape_of(desc), T_max).total;
}

int flint_moe_workspace_status(void *ws, size_t ws_bytes, int32_t *flags, void *stream)
{
    if (!ws || !flags) return FLINT_ERR_NULL;
    if (!aligned16(ws) || ((uintptr_t)flags & 3u)) return FLINT_ERR_ALIGN;
    if (ws_bytes < kSyncBytes) return FLINT_ERR_WORKSPACE;
    return hip_status(launch_ws_status(ws, flags, (hipStream_t)stream));
}

const char *flint_moe_status_string(int status)
{
    switch (status) {
    case FLINT_OK: return "ok";
    case FLINT_ERR_NULL: return "a required pointer is NULL";
    case FLINT_ERR_SHAPE: return "descriptor or token count outside the supported range";
    case FLINT_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case FLINT_ERR_WORKSPACE: return "workspace smaller than flint_moe_workspace_bytes()";
    case FLINT_ERR_FORMAT: return "unknown weight format or inconsistent scale arrays";
    case FLINT_ERR_HIP:
        snprintf(g_msg, sizeof g_msg, "HIP launch error: %s", hipGetErrorString(g_last_hip));
        return g_msg;
    default: return "unknown status";
    }
}

int flint_moe_route(const flint_moe_desc *desc, int64_t T, const uint16_t *x,
                    const float *w_router, const float *logit_bias, float *logits,
                    int32_t *topk_ids, float *topk_w, uint32_t flags, void *ws,
                    size_t ws_bytes, void *stream)
{
    int rc = check_desc(desc);
    if (rc) return rc;
    if (desc->n_experts == 0 || T < 0 || T > kMaxT) return FLINT_ERR_SHAPE;
    if (flags & ~(uint32_t)FLINT_ROUTE_LOGITS_IN) return FLINT_ERR_FORMAT;
    if (T == 0) return FLINT_OK;
    const bool lin = flags & FLINT_ROUTE_LOGITS_IN;
    if (!topk_ids || !topk_w) return FLINT_ERR_NULL;
    if (lin && !logits) return FLINT_ERR_NULL;
    if (!lin && (!x || !w_router)) return FLINT_ERR_NULL;
    const void *ptrs[] = {x, w_router, logit_bias, logits, topk_ids, topk_w, ws};
    for (const void *p : ptrs)
        if (!aligned16(p)) return FLINT_ERR_ALIGN;
    const Shape s = shape_of(desc);
    const WsLayout L = ws_layout(s, T);
    float *lg = logits;
    if (!lg) {
        if (!ws) return FLINT_ERR_NULL;
        if (ws_bytes < L.total) return FLINT_ERR_WORKSPACE;
        lg = (float *)((char *)ws + L.logits);
    }
    hipStream_t st = (hipStream_t)stream;
    if (!lin) {
        rc = hip_status(launch_router(s, T, x, w_router, logit_bias, lg, st));
        if (rc) return rc;
    }
    return hip_status(launch_topk(s, T, lg, topk_ids, topk_w, st));
}

int flint_moe_permute(const flint_moe_desc *desc, int64_t T, const int32_t *topk_ids,
                      int32_t *counts, int32_t *offsets, int32_t *sorted_assign,
                      int32_t *assign_pos, void *ws, size_t ws_bytes, void *stream)
{
    int rc = check_desc(desc);
    if (rc) return rc;
    if (desc->n_experts == 0 || T < 0 || T > kMaxT) return FLINT_ERR_SHAPE;
    if (T == 0) return FLINT_OK;
    if (!topk_ids || !counts || !offsets || !sorted_assign || !assign_pos) return FLINT_ERR_NULL;
    const void *ptrs[] = {topk_ids, counts, offsets, sorted_assign, assign_pos};
    for (const void *p : ptrs)
        if (!aligned16(p)) return FLINT_ERR_ALIGN;
    const Shape s = shape_of(desc);
    const WsLayout L = ws_layout(s, T);
    int32_t *hist = nullptr;
    if (ws && ws_bytes >= L.total) hist = (int32_t *)((char *)ws + L.hist);
    return hip_status(launch_permute(s, T, topk_ids, counts, offsets, sorted_assign, assign_pos,
                                     nullptr, hist, (hipStream_t)stream));
}

static int forward_impl(const Shape &s, const WSet &wset, int64_t T, const uint16_t *x,
                        const float *topk_w, const int32_t *sa, const int32_t *ap, uint16_t *y,
                        void *ws, const WsLayout &L, const Plan &plan, hipStream_t st)
{
    char *b = (char *)ws;
    if (T <= kGemvMaxT) {
        return hip_status(launch_gemv_forward(s, wset, T, x, topk_w, sa, ap, plan,
                                              (uint16_t *)(b + L.h), (float *)(b + L.o), y, st));
    }
    return hip_status(launch_gemm_forward(s, wset, T, x, topk_w, sa, ap, plan,
                                          (uint16_t *)(b + L.h), (uint16_t *)(b + L.o), y, st));
}

int flint_moe_forward(const flint_moe_desc *desc, const flint_moe_weights *weights, int64_t T,
                      const uint16_t *x, const int32_t *topk_ids, const float *topk_w,
                      const int32_t *offsets, const int32_t *sorted_assign,
                      const int32_t *assign_pos, uint16_t *y, void *ws, size_t ws_bytes,
                      void *stream)
{
    (void)topk_ids;
    int rc = check_desc(desc);
    if (rc) return rc;
    if (T < 0 || T > kMaxT) return FLINT_ERR_SHAPE;
    rc = check_weights(desc, weights);
    if (rc) return rc;
    if (T == 0) return FLINT_OK;
    const bool dense = desc->n_experts == 0;  // routing arguments unused (may be NULL)
    if (!x || !y || !ws) return FLINT_ERR_NULL;
    if (!dense && (!topk_ids || !topk_w || !offsets || !sorted_assign || !assign_pos))
        return FLINT_ERR_NULL;
    const void *ptrs[] = {x, topk_ids, topk_w, offsets, sorted_assign, assign_pos, y, ws};
    for (const void *p : ptrs)
        if (!aligned16(p)) return FLINT_ERR_ALIGN;
    const Shape s = shape_of(desc);
    const WsLayout L = ws_layout(s, T);
    if (ws_bytes < L.total) return FLINT_ERR_WORKSPACE;
    const Plan plan = plan_view(ws, L, s);
    hipStream_t st = (hipStream_t)stream;
    if (dense && T == 1 && dense1_supported(s, weights->format))
        return hip_status(launch_dense1(s, wset_of(weights), x, y, (char *)ws + L.sync, st));
    if (!dense || T > kGemvMaxT) {  // the streaming kernels take a dense layer's plan as implicit
        rc = hip_status(launch_plan(s, T, dense ? nullptr : offsets, plan, st));
        if (rc) return rc;
    }
    return forward_impl(s, wset_of(weights), T, x, topk_w, sorted_assign, assign_pos, y, ws, L,
                        plan, st);
}

}  // extern "C"

// Arguments of flint_moe_layer other than the workspace; T == 0 passes (a no-op).
static int check_layer_args(const flint_moe_desc *desc, const flint_moe_weights *weights, int64_t T,
                            const uint16_t *x, const float *w_router, const float *logit_bias,
                            const uint16_t *y, const flint_moe_routing *routing)
{
    int rc = check_desc(desc);
    if (rc) return rc;
    if (T < 0 || T > kMaxT) return FLINT_ERR_SHAPE;
    rc = check_weights(desc, weights);
    if (rc) return rc;
    if (T == 0) return FLINT_OK;
    const bool dense = desc->n_experts == 0;  // no router: w_router, logit_bias, routing unused
    if (!x || (!dense && !w_router) || !y) return FLINT_ERR_NULL;
    const void *ptrs[] = {x, w_router, logit_bias, y};
    for (const void *p : ptrs)
        if (!aligned16(p)) return FLINT_ERR_ALIGN;
    if (routing) {
        const void *rptrs[] = {routing->logits, routing->topk_ids, routing->topk_w, routing->counts,
                               routing->offsets, routing->sorted_assign, routing->assign_pos};
        for (const void *p : rptrs)
            if (!aligned16(p)) return FLINT_ERR_ALIGN;
    }
    return FLINT_OK;
}

extern "C" {

int flint_moe_layer(const flint_moe_desc *desc, const flint_moe_weights *weights, int64_t T,
                    const uint16_t *x, const float *w_router, const float *logit_bias,
                    uint16_t *y, const flint_moe_routing *routing, void *ws, size_t ws_bytes,
                    void *stream)
{
    int rc = check_layer_args(desc, weights, T, x, w_router, logit_bias, y, routing);
    if (rc || T == 0) return rc;
    if (!ws) return FLINT_ERR_NULL;
    if (!aligned16(ws)) return FLINT_ERR_ALIGN;
    const bool dense = desc->n_experts == 0;
    flint_moe_routing R{};
    if (routing) R = *routing;
    const Shape s = shape_of(desc);
    const WsLayout L = ws_layout(s, T);
    if (ws_bytes < L.total) return FLINT_ERR_WORKSPACE;
    char *b = (char *)ws;
    float *lg = R.logits ? R.logits : (float *)(b + L.logits);
    int32_t *ids = R.topk_ids ? R.topk_ids : (int32_t *)(b + L.ids);
    float *tw = R.topk_w ? R.topk_w : (float *)(b + L.w);
    int32_t *cnt = R.counts ? R.counts : (int32_t *)(b + L.counts);
    int32_t *off = R.offsets ? R.offsets : (int32_t *)(b + L.offsets);
    int32_t *sa = R.sorted_assign ? R.sorted_assign : (int32_t *)(b + L.sa);
    int32_t *ap = R.assign_pos ? R.assign_pos : (int32_t *)(b + L.ap);
    hipStream_t st = (hipStream_t)stream;
    const Plan plan = plan_view(ws, L, s);
    if (dense) {
        if (T == 1 && dense1_supported(s, weights->format))
            return hip_status(launch_dense1(s, wset_of(weights), x, y, b + L.sync, st));
        if (T > kGemvMaxT) {  // the streaming kernels take a dense layer's plan as implicit
            rc = hip_status(launch_plan(s, T, nullptr, plan, st));
            if (rc) return rc;
        }
        return forward_impl(s, wset_of(weights), T, x, nullptr, nullptr, nullptr, y, ws, L, plan, st);
    }
    if (T == 1 && decode1_supported(s, weights->format)) {
        return hip_status(launch_decode1(s, wset_of(weights), x, w_router, logit_bias, y, lg, ids, tw,
                                         cnt, off, sa, ap, b + L.sync, st));
    }
    // The small-batch launch for bf16 weights; with 4-bit weights the dequantisation makes its
    // streaming waves VALU-bound and the four-launch path below measured faster per layer.
    if (weights->format == FLINT_WFMT_BF16 && decode_few_supported(s, weights->format, T)) {
        return hip_status(launch_decode_few(s, wset_of(weights), T, x, w_router, logit_bias, y, lg, ids, tw,
                                            cnt, off, sa, ap, b + L.sync, st));
    }
    if (router_select_supported(s, T)) {  // T <= kGemvMaxT: one persistent launch
        rc = hip_status(launch_router_select(s, T, x, w_router, logit_bias, lg, ids, tw, cnt, off,
                                             sa, ap, plan, (uint8_t *)(b + L.sync), st));
        if (rc) return rc;
    } else {
        rc = hip_status(launch_router(s, T, x, w_router, logit_bias, lg, st));
        if (rc) return rc;
        rc = hip_status(launch_topk(s, T, lg, ids, tw, st));
        if (rc) return rc;
        rc = hip_status(launch_permute(s, T, ids, cnt, off, sa, ap, &plan,
                                       (int32_t *)(b + L.hist), st));
        if (rc) return rc;
    }
    return forward_impl(s, wset_of(weights), T, x, tw, sa, ap, y, ws, L, plan, st);
}

int flint_moe_decode_chain(const flint_moe_desc *desc, const flint_moe_layer_ref *layers,
                           int32_t n_layers, uint32_t flags, int64_t T, const uint16_t *x, uint16_t *y,
                           int32_t *topk_ids, float *topk_w, float *logits, void *ws,
                           size_t ws_bytes, void *stream)
{
    int rc = check_desc(desc);
    if (rc) return rc;
    if (desc->n_experts == 0 || n_layers < 0 || n_layers > kMaxChainLayers) return FLINT_ERR_SHAPE;
    if (T < 1 || T > kChainMaxT) return FLINT_ERR_SHAPE;
    if (flags & ~(uint32_t)FLINT_CHAIN_RESIDUAL) return FLINT_ERR_FORMAT;
    if (n_layers == 0) return FLINT_OK;
    if (!layers || !x || !y || !ws) return FLINT_ERR_NULL;
    const void *ptrs[] = {x, y, topk_ids, topk_w, logits, ws};
    for (const void *p : ptrs)
        if (!aligned16(p)) return FLINT_ERR_ALIGN;
    const int fmt = layers[0].weights.format;
    for (int l = 0; l < n_layers; l++) {
        rc = check_weights(desc, &layers[l].weights);
        if (rc) return rc;
        if (layers[l].weights.format != fmt) return FLINT_ERR_FORMAT;
        if (!layers[l].w_router) return FLINT_ERR_NULL;
        if (!aligned16(layers[l].w_router) || !aligned16(layers[l].logit_bias)) return FLINT_ERR_ALIGN;
    }
    const Shape s = shape_of(desc);
    const WsLayout L = ws_layout(s, T);
    if (ws_bytes < L.total) return FLINT_ERR_WORKSPACE;
    if (T == 1 ? !decode1_supported(s, fmt) : !decode_few_supported(s, fmt, T)) return FLINT_ERR_SHAPE;
    hipStream_t st = (hipStream_t)stream;
    char *b = (char *)ws;
    for (int l0 = 0; l0 < n_layers; l0 += kChainChunk) {
        const int n = n_layers - l0 < kChainChunk ? n_layers - l0 : kChainChunk;
        WSet w[kChainChunk];
        const float *wr[kChainChunk], *bias[kChainChunk];
        for (int i = 0; i < n; i++) {
            w[i] = wset_of(&layers[l0 + i].weights);
            wr[i] = layers[l0 + i].w_router;
            bias[i] = layers[l0 + i].logit_bias;
        }
        const bool residual = flags & FLINT_CHAIN_RESIDUAL, hand_on = l0 + n < n_layers;
        int32_t *ids = topk_ids ? topk_ids + (size_t)l0 * T * s.k : nullptr;
        float *tw = topk_w ? topk_w + (size_t)l0 * T * s.k : nullptr;
        float *lg = logits ? logits + (size_t)l0 * T * s.E : nullptr;
        if (T == 1)
            rc = hip_status(launch_decode_chain(s, w, wr, bias, n, residual, l0 == 0 ? x : nullptr, hand_on,
                                                y + (size_t)l0 * s.H, ids, tw, lg, ws, st));
        else
            rc = hip_status(launch_decode_few_chain(s, w, wr, bias, n, l0, residual, T, x, hand_on,
                                                    y + (size_t)l0 * T * s.H, ids, tw, lg, (int32_t *)(b + L.ids),
                                                    (float *)(b + L.w), ws, st));
        if (rc) return rc;
    }
    return FLINT_OK;
}

int flint_moe_layer_noalloc(const flint_moe_desc *desc, const flint_moe_weights *weights, int64_t T,
                            const uint16_t *x, const float *w_router, const float *logit_bias,
                            uint16_t *y, const flint_moe_routing *routing, void *stream)
{
    int rc = check_layer_args(desc, weights, T, x, w_router, logit_bias, y, routing);
    if (rc || T == 0) return rc;
    if (ws_layout(shape_of(desc), T).total > kNoallocScratchBytes) return FLINT_ERR_WORKSPACE;
    void *ws = nullptr;
    rc = noalloc_scratch(&ws);
    if (rc) return rc;
    return flint_moe_layer(desc, weights, T, x, w_router, logit_bias, y, routing, ws, kNoallocScratchBytes,
                           stream);
}

}  // extern "C"
