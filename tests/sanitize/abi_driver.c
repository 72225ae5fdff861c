/* Drives every entry point of include/flint_moe.h through its argument validation (every
   call here is rejected before any HIP call, so no GPU is needed), for a build of the
   library's host code with AddressSanitizer and UndefinedBehaviorSanitizer.  Checks the
   documented status codes; any out-of-bounds access or undefined operation in the host
   code aborts the program.  Exit status 0 = clean. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../../include/flint_moe.h"

#define A ((void *)(uintptr_t)(1 << 20)) /* a 16-byte aligned address, never dereferenced */
#define MIS ((void *)(uintptr_t)((1 << 20) + 8))

static int failures = 0;
static void expect(int got, int want, const char *what)
{
    if (got != want) {
        fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
        failures++;
    }
}

static flint_moe_weights weights(int fmt)
{
    flint_moe_weights w;
    memset(&w, 0, sizeof w);
    w.format = fmt;
    w.gate = w.up = w.down = A;
    w.sh_gate = w.sh_up = w.sh_down = A;
    if (fmt != FLINT_WFMT_BF16) {
        w.gate_sf = w.up_sf = w.down_sf = A;
        w.sh_gate_sf = w.sh_up_sf = w.sh_down_sf = A;
    }
    if (fmt == FLINT_WFMT_NVFP4) {
        w.gate_ts = w.up_ts = w.down_ts = w.sh_ts = A;
    }
    return w;
}

int main(void)
{
    for (int s = -1; s < 9; s++)
        if (!flint_moe_status_string(s) || !flint_moe_status_string(s)[0]) failures++;
    /* sizing over the whole shape range, extremes included */
    const int Hs[] = {0, 32, 64, 320, 2048, 8192, 8256}, Is[] = {0, 16, 32, 96, 768, 4096, 4128};
    const int64_t Ts[] = {-1, 0, 1, 32, 33, 8192, 65536, 65537};
    for (int hi = 0; hi < 7; hi++)
        for (int ii = 0; ii < 7; ii++)
            for (int ti = 0; ti < 8; ti++)
                for (int fmt = -1; fmt < 4; fmt++) {
                    flint_moe_desc d = {Hs[hi], Is[ii], 256, 6, 1, 1};
                    size_t b = flint_moe_workspace_bytes(&d, Ts[ti], fmt);
                    const int ok_shape = Hs[hi] >= 64 && Hs[hi] <= 8192 && Is[ii] >= 32 && Is[ii] <= 4096 &&
                                         Hs[hi] % 64 == 0 && Is[ii] % 32 == 0 && Ts[ti] >= 0 && Ts[ti] <= 65536 &&
                                         fmt >= 0 && fmt <= 2 &&
                                         (fmt != 2 || (Hs[hi] % 128 == 0 && Is[ii] % 128 == 0));
                    if ((b != 0) != ok_shape) {
                        fprintf(stderr, "workspace_bytes H=%d I=%d T=%lld fmt=%d: %zu\n", Hs[hi], Is[ii],
                                (long long)Ts[ti], fmt, b);
                        failures++;
                    }
                }
    flint_moe_desc d = {2048, 768, 256, 6, 1, 1};
    const size_t need = flint_moe_workspace_bytes(&d, 8, FLINT_WFMT_BF16);
    flint_moe_weights wb = weights(FLINT_WFMT_BF16), wn = weights(FLINT_WFMT_NVFP4), wi = weights(FLINT_WFMT_INT4);
    /* route */
    expect(flint_moe_route(NULL, 1, A, A, NULL, NULL, A, A, 0, A, need, NULL), FLINT_ERR_NULL, "route desc");
    expect(flint_moe_route(&d, -1, A, A, NULL, NULL, A, A, 0, A, need, NULL), FLINT_ERR_SHAPE, "route T");
    expect(flint_moe_route(&d, 1, MIS, A, NULL, NULL, A, A, 0, A, need, NULL), FLINT_ERR_ALIGN, "route align");
    expect(flint_moe_route(&d, 1, A, A, NULL, NULL, A, A, 8, A, need, NULL), FLINT_ERR_FORMAT, "route flags");
    expect(flint_moe_route(&d, 1, A, A, NULL, NULL, A, A, 0, A, 16, NULL), FLINT_ERR_WORKSPACE, "route ws");
    /* permute */
    expect(flint_moe_permute(&d, 4, A, NULL, A, A, A, NULL, 0, NULL), FLINT_ERR_NULL, "permute null");
    expect(flint_moe_permute(&d, 70000, A, A, A, A, A, NULL, 0, NULL), FLINT_ERR_SHAPE, "permute T");
    /* forward */
    expect(flint_moe_forward(&d, &wb, 8, A, A, A, A, A, A, A, A, need - 1, NULL), FLINT_ERR_WORKSPACE, "forward ws");
    expect(flint_moe_forward(&d, &wb, 8, A, A, A, A, A, A, NULL, A, need, NULL), FLINT_ERR_NULL, "forward y");
    expect(flint_moe_forward(&d, &wn, 8, A, A, A, A, A, A, A, A, need - 1, NULL), FLINT_ERR_WORKSPACE, "forward nvfp4 ws");
    flint_moe_weights nots = wn;
    nots.sh_ts = NULL;
    expect(flint_moe_forward(&d, &nots, 8, A, A, A, A, A, A, A, A, need, NULL), FLINT_ERR_FORMAT, "forward nvfp4 sh_ts");
    flint_moe_weights bad = wb;
    bad.format = 7;
    expect(flint_moe_forward(&d, &bad, 8, A, A, A, A, A, A, A, A, need, NULL), FLINT_ERR_FORMAT, "forward format");
    flint_moe_desc d96 = {2048, 96, 256, 6, 1, 1};
    expect(flint_moe_forward(&d96, &wi, 8, A, A, A, A, A, A, A, A, need, NULL), FLINT_ERR_SHAPE, "forward int4 I=96");
    /* layer, layer_noalloc */
    expect(flint_moe_layer(&d, &wb, 4, A, NULL, NULL, A, NULL, A, need, NULL), FLINT_ERR_NULL, "layer router");
    expect(flint_moe_layer(&d, &wb, 4, A, A, NULL, A, NULL, MIS, need, NULL), FLINT_ERR_ALIGN, "layer ws align");
    flint_moe_routing r;
    memset(&r, 0, sizeof r);
    r.topk_w = MIS;
    expect(flint_moe_layer(&d, &wb, 4, A, A, NULL, A, &r, A, need, NULL), FLINT_ERR_ALIGN, "layer routing align");
    expect(flint_moe_layer_noalloc(&d, &wb, 4096, A, A, NULL, A, NULL, NULL), FLINT_ERR_WORKSPACE, "noalloc size");
    expect(flint_moe_layer_noalloc(&d, &wb, 4, A, A, NULL, NULL, NULL, NULL), FLINT_ERR_NULL, "noalloc y");
    /* decode chain */
    flint_moe_layer_ref lr[2];
    memset(lr, 0, sizeof lr);
    lr[0].weights = wb;
    lr[0].w_router = A;
    lr[1].weights = wn;
    lr[1].w_router = A;
    const size_t need1 = flint_moe_workspace_bytes(&d, 1, FLINT_WFMT_BF16);
    expect(flint_moe_decode_chain(&d, lr, 2, 0, 1, A, A, NULL, NULL, NULL, A, need1, NULL), FLINT_ERR_FORMAT, "chain formats");
    expect(flint_moe_decode_chain(&d, lr, 5000, 0, 1, A, A, NULL, NULL, NULL, A, need1, NULL), FLINT_ERR_SHAPE, "chain n");
    expect(flint_moe_decode_chain(&d, lr, 1, 0, 17, A, A, NULL, NULL, NULL, A, need1, NULL), FLINT_ERR_SHAPE, "chain T");
    expect(flint_moe_decode_chain(&d, lr, 1, 0, 1, A, A, NULL, NULL, NULL, A, need1 - 1, NULL), FLINT_ERR_WORKSPACE, "chain ws");
    /* workspace init / status */
    expect(flint_moe_workspace_init(MIS, need, NULL), FLINT_ERR_ALIGN, "init align");
    expect(flint_moe_workspace_init(A, 100, NULL), FLINT_ERR_WORKSPACE, "init size");
    expect(flint_moe_workspace_status(A, need, NULL, NULL), FLINT_ERR_NULL, "status out");
    printf("abi driver: %s\n", failures ? "FAILED" : "ok");
    return failures ? 1 : 0;
}
