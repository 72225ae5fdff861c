"""GPU parity: the HIP library (through the C ABI) against the reference on the same
seeded bytes.  See tests/moe_cases.py for the two-stage protocol and tolerances."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(__file__))

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
import sparse_moe_transformer_wave_amd as fm  # noqa: E402
from sparse_moe_transformer_wave_amd import datagen as dg  # noqa: E402
from moe_cases import Case, check_forward, check_routing, to_host  # noqa: E402


def _say(msg):
    print(msg, flush=True)


def _launches(ws):
    """Persistent launches made on a workspace: the head holds one launch counter per
    workgroup index (256 of them, all equal between launches)."""
    c = ws[fm.HEAD_COUNTERS:fm.HEAD_COUNTERS + 4 * 256].view(torch.int32).cpu().numpy()
    assert np.all(c == c[0]), "launch counters disagree"
    return int(c[0])


def _tile_edge_tokens(c, g, n_hot=4, bm=256):
    """Tokens in the first and the last row of every 256-row tile of the n_hot experts with
    the most rows and of the shared expert (slot T k + t holds token t), from the GPU's own
    grouping."""
    counts, off, sa = g["counts"], g["offsets"], g["sorted_assign"]
    toks = set()
    for e in np.argsort(-counts, kind="stable")[:n_hot]:
        n = int(counts[e])
        for m0 in range(0, n, bm):
            for r in (m0, min(m0 + bm, n) - 1):
                toks.add(int(sa[off[e] + r]) // c.k)
    for m0 in range(0, c.T, bm):
        toks.update((m0, min(m0 + bm, c.T) - 1))
    return np.array(sorted(toks), np.int64)


def _parity(c, steps=False, tokens=None):
    """tokens: None (all), an index array, or a function of the GPU's host-side outputs
    returning one (for samples chosen from the GPU's own grouping)."""
    _say("case T=%d H=%d I=%d E=%d k=%d S=%d fmt=%d" % (c.T, c.H, c.I, c.E, c.k, c.S, c.fmt))
    c.upload()
    g = c.run_steps() if steps else c.run_layer()
    rep = {}
    w64 = check_routing(c, g, rep)
    if callable(tokens):
        tokens = tokens(g)
        _say("  %d sampled tokens" % len(tokens))
    rm, rl = check_forward(c, g, w64, tokens)
    _say("  ok: max rel %.2e, rel L1 %.2e, near ties %s" % (rm, rl, rep.get("near_ties")))
    return g


# ---------------------------------------------------------------- tiny layer (H=256, I=128)
@pytest.mark.parametrize("T", [32, 1, 3, 8, 17, 31])
def test_tiny_streaming_path(T):
    _parity(Case(T, 256, 128, 256, 6))


@pytest.mark.parametrize("T", [33, 100, 257, 1000])
def test_tiny_grouped_gemm_path(T):
    _parity(Case(T, 256, 128, 256, 6))


@pytest.mark.parametrize("T", [1, 32, 300])
def test_tiny_three_call_path(T):
    _parity(Case(T, 256, 128, 256, 6), steps=True)


@pytest.mark.parametrize("T,E,k,S,renorm", [
    (5, 1, 1, 0, 1), (40, 1, 1, 1, 1), (7, 8, 8, 1, 1), (50, 8, 8, 0, 1),
    (9, 16, 4, 0, 0), (64, 16, 4, 1, 0), (3, 256, 8, 1, 1),
    # streaming path with experts of more than 16 tokens (split into 16-row units)
    (32, 8, 8, 1, 1), (24, 4, 4, 0, 1), (17, 2, 2, 1, 0)])
def test_edge_shapes(T, E, k, S, renorm):
    _parity(Case(T, 256, 128, E, k, S=S, renorm=renorm))


@pytest.mark.parametrize("T", [1, 8, 32, 40, 200])
def test_tiny_nvfp4(T):
    _parity(Case(T, 256, 128, 256, 6, fmt=fm.WFMT_NVFP4))


def test_zero_tokens_is_a_noop():
    c = Case(1, 256, 128, 256, 6).upload()
    y = torch.full((1, 256), 7, dtype=torch.int16, device="cuda")
    ws = c.workspace(1)
    fm.layer(c.desc, c.weights, 0, c.d_x, c.d_Wr, None, y, ws)
    torch.cuda.synchronize()
    assert torch.all(y == 7)


# ---------------------------------------------------------------- invariants on the GPU
def test_determinism_duplicates_scaling_permutation():
    T, H, I = 48, 256, 128
    x = dg.normal_bf16((T, H), 0, dg.stream_id(0, dg.KIND_X, 0), 1.0)
    x[7] = x[3]
    x[40] = x[3]
    for Tn in (T, 20):  # grouped-GEMM path and streaming path
        xs = np.ascontiguousarray(x[:Tn])
        c = Case(Tn, H, I, 256, 6, x=xs).upload()
        a, b = c.run_layer(), c.run_layer()
        np.testing.assert_array_equal(a["y"], b["y"])  # run-to-run bitwise
        np.testing.assert_array_equal(a["y"][7], a["y"][3])  # duplicate tokens bitwise
        if Tn > 40:
            np.testing.assert_array_equal(a["y"][40], a["y"][3])
        c2 = Case(Tn, H, I, 256, 6, x=xs, wscale=2.0).upload()
        d = c2.run_layer()
        np.testing.assert_array_equal(dg.bf16_bits_to_f32(d["y"]), 2 * dg.bf16_bits_to_f32(a["y"]))
        P = np.random.default_rng(5).permutation(Tn)
        c3 = Case(Tn, H, I, 256, 6, x=np.ascontiguousarray(xs[P])).upload()
        p = c3.run_layer()
        np.testing.assert_array_equal(p["topk_ids"], a["topk_ids"][P])
        ya, yp = dg.bf16_bits_to_f32(a["y"][P]), dg.bf16_bits_to_f32(p["y"])
        assert np.abs(ya - yp).max() <= 2e-2 * np.abs(ya).max()
        _say("permutation: bitwise equal rows %d of %d" % (int((a["y"][P] == p["y"]).all(1).sum()), Tn))


def test_route_logits_in_ties_signed_zero_nan():
    E, k, T = 256, 6, 64
    rng = np.random.default_rng(3)
    lg = rng.integers(-2, 3, (T, E)).astype(np.float32)  # heavy ties
    lg[0, :] = 0.0
    lg[1, ::2] = -0.0
    lg[2, 5] = np.nan
    lg[2, 9] = -np.inf
    lg[3, :] = -np.inf
    lg[3, 200] = np.nan
    d = fm.desc(256, 128, E, k, 1, 1)
    dl = torch.from_numpy(lg).cuda()
    ids = torch.zeros((T, k), dtype=torch.int32, device="cuda")
    w = torch.zeros((T, k), dtype=torch.float32, device="cuda")
    ws = fm.workspace(d, T)
    fm.route(d, T, None, None, None, ids, w, ws, logits=dl, logits_in=True)
    torch.cuda.synchronize()
    got = ids.cpu().numpy()
    ref_in = lg.astype(np.float64)
    ref_in[np.isnan(ref_in)] = -np.inf  # reading: NaN orders below -inf; rows 2, 3 checked by hand
    for t in range(T):
        if t in (2, 3):
            continue
        order = sorted(range(E), key=lambda e: (-ref_in[t, e], e))[:k]
        assert list(got[t]) == order
    # row 2: NaN at 5 ranks last, -inf at 9 next to last: top-6 are the 6 largest finite
    order2 = sorted([e for e in range(E) if e not in (5, 9)], key=lambda e: (-lg[2, e], e))[:k]
    assert list(got[2]) == order2
    # row 3: all -inf except a NaN: lowest indices 0..5 (the NaN, expert 200, is last)
    assert list(got[3]) == [0, 1, 2, 3, 4, 5]


# ---------------------------------------------------------------- full-size layer
_FULL = {}


def _full_case(T, fmt=fm.WFMT_BF16, bias_c=None, layer=0, routed_only=False):
    H, I, E, k = 2048, 768, 256, 6
    if fmt == fm.WFMT_BF16 and not routed_only:
        return Case(T, H, I, E, k, bias_c=bias_c, layer=layer)
    # Only the experts the reference routing touches get weights; the others hold zeros,
    # identically on both sides (a wrongly chosen expert would still show up as a mismatch).
    x = dg.normal_bf16((T, H), 0, dg.stream_id(layer, dg.KIND_X, 0), 1.0)
    Wr = dg.normal_f32((E, H), 0, dg.stream_id(layer, dg.KIND_ROUTER, 0), dg.ROUTER_STD)
    ids = oracle.select(oracle.router(x, Wr), k)
    return Case(T, H, I, E, k, fmt=fmt, layer=layer, experts=sorted(set(ids.reshape(-1).tolist())))


@pytest.mark.parametrize("T", [1, 8, 32])
def test_full_decode_bf16(T):
    _parity(_full_case(T))


@pytest.mark.parametrize("T", [1, 8, 32])
def test_full_decode_nvfp4(T):
    _parity(_full_case(T, fmt=fm.WFMT_NVFP4))


@pytest.mark.parametrize("zipf", [False, True])
def test_full_prefill_8192(zipf):
    """Routing on all 8192 tokens; y on a spread of tokens plus, from the GPU's grouping,
    the tokens in the first and last row of every 256-row tile of the four experts with the
    most rows (under the Zipf bias, the hot experts with up to ~18 tiles) and of the shared
    expert (32 tiles)."""
    c = _full_case(8192, bias_c=dg.ZIPF_C if zipf else None)
    spread = np.unique(np.concatenate([np.arange(0, 8192, 523), [8191]])).astype(np.int64)
    _parity(c, tokens=lambda g: np.union1d(spread, _tile_edge_tokens(c, g)))


@pytest.mark.parametrize("fmt", [fm.WFMT_BF16, fm.WFMT_NVFP4])
def test_single_token_launch_reuses_workspace(fmt):
    """T = 1 runs as one persistent launch whose workgroups exchange logits and h through
    launch-tagged words at the start of the workspace: consecutive calls on one workspace
    (each reading words the previous call tagged) all match the reference, the launch
    counters advance by one per call and no wait ever timed out."""
    d = fm.desc(2048, 768)
    ws = fm.workspace(d, 1, fmt)
    for n_call, layer in enumerate((0, 1, 2, 3, 0)):
        c = _full_case(1, fmt=fmt, layer=layer, routed_only=True).upload()
        out = c.alloc_out()
        routing = {kk: out[kk] for kk in ("logits", "topk_ids", "topk_w", "counts", "offsets",
                                          "sorted_assign", "assign_pos")}
        fm.layer(c.desc, c.weights, 1, c.d_x, c.d_Wr, None, out["y"], ws, routing)
        torch.cuda.synchronize()
        from moe_cases import to_host
        g = to_host(out, c)
        w64 = check_routing(c, g)
        rm, rl = check_forward(c, g, w64)
        assert fm.workspace_status(ws) == 0, "a wait timed out"
        assert _launches(ws) == n_call + 1
        _say("layer %d fmt %d: max rel %.2e rel L1 %.2e" % (layer, fmt, rm, rl))


# ---------------------------------------------------------------- NVFP4 prefill
def test_full_prefill_nvfp4_8192():
    """T = 8192 on the grouped NVFP4 path.  Weights for the experts of the sampled tokens
    (host quantisation of all 257 would take minutes); the other experts hold zeros on
    both sides, and their tiles still run."""
    H, I, E, k, T = 2048, 768, 256, 6, 8192
    toks = np.unique(np.concatenate([np.arange(0, T, 523), [T - 1]])).astype(np.int64)
    x = dg.normal_bf16((T, H), 0, dg.stream_id(0, dg.KIND_X, 0), 1.0)
    Wr = dg.normal_f32((E, H), 0, dg.stream_id(0, dg.KIND_ROUTER, 0), dg.ROUTER_STD)
    ids = oracle.select(oracle.router(x[toks], Wr), k)
    c = Case(T, H, I, E, k, fmt=fm.WFMT_NVFP4, experts=sorted(set(ids.reshape(-1).tolist())))
    _parity(c, tokens=toks)


# ---------------------------------------------------------------- dense SwiGLU layer
def _dense_check(T, H, I, fmt, layer=0, tokens=None, three_call=False, ws=None):
    """n_experts = 0: y = bf16(down(silu(gate x) * up x)) with the shared-expert pointers,
    against the reference's SwiGLU expert (sum in fp64) for each checked token."""
    _say("dense T=%d H=%d I=%d fmt=%d" % (T, H, I, fmt))
    c = Case(T, H, I, 0, 0, S=1, fmt=fmt, layer=layer).upload()
    w = c.weights
    w.gate = w.up = w.down = None
    w.gate_sf = w.up_sf = w.down_sf = w.gate_ts = w.up_ts = w.down_ts = None
    y = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    if ws is None:
        ws = c.workspace()
    if three_call:
        fm.forward(c.desc, w, T, c.d_x, None, None, None, None, None, y, ws)
    else:
        fm.layer(c.desc, w, T, c.d_x, None, None, y, ws)
    torch.cuda.synchronize()
    tok = np.arange(T) if tokens is None else tokens
    yg = dg.bf16_bits_to_f32(y.cpu().numpy().view(np.uint16)[tok]).astype(np.float64)
    xf = dg.bf16_bits_to_f32(c.x).astype(np.float64)
    ref = np.stack([oracle.expert_ffn(c.shared, 0, xf[t]) for t in tok])
    d = np.abs(yg - ref)
    assert np.all(np.isfinite(yg))
    rm, rl = d.max() / np.abs(ref).max(), d.sum() / np.abs(ref).sum()
    _say("  ok: max rel %.2e, rel L1 %.2e" % (rm, rl))
    from moe_cases import MAX_REL, MEAN_REL
    assert rm <= MAX_REL and rl <= MEAN_REL, (rm, rl)


@pytest.mark.parametrize("T", [1, 5, 32, 33, 300])
def test_dense_tiny(T):
    _dense_check(T, 256, 128, fm.WFMT_BF16)


def test_dense_tiny_three_call_and_nvfp4():
    _dense_check(7, 256, 128, fm.WFMT_BF16, three_call=True)
    _dense_check(40, 256, 128, fm.WFMT_BF16, three_call=True)
    for T in (1, 8, 100):
        _dense_check(T, 256, 256, fm.WFMT_NVFP4)


@pytest.mark.parametrize("T", [1, 8, 32])
def test_dense_full_decode(T):
    _dense_check(T, 2048, 4096, fm.WFMT_BF16, layer=1)


@pytest.mark.parametrize("H,I", [(2048, 1152), (512, 512), (1024, 2176), (256, 4096), (2048, 640)])
def test_dense_single_token_shapes(H, I):
    """One bf16 token of a dense layer with 512 <= I <= 4096 runs as one persistent launch:
    1 to 8 h words per workgroup (uneven for I = 640, 1152, 2176), 1 to 8 down rows each."""
    _dense_check(1, H, I, fm.WFMT_BF16, layer=2)


@pytest.mark.parametrize("fmt,H,I", [(fm.WFMT_NVFP4, 2048, 4096), (fm.WFMT_INT4, 2048, 4096),
                                     (fm.WFMT_NVFP4, 512, 640), (fm.WFMT_INT4, 2048, 640),
                                     (fm.WFMT_INT4, 1024, 2048)])
def test_dense_single_token_4bit(fmt, H, I):
    """The dense single-token launch with NVFP4 and INT4 weights: codes and scales of the
    down rows staged in LDS, uneven h words per workgroup for I = 640; through
    flint_moe_layer and through flint_moe_forward."""
    _dense_check(1, H, I, fmt, layer=4)
    _dense_check(1, H, I, fmt, layer=5, three_call=True)


def test_dense_and_moe_single_token_share_a_workspace():
    """The dense and the MoE single-token launches take turns on one workspace (the launch
    counter and the tagged words carry over from one to the other), through
    flint_moe_layer and flint_moe_forward."""
    c = Case(1, 2048, 768, 256, 6, layer=3)
    dd = fm.desc(2048, 4096, n_experts=0, top_k=0, n_shared=1)
    ws = torch.empty(max(fm.workspace_bytes(c.desc, 1), fm.workspace_bytes(dd, 1)),
                     dtype=torch.uint8, device="cuda")
    fm.workspace_init(ws)
    c.upload()
    for rep in range(3):
        _dense_check(1, 2048, 4096, fm.WFMT_BF16, layer=rep, three_call=rep == 1, ws=ws)
        out = c.alloc_out()
        routing = {k: out[k] for k in ("logits", "topk_ids", "topk_w", "counts", "offsets",
                                       "sorted_assign", "assign_pos")}
        fm.layer(c.desc, c.weights, 1, c.d_x, c.d_Wr, c.d_bias, out["y"], ws, routing)
        torch.cuda.synchronize()
        g = to_host(out, c)
        w64 = check_routing(c, g, {})
        check_forward(c, g, w64, None)
    assert fm.workspace_status(ws) == 0  # no wait ran out


def test_dense_full_prefill_8192():
    toks = np.unique(np.concatenate([np.arange(0, 8192, 1021), [8191]])).astype(np.int64)
    _dense_check(8192, 2048, 4096, fm.WFMT_BF16, layer=1, tokens=toks)


# ---------------------------------------------------------------- persistent decode chain
def _next_token(x_bits, y_bits, residual):
    """x_{l+1}: y_l, or bf16(x_l + y_l) from one fp32 sum (round to nearest even)."""
    if not residual:
        return y_bits.copy()
    s = (dg.bf16_bits_to_f32(x_bits).astype(np.float32) + dg.bf16_bits_to_f32(y_bits).astype(np.float32))
    return dg.f32_to_bf16_bits(s.astype(np.float32))


def _chain_check(H, I, E, k, fmt, L, residual, predict_experts=False, ws=None, T=1):
    """flint_moe_decode_chain over L layers for T tokens, each layer checked against the
    reference on the tokens the GPU fed it (recomputed on the host from the GPU's y of the
    previous layer), with the two-stage protocol of a layer call."""
    _say("chain T=%d H=%d I=%d E=%d k=%d fmt=%d L=%d residual=%d" % (T, H, I, E, k, fmt, L, residual))
    x0 = dg.normal_bf16((T, H), 0, dg.stream_id(0, dg.KIND_X, 0), dg.X_STD)
    cases = []
    xh = x0
    for l in range(L):
        experts = None
        if predict_experts:  # the reference's own chain decides which experts get weights
            Wr = dg.normal_f32((E, H), 0, dg.stream_id(l, dg.KIND_ROUTER, 0), dg.ROUTER_STD)
            experts = sorted(set(oracle.select(oracle.router(xh, Wr), k).reshape(-1).tolist()))
        c = Case(T, H, I, E, k, fmt=fmt, layer=l, experts=experts, x=xh).upload()
        cases.append(c)
        if predict_experts and l + 1 < L:
            lg = oracle.router(xh, c.Wr)
            ids = oracle.select(lg, k)
            yr = oracle.moe_tokens(c.routed, c.shared, xh, ids, oracle.weights(lg, ids, True))
            xh = _next_token(xh, dg.f32_to_bf16_bits(yr.astype(np.float32)), residual)
    d = cases[0].desc
    y = torch.zeros((L, T, H), dtype=torch.int16, device="cuda")
    ids = torch.zeros((L, T, k), dtype=torch.int32, device="cuda")
    tw = torch.zeros((L, T, k), dtype=torch.float32, device="cuda")
    lg = torch.zeros((L, T, E), dtype=torch.float32, device="cuda")
    ws = fm.workspace(d, T, fmt) if ws is None else ws
    fm.decode_chain(d, [(c.weights, c.d_Wr, None) for c in cases], cases[0].d_x, y, ws, ids, tw, lg,
                    residual=residual)
    torch.cuda.synchronize()
    yg, idg, twg, lgg = (t.cpu().numpy() for t in (y, ids, tw, lg))
    yg = yg.view(np.uint16)
    xl = x0
    for l, c in enumerate(cases):
        c.x = xl  # the token the GPU fed layer l
        g = {"logits": lgg[l], "topk_ids": idg[l], "topk_w": twg[l], "y": yg[l]}
        w64 = check_routing(c, g)
        rm, rl = check_forward(c, g, w64)
        _say("  layer %d: max rel %.2e, rel L1 %.2e" % (l, rm, rl))
        xl = _next_token(xl, yg[l], residual)
    assert fm.workspace_status(ws) == 0, "a wait timed out"
    return ws, _launches(ws)


@pytest.mark.parametrize("residual", [False, True])
def test_chain_tiny(residual):
    # Without the residual the token shrinks about quadratically per layer (x -> ~1e-2 ->
    # ~1e-6 -> ~1e-14 -> ~1e-30 here), and the fifth layer's h underflows fp32 while the fp64
    # reference keeps ~1e-62: four layers are the meaningful length of that chain.
    _chain_check(256, 128, 256, 6, fm.WFMT_BF16, 7 if residual else 4, residual)


def test_chain_tiny_two_launches_and_counter():
    """20 layers (the host gathers layer descriptors 16 at a time, so the token crosses
    that boundary too); the launch counters advance by one per layer, and a following
    single-token layer call on the same workspace is still correct."""
    ws, launches = _chain_check(256, 128, 256, 6, fm.WFMT_BF16, 20, True)
    assert launches == 20, launches
    c = Case(1, 256, 128, 256, 6, layer=3).upload()
    out = c.alloc_out()
    routing = {kk: out[kk] for kk in ("logits", "topk_ids", "topk_w", "counts", "offsets",
                                      "sorted_assign", "assign_pos")}
    fm.layer(c.desc, c.weights, 1, c.d_x, c.d_Wr, None, out["y"], ws, routing)
    torch.cuda.synchronize()
    from moe_cases import to_host
    g = to_host(out, c)
    check_forward(c, g, check_routing(c, g))
    assert _launches(ws) == 21 and fm.workspace_status(ws) == 0


def test_chain_tiny_nvfp4():
    # I = 256: a workgroup's NVFP4 down rows (codes + scales) must fill whole 16-byte chunks
    _chain_check(256, 256, 256, 6, fm.WFMT_NVFP4, 3, True)


@pytest.mark.parametrize("fmt", [fm.WFMT_BF16, fm.WFMT_NVFP4])
def test_chain_full(fmt):
    _chain_check(2048, 768, 256, 6, fmt, 3, True, predict_experts=True)


# ---------------------------------------------------------------- INT4 (W4A16)
@pytest.mark.parametrize("T", [1, 8, 32, 40, 200])
def test_tiny_int4(T):
    _parity(Case(T, 256, 128, 256, 6, fmt=fm.WFMT_INT4))


def test_int4_single_token_launch():
    """H = 1024, I = 768: the single-token persistent launch with INT4 rows (a workgroup's
    down rows, codes plus group scales, fill whole 16-byte chunks)."""
    _parity(Case(1, 1024, 768, 256, 6, fmt=fm.WFMT_INT4))


@pytest.mark.parametrize("T", [1, 8, 32])
def test_full_decode_int4(T):
    _parity(_full_case(T, fmt=fm.WFMT_INT4))


def test_full_prefill_int4_8192():
    H, I, E, k, T = 2048, 768, 256, 6, 8192
    toks = np.unique(np.concatenate([np.arange(0, T, 523), [T - 1]])).astype(np.int64)
    x = dg.normal_bf16((T, H), 0, dg.stream_id(0, dg.KIND_X, 0), 1.0)
    Wr = dg.normal_f32((E, H), 0, dg.stream_id(0, dg.KIND_ROUTER, 0), dg.ROUTER_STD)
    ids = oracle.select(oracle.router(x[toks], Wr), k)
    c = Case(T, H, I, E, k, fmt=fm.WFMT_INT4, experts=sorted(set(ids.reshape(-1).tolist())))
    _parity(c, tokens=toks)


def test_chain_full_int4():
    _chain_check(2048, 768, 256, 6, fm.WFMT_INT4, 3, True, predict_experts=True)


# ---------------------------------------------------------------- decode chains of a small batch
@pytest.mark.parametrize("T,residual", [(8, True), (8, False), (16, True), (2, True)])
def test_chain_batch_tiny(T, residual):
    """A small batch through the layers: each layer is the small-batch launch, which forms
    the next layer's tokens in its combine phase (two token buffers in the head, used in
    turn); every layer checked on the tokens the GPU fed it."""
    ws, launches = _chain_check(256, 128, 256, 6, fm.WFMT_BF16, 5 if residual else 4, residual, T=T)
    assert launches == (5 if residual else 4)


def test_chain_batch_crosses_the_descriptor_batches():
    """18 layers (the host gathers descriptors 16 at a time: the token buffer of layer 16
    comes from the previous batch's last launch), then a single-layer call on the same
    workspace."""
    ws, launches = _chain_check(256, 128, 256, 6, fm.WFMT_BF16, 18, True, T=8)
    assert launches == 18
    c = Case(8, 256, 128, 256, 6, layer=3).upload()
    out = c.alloc_out()
    fm.layer(c.desc, c.weights, 8, c.d_x, c.d_Wr, None, out["y"], ws,
             {kk: out[kk] for kk in ("logits", "topk_ids", "topk_w", "counts", "offsets",
                                     "sorted_assign", "assign_pos")})
    torch.cuda.synchronize()
    from moe_cases import to_host
    g = to_host(out, c)
    check_forward(c, g, check_routing(c, g))
    assert _launches(ws) == 19 and fm.workspace_status(ws) == 0


@pytest.mark.parametrize("fmt", [fm.WFMT_BF16, fm.WFMT_NVFP4, fm.WFMT_INT4])
def test_chain_batch_full(fmt):
    _chain_check(2048, 768, 256, 6, fmt, 3, True, predict_experts=True, T=8)


# ---------------------------------------------------------------- HIP graph replay
@pytest.mark.parametrize("T", [1, 8, 100])
def test_graph_replays_match_eager(T):
    """The layer captured in a HIP graph (as the benchmark runs it), replayed several times
    with eager calls on the same workspace in between: every replay gives the eager
    result bit for bit (the persistent launches' tags come from the launch counters in
    device memory, so replays never reuse a tag; nothing is cleared with a memset node)."""
    c = Case(T, 256, 128, 256, 6, layer=2).upload()
    ws = c.workspace()
    y_eager = torch.zeros((T, 256), dtype=torch.int16, device="cuda")
    fm.layer(c.desc, c.weights, T, c.d_x, c.d_Wr, None, y_eager, ws)
    torch.cuda.synchronize()
    ref = y_eager.clone()
    y_graph = torch.zeros_like(y_eager)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fm.layer(c.desc, c.weights, T, c.d_x, c.d_Wr, None, y_graph, ws)  # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for _ in range(3):
            fm.layer(c.desc, c.weights, T, c.d_x, c.d_Wr, None, y_graph,
                     ws, stream=torch.cuda.current_stream().cuda_stream)
    for rep in range(3):
        y_graph.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_graph, ref), "replay %d differs from the eager result" % rep
        fm.layer(c.desc, c.weights, T, c.d_x, c.d_Wr, None, y_eager, ws)  # eager work in between
        torch.cuda.synchronize()
        assert torch.equal(y_eager, ref)
    if T == 1:
        assert fm.workspace_status(ws) == 0, "a wait timed out"
