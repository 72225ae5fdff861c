"""GPU parity on the edges of the method and of the boundary, through the C ABI, against the
reference (tests/moe_cases.py has the two-stage protocol and the tolerances):

  * ties at the k-th place through every selector: the single-token launch (T = 1), the
    small-batch router launch (T = 8, 32) and the batched top-k (T = 64), with router rows
    repeated so that equal fp32 logits straddle the 6th and 7th place, and with zero router
    rows, +-0 and -inf logit biases;
  * the single-token launch's branches: k in {1, 5, 7, 8}, no shared expert, E in {1, 8, 100},
    unnormalised weights;
  * NVFP4 dequantisation over every finite E4M3 block-scale code (subnormals and zero
    included) and all 16 E2M1 codes, on the single-token launch, the streaming kernels and
    the grouped GEMMs, checked column by column;
  * assignments with expert ids outside [0, E) (dropped);
  * a timed-out wait of a persistent launch, forced from the host, reported and cleared;
  * shapes with H % 256 != 0 and I % 128 != 0, among them one GPU's share of the layer split
    eight ways over I (I = 96);
  * the device-drawn benchmark pools against the host generator and the reference's
    quantisers.
"""
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
from moe_cases import MAX_REL, MEAN_REL, Case, check_forward, check_routing, to_host  # noqa: E402


def _say(msg):
    print(msg, flush=True)


def _launches(ws):
    """Persistent launches made on a workspace: the head holds one launch counter per
    workgroup index (256 of them, all equal between launches)."""
    c = ws[fm.HEAD_COUNTERS:fm.HEAD_COUNTERS + 4 * 256].view(torch.int32).cpu().numpy()
    assert np.all(c == c[0]), "launch counters disagree"
    return int(c[0])


def _run(c, ws=None):
    """flint_moe_layer on a case (uploaded here), every routing output returned."""
    c.upload()
    out = c.alloc_out()
    ws = c.workspace() if ws is None else ws
    routing = {k: out[k] for k in ("logits", "topk_ids", "topk_w", "counts", "offsets",
                                   "sorted_assign", "assign_pos")}
    fm.layer(c.desc, c.weights, c.T, c.d_x, c.d_Wr, c.d_bias, out["y"], ws, routing)
    torch.cuda.synchronize()
    return to_host(out, c), ws


def _check(c, g, tokens=None):
    rep = {}
    w64 = check_routing(c, g, rep)
    rm, rl = check_forward(c, g, w64, tokens)
    _say("  ok: max rel %.2e, rel L1 %.2e, near ties %s" % (rm, rl, rep.get("near_ties")))


def _routed_experts(T, H, E, k, layer=0, Wr=None, bias=None, x=None):
    """Experts the reference's own routing touches (the only ones given weights in the
    full-size cases; the others hold zeros on both sides)."""
    x = dg.normal_bf16((T, H), 0, dg.stream_id(layer, dg.KIND_X, 0), dg.X_STD) if x is None else x
    if Wr is None:
        Wr = dg.normal_f32((E, H), 0, dg.stream_id(layer, dg.KIND_ROUTER, 0), dg.ROUTER_STD)
    return sorted(set(oracle.select(oracle.router(x, Wr, bias), k).reshape(-1).tolist()))


# ---------------------------------------------------------------- ties through every selector
def _repeated_rows(E, H, groups, layer=0):
    """Router weights where expert e has row e % groups: experts e, e + groups, ... get
    bit-identical fp32 logits on every path (same row, same summation), so each token's
    6th and 7th places are taken from a group of equal logits and the lowest indices win."""
    R = dg.normal_f32((groups, H), 0, dg.stream_id(layer, dg.KIND_ROUTER, 0), dg.ROUTER_STD)
    return np.ascontiguousarray(R[np.arange(E) % groups])


@pytest.mark.parametrize("T", [1, 8, 32, 64])
def test_ties_from_repeated_router_rows_tiny(T):
    H, I, E, k = 256, 128, 256, 6
    c = Case(T, H, I, E, k)
    c.Wr = _repeated_rows(E, H, 64)  # 4-way ties everywhere: places 5-8 are always a tie
    g, ws = _run(c)
    ids = g["topk_ids"]
    # the top group (4 equal logits) is taken whole, then the 2 lowest of the second group
    assert np.all(ids[:, :4] % 64 == ids[:, :1] % 64) and np.all(np.diff(ids[:, :4], axis=1) > 0)
    assert np.all(ids[:, 4:] % 64 == ids[:, 4:5] % 64) and np.all(ids[:, 5] - ids[:, 4] == 64)
    assert np.all(ids[:, 4] == ids[:, 4] % 64)  # lowest index of its group
    if T == 1:
        assert _launches(ws) == 1, "the single-token launch ran"
    _check(c, g)


@pytest.mark.parametrize("T", [1, 8])
def test_ties_from_repeated_router_rows_full(T):
    H, I, E, k = 2048, 768, 256, 6
    Wr = _repeated_rows(E, H, 96)  # experts e, e + 96, e + 192 share a row
    c = Case(T, H, I, E, k, experts=_routed_experts(T, H, E, k, Wr=Wr))
    c.Wr = Wr
    g, ws = _run(c)
    if T == 1:
        assert _launches(ws) == 1
    _check(c, g)


def _special_bias(E, zero_rows, signed=True):
    """-inf bias everywhere but `zero_rows`, whose bias is +0 or -0 (alternately); with
    zero router rows those logits are exactly +0 (x * 0 sums to +0, and +0 + -0 = +0)."""
    b = np.full(E, -np.inf, np.float32)
    for i, e in enumerate(zero_rows):
        b[e] = -0.0 if (signed and i % 2) else 0.0
    return b


@pytest.mark.parametrize("T", [1, 8, 32, 64])
@pytest.mark.parametrize("n_zero", [16, 3])
def test_zero_and_minus_inf_logits(T, n_zero):
    """n_zero = 16: every token's top 6 are the 6 lowest indices of 16 experts tied at
    logit +0 (weights 1/6).  n_zero = 3: the 3 zero experts, then the 3 lowest-index
    experts among those at -inf (weights 1/3, 1/3, 1/3, 0, 0, 0)."""
    H, I, E, k = 256, 128, 256, 6
    c = Case(T, H, I, E, k)
    zero = sorted(np.random.default_rng(11 + n_zero).choice(E, n_zero, replace=False).tolist())
    Wr = c.Wr.copy()
    Wr[zero] = 0.0
    c.Wr = Wr
    c.bias = _special_bias(E, zero)
    g, ws = _run(c)
    if n_zero == 16:
        assert np.all(g["topk_ids"] == np.array(zero[:6])[None, :])
        assert np.all(np.abs(g["topk_w"] - 1.0 / 6) <= 1e-6)
    else:
        rest = [e for e in range(E) if e not in zero][:3]
        assert np.all(g["topk_ids"] == np.array(zero + rest)[None, :])
        assert np.all(g["topk_w"][:, 3:] == 0.0)
    assert np.all(g["logits"][:, zero] == 0.0) and not np.any(np.signbit(g["logits"][:, zero]))
    _check(c, g)


# ---------------------------------------------------------------- single-token launch branches
_BRANCHES = [(256, 1, 1, 1), (256, 5, 1, 1), (256, 7, 1, 1), (256, 8, 1, 1), (256, 6, 0, 1),
             (1, 1, 1, 1), (8, 8, 0, 1), (100, 7, 1, 0), (256, 6, 1, 0)]


@pytest.mark.parametrize("E,k,S,renorm", _BRANCHES)
def test_single_token_branches_tiny(E, k, S, renorm):
    """Odd k (the shared slot shares an h word with slot k - 1), no shared expert, fewer
    than 256 experts (workgroups past E publish no logit) and raw sigmoid weights."""
    c = Case(1, 256, 128, E, k, S=S, renorm=renorm)
    g, ws = _run(c)
    assert _launches(ws) == 1, "the single-token launch ran"
    _check(c, g)


@pytest.mark.parametrize("E,k,S,renorm", _BRANCHES)
def test_single_token_branches_full(E, k, S, renorm):
    H, I = 2048, 768
    c = Case(1, H, I, E, k, S=S, renorm=renorm, experts=_routed_experts(1, H, E, k))
    g, ws = _run(c)
    assert _launches(ws) == 1
    _check(c, g)


# ---------------------------------------------------------------- NVFP4 scale-code sweep
_FINITE_E4M3 = [cde for cde in range(256) if (cde & 0x7F) != 0x7F]  # 254 codes, +-0 included


def _nvfp4_sweep_case(T, H, I):
    """One routed expert (E = 1, k = 1, no shared expert, so y = o exactly with weight 1)
    whose NVFP4 weights walk the code space:
      gate row i: block scale code i mod 127 (every non-negative finite E4M3 code, 0x00 and
        the subnormals 0x01-0x07 included), element codes 1-7 (positive);
      up row i: block scale code (37 i + 11) mod 127, element codes 1-7;
      down row n: all codes 0 or 8 (+0, -0) except column n mod I, which holds code
        1 + n mod 15 (every nonzero E2M1 code, negative ones included) under a block scale
        that walks all 254 finite E4M3 codes, negative ones included.
    x is positive, so g, u > 0 and y[t][n] = e4m3(sd(n)) e2m1(m(n)) h[t][n mod I]: every
    output column carries one down scale code and one (gate, up) scale pair, and a wrong
    scale in any of them shows in that column."""
    rng = np.random.default_rng(7)
    c = Case(T, H, I, 1, 1, S=0, fmt=fm.WFMT_NVFP4, experts=[])
    x = np.abs(rng.standard_normal((T, H))) + 0.25
    c.x = dg.f32_to_bf16_bits(x.astype(np.float32))

    def pack(codes):
        return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)

    gq = rng.integers(1, 8, (I, H)).astype(np.uint8)
    uq = rng.integers(1, 8, (I, H)).astype(np.uint8)
    gs = (np.arange(I)[:, None] % 127 + np.zeros((1, H // 16), int)).astype(np.uint8)
    us = ((37 * np.arange(I) + 11)[:, None] % 127 + np.zeros((1, H // 16), int)).astype(np.uint8)
    dq = (rng.integers(0, 2, (H, I)) * 8).astype(np.uint8)  # +0 or -0
    ds = rng.choice(_FINITE_E4M3, (H, I // 16)).astype(np.uint8)
    for n in range(H):
        col = n % I
        dq[n, col] = 1 + n % 15
        ds[n, col // 16] = _FINITE_E4M3[n % len(_FINITE_E4M3)]
    host = {"q_gate": pack(gq)[None], "sb_gate": gs[None], "st_gate": np.ones(1, np.float32),
            "q_up": pack(uq)[None], "sb_up": us[None], "st_up": np.ones(1, np.float32),
            "q_down": pack(dq)[None], "sb_down": ds[None], "st_down": np.ones(1, np.float32)}
    c.host = host
    c.routed = oracle.Experts(oracle.FMT_NVFP4, H, I, host)
    return c


@pytest.mark.parametrize("H,I", [(256, 256), (2048, 768), (320, 96)])
@pytest.mark.parametrize("T", [1, 8, 64])
def test_nvfp4_scale_code_sweep(T, H, I):
    c = _nvfp4_sweep_case(T, H, I)
    g, ws = _run(c)
    assert np.all(g["topk_ids"] == 0) and np.all(g["topk_w"] == 1.0)
    ref = oracle.moe_tokens(c.routed, None, c.x, g["topk_ids"], np.ones((T, 1)))
    y = dg.bf16_bits_to_f32(g["y"]).astype(np.float64)
    assert np.all(np.isfinite(y))
    zero = ref == 0.0
    assert np.all(y[zero] == 0.0), "a zero scale or zero h must give an exact zero"
    rel = np.abs(y[~zero] - ref[~zero]) / np.abs(ref[~zero])
    # h, the per-slot output (grouped path) and y are each rounded to bf16 once (2^-9 each)
    _say("  H=%d I=%d T=%d: %d zero columns, max column rel err %.2e" % (H, I, T, int(zero.sum()), rel.max()))
    assert rel.max() <= 1e-2, "worst column %d" % int(np.argmax(rel))


# ---------------------------------------------------------------- dropped assignments
@pytest.mark.parametrize("T", [8, 64, 2000])
def test_out_of_range_ids_are_dropped(T):
    """route -> permute -> forward with a few ids replaced by -1, E and 1000: permute leaves
    those assignments out (assign_pos -1, sorted_assign -1 past offsets[E]) and forward's
    combine skips them, which matches the reference with those terms given weight 0.
    T = 2000 takes the multi-block grouping (T k > 4096)."""
    H, I, E, k = 256, 128, 256, 6
    c = Case(T, H, I, E, k).upload()
    out = c.alloc_out()
    ws = c.workspace()
    fm.route(c.desc, T, c.d_x, c.d_Wr, None, out["topk_ids"], out["topk_w"], ws, logits=out["logits"])
    torch.cuda.synchronize()
    ids0 = out["topk_ids"].cpu().numpy()
    ids = ids0.copy()
    rng = np.random.default_rng(T)
    bad = rng.random(ids.shape) < 0.05
    bad[0, 0] = True
    ids[bad] = rng.choice([-1, E, 1000], int(bad.sum()))
    out["topk_ids"].copy_(torch.from_numpy(ids))
    fm.permute(c.desc, T, out["topk_ids"], out["counts"], out["offsets"], out["sorted_assign"],
               out["assign_pos"], ws)
    fm.forward(c.desc, c.weights, T, c.d_x, out["topk_ids"], out["topk_w"], out["offsets"],
               out["sorted_assign"], out["assign_pos"], out["y"], ws)
    torch.cuda.synchronize()
    g = to_host(out, c)
    flat = ids.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    a_valid = np.nonzero(valid)[0]
    order = a_valid[np.argsort(flat[a_valid], kind="stable")]  # grouped by expert, a ascending
    counts = np.bincount(flat[a_valid], minlength=E)
    np.testing.assert_array_equal(g["counts"], counts)
    np.testing.assert_array_equal(g["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    sa = np.full(T * k, -1, np.int64)
    sa[:order.size] = order
    np.testing.assert_array_equal(g["sorted_assign"], sa)
    ap = np.full(T * k, -1, np.int64)
    ap[order] = np.arange(order.size)
    np.testing.assert_array_equal(g["assign_pos"], ap)
    # route's weights were renormalised over the original ids; a dropped term has weight 0
    w64 = oracle.weights(g["logits"].astype(np.float64), ids0, True)
    w64[bad] = 0.0
    g["topk_ids"] = np.where(bad, 0, ids).astype(np.int32)
    rm, rl = check_forward(c, g, w64)
    _say("  %d dropped assignments; max rel %.2e, rel L1 %.2e" % (int(bad.sum()), rm, rl))


# ---------------------------------------------------------------- timed-out waits
def _set_diag(ws, v):
    ws[fm.HEAD_DIAG:fm.HEAD_DIAG + 4].view(torch.int32).fill_(v)
    torch.cuda.synchronize()


@pytest.mark.parametrize("kind", ["moe", "few", "select", "dense", "chain"])
def test_forced_timeout_is_reported_and_cleared(kind):
    """The head's diagnostic switch makes every bounded wait give up at once (the kernels
    still end normally): the status call reports FLINT_WS_WAIT_TIMEOUT once and clears it,
    and the next call on the same workspace, with the switch off, is correct again (its
    exchange words carry a new launch tag, so none of the abandoned launch's words match)."""
    H, I = 256, 128
    if kind == "dense":
        c = Case(1, H, 512, 0, 0, S=1)
        c.upload()
        w = c.weights
        w.gate = w.up = w.down = None
        ws = c.workspace()
        y = torch.zeros((1, H), dtype=torch.int16, device="cuda")

        def call():
            fm.layer(c.desc, w, 1, c.d_x, None, None, y, ws)
            torch.cuda.synchronize()
    elif kind in ("moe", "few", "select"):  # one token; small batches (every wait gives up)
        # 24 tokens: the router launch's two selecting workgroups, and their second wait
        c = Case({"moe": 1, "few": 8, "select": 24}[kind], H, I, 256, 6).upload()
        ws = c.workspace()

        def call():
            return _run(c, ws)[0]
    else:
        c = Case(1, H, I, 256, 6).upload()
        ws = c.workspace()
        yl = torch.zeros((2, H), dtype=torch.int16, device="cuda")

        def call():
            fm.decode_chain(c.desc, [(c.weights, c.d_Wr, None)] * 2, c.d_x, yl, ws, residual=True)
            torch.cuda.synchronize()
    assert fm.workspace_status(ws) == 0
    _set_diag(ws, 1)
    call()
    assert fm.workspace_status(ws) == fm.WS_WAIT_TIMEOUT
    assert fm.workspace_status(ws) == 0, "the status call clears the flags"
    _set_diag(ws, 0)
    g = call()
    assert fm.workspace_status(ws) == 0
    n_launch = 2 if kind != "chain" else 4
    assert _launches(ws) == n_launch
    if kind in ("moe", "few", "select"):
        _check(c, g)
    elif kind == "dense":
        ref = oracle.expert_ffn(c.shared, 0, dg.bf16_bits_to_f32(c.x[0]).astype(np.float64))
        yg = dg.bf16_bits_to_f32(y.cpu().numpy().view(np.uint16)[0]).astype(np.float64)
        d = np.abs(yg - ref)
        assert d.max() <= MAX_REL * np.abs(ref).max() and d.sum() <= MEAN_REL * np.abs(ref).sum()
    else:  # the chain's first layer: y_0 = layer(x)
        y0 = yl.cpu().numpy().view(np.uint16)[:1]
        lg = oracle.router(c.x, c.Wr)
        ids = oracle.select(lg, 6)
        ref = oracle.moe_tokens(c.routed, c.shared, c.x, ids, oracle.weights(lg, ids, True))
        d = np.abs(dg.bf16_bits_to_f32(y0).astype(np.float64) - ref)
        assert d.max() <= MAX_REL * np.abs(ref).max() and d.sum() <= MEAN_REL * np.abs(ref).sum()


# ---------------------------------------------------------------- shapes past the 256/128 grid
@pytest.mark.parametrize("fmt", [fm.WFMT_BF16, fm.WFMT_NVFP4])
@pytest.mark.parametrize("H,I", [(320, 96), (192, 160), (64, 64)])
@pytest.mark.parametrize("T", [1, 8, 33, 300])
def test_shapes_h64_i32(T, H, I, fmt):
    """H a multiple of 64 but not of 128 or 256, I a multiple of 32 but not of 128: K tails
    in the streaming kernels, partial N tiles in the grouped GEMMs and, for NVFP4, the
    register-staged GEMM with zeros past K; T = 1 takes the small-batch router launch (the
    single-token launch needs H % 256 == 0), T = 8 with bf16 weights the one-launch
    small-batch layer and with NVFP4 weights the router launch: each one persistent launch.  bf16 grouped GEMMs: I % 64 == 32 sends the down pass to the 32-wide
    ring; H = I = 64 runs both passes on the 64-wide kernel with a single K stage."""
    _say("case T=%d H=%d I=%d fmt=%d" % (T, H, I, fmt))
    c = Case(T, H, I, 256, 6, fmt=fmt)
    g, ws = _run(c)
    assert _launches(ws) == (1 if T <= 32 else 0)
    _check(c, g)


@pytest.mark.parametrize("T", [1, 40])
def test_int4_h_multiple_of_128(T):
    c = Case(T, 384, 128, 256, 6, fmt=fm.WFMT_INT4)
    g, _ = _run(c)
    _check(c, g)


@pytest.mark.parametrize("fmt", [fm.WFMT_BF16, fm.WFMT_NVFP4])
@pytest.mark.parametrize("T", [1, 8, 32])
def test_tp8_share_decode(T, fmt):
    """One GPU's share of the layer split eight ways over I (H = 2048, I = 768 / 8 = 96):
    T = 1 runs the single-token launch with 0 or 1 gate/up rows per workgroup."""
    H, I, E, k = 2048, 96, 256, 6
    c = Case(T, H, I, E, k, fmt=fmt, experts=_routed_experts(T, H, E, k))
    g, ws = _run(c)
    if T == 1:
        assert _launches(ws) == 1
    _check(c, g)


@pytest.mark.parametrize("fmt", [fm.WFMT_BF16, fm.WFMT_NVFP4])
def test_tp8_share_prefill_8192(fmt):
    """The same share at T = 8192: 192-row gate/up tiles, K = 96 for down (NVFP4: the
    register-staged GEMM).  Weights for the sampled tokens' experts only."""
    H, I, E, k, T = 2048, 96, 256, 6, 8192
    toks = np.unique(np.concatenate([np.arange(0, T, 401), [T - 1]])).astype(np.int64)
    x = dg.normal_bf16((T, H), 0, dg.stream_id(0, dg.KIND_X, 0), dg.X_STD)
    c = Case(T, H, I, E, k, fmt=fmt, experts=_routed_experts(len(toks), H, E, k, x=x[toks]))
    g, _ = _run(c)
    _check(c, g, tokens=toks)


@pytest.mark.parametrize("T", [1, 40])
def test_dense_h64_i32(T):
    """Dense layer (E = 0) off the 256/128 grid: the streaming units, or the grouped GEMMs."""
    H, I = 320, 96
    c = Case(T, H, I, 0, 0, S=1).upload()
    w = c.weights
    w.gate = w.up = w.down = None
    y = torch.zeros((T, H), dtype=torch.int16, device="cuda")
    fm.layer(c.desc, w, T, c.d_x, None, None, y, c.workspace())
    torch.cuda.synchronize()
    xf = dg.bf16_bits_to_f32(c.x).astype(np.float64)
    ref = np.stack([oracle.expert_ffn(c.shared, 0, xf[t]) for t in range(T)])
    yg = dg.bf16_bits_to_f32(y.cpu().numpy().view(np.uint16)).astype(np.float64)
    d = np.abs(yg - ref)
    assert d.max() <= MAX_REL * np.abs(ref).max() and d.sum() <= MEAN_REL * np.abs(ref).sum()


# ---------------------------------------------------------------- benchmark pools
def test_device_pools_match_host_generator_and_reference_quantisers():
    """The benchmark draws its pools on the device.  One layer's bf16 matrices equal the host
    generator's bytes (the device's log/cos/sin may differ from the host's in a last bit,
    which can move a rare element by one bf16 step), and the device NVFP4 and INT4
    quantisers give the reference quantisers' codes and scales on the same draws."""
    N, K, n_mat = 768, 2048, 2
    sid = dg.stream_id(5, dg.KIND_GATE, 0)
    t = torch.empty((n_mat, N, K), dtype=torch.int16, device="cuda")
    dg.device_normal_bf16(t, n_mat, N * K, 0, sid, dg.W_STD)
    dev = t.cpu().numpy().view(np.uint16)
    for m in range(n_mat):
        host = dg.normal_bf16((N, K), 0, sid + m, dg.W_STD)
        diff = dev[m] != host
        step = np.abs(dev[m].astype(np.int32) - host.astype(np.int32))
        _say("  bf16 matrix %d: %d of %d elements differ" % (m, int(diff.sum()), host.size))
        assert diff.mean() <= 1e-5 and np.all(step[diff] == 1)
    q = torch.empty((n_mat, N, K // 2), dtype=torch.uint8, device="cuda")
    sf = torch.empty((n_mat, N, K // 16), dtype=torch.uint8, device="cuda")
    ts = torch.empty(n_mat + 3, dtype=torch.float32, device="cuda")
    scratch = torch.empty(n_mat, dtype=torch.int32, device="cuda")
    dg.device_nvfp4(q, sf, ts, scratch, n_mat, N, K, 0, sid, dg.W_STD)
    qi = torch.empty((n_mat, N, K // 2), dtype=torch.uint8, device="cuda")
    sc = torch.empty((n_mat, N, K // 128), dtype=torch.int16, device="cuda")
    dg.device_int4(qi, sc, n_mat, N, K, 0, sid, dg.W_STD)
    torch.cuda.synchronize()
    qd, sfd, tsd = q.cpu().numpy(), sf.cpu().numpy(), ts.cpu().numpy()
    qid, scd = qi.cpu().numpy(), sc.cpu().numpy().view(np.uint16)
    for m in range(n_mat):
        W = dg.normal_f64((N, K), 0, sid + m, dg.W_STD)
        rq, rsb, rst = oracle.nvfp4_quantize(W)
        assert np.float32(rst) == tsd[m]
        assert np.mean(sfd[m] != rsb) <= 1e-5 and np.mean(qd[m] != rq) <= 1e-5
        iq, isc = oracle.int4_quantize(W)
        assert np.mean(scd[m] != isc) <= 1e-5 and np.mean(qid[m] != iq) <= 1e-5
        _say("  nvfp4 matrix %d: %d code bytes, %d scales differ; int4: %d, %d"
             % (m, int((qd[m] != rq).sum()), int((sfd[m] != rsb).sum()), int((qid[m] != iq).sum()),
                int((scd[m] != isc).sum())))
