"""GPU parity of the small-batch layer launch (2 <= T <= 16 tokens through flint_moe_layer:
one persistent launch that routes, selects, streams the touched experts and combines),
against the reference on the same seeded bytes, with the two-stage protocol of
tests/moe_cases.py.  Each case also checks that the launch ran (the workspace head's launch
counters advance by one per call) and that no wait timed out."""
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
    c = ws[fm.HEAD_COUNTERS:fm.HEAD_COUNTERS + 4 * 256].view(torch.int32).cpu().numpy()
    assert np.all(c == c[0]), "launch counters disagree"
    return int(c[0])


def _layer(c, ws):
    """flint_moe_layer on an uploaded case, every routing output returned."""
    out = c.alloc_out()
    routing = {k: out[k] for k in ("logits", "topk_ids", "topk_w", "counts", "offsets",
                                   "sorted_assign", "assign_pos")}
    fm.layer(c.desc, c.weights, c.T, c.d_x, c.d_Wr, c.d_bias, out["y"], ws, routing)
    torch.cuda.synchronize()
    return to_host(out, c)


def _parity(c, ws=None, launches_before=0):
    """flint_moe_layer takes the small-batch launch for bf16 weights; 4-bit weights go
    through it in a decode chain (here: a chain of one layer)."""
    _say("case T=%d H=%d I=%d E=%d k=%d S=%d renorm=%d fmt=%d" % (c.T, c.H, c.I, c.E, c.k, c.S, c.renorm, c.fmt))
    c.upload()
    ws = c.workspace() if ws is None else ws
    if c.fmt == fm.WFMT_BF16:
        g = _layer(c, ws)
    else:
        out = c.alloc_out()
        fm.decode_chain(c.desc, [(c.weights, c.d_Wr, c.d_bias)], c.d_x, out["y"], ws,
                        topk_ids=out["topk_ids"], topk_w=out["topk_w"], logits=out["logits"])
        torch.cuda.synchronize()
        g = to_host(out, c)
        for key in ("counts", "offsets", "sorted_assign", "assign_pos"):  # a chain returns none
            del g[key]
    assert _launches(ws) == launches_before + 1, "the small-batch launch ran"
    assert fm.workspace_status(ws) == 0, "no wait timed out"
    rep = {}
    w64 = check_routing(c, g, rep)
    rm, rl = check_forward(c, g, w64)
    _say("  ok: max rel %.2e, rel L1 %.2e, near ties %s" % (rm, rl, rep.get("near_ties")))
    return g, ws


@pytest.mark.parametrize("T", [2, 3, 8, 9, 15, 16])
def test_few_tiny_bf16(T):
    """Token counts across the range, including 9 and 16 (tokens 8-15 take the second
    selection round of each wave) and odd counts."""
    _parity(Case(T, 256, 128, 256, 6))


@pytest.mark.parametrize("fmt", [fm.WFMT_NVFP4, fm.WFMT_INT4])
@pytest.mark.parametrize("T", [2, 8, 16])
def test_few_tiny_4bit(T, fmt):
    _parity(Case(T, 256, 128, 256, 6, fmt=fmt))


@pytest.mark.parametrize("T,E,k,S,renorm", [
    (2, 1, 1, 1, 1), (16, 1, 1, 0, 1), (8, 8, 8, 1, 1), (16, 8, 8, 0, 0), (12, 100, 5, 1, 0),
    (16, 256, 8, 1, 1), (5, 256, 7, 0, 1), (10, 256, 1, 1, 1), (4, 3, 2, 1, 1)])
def test_few_branches(T, E, k, S, renorm):
    """E below 256 (workgroups past E compute no logit), every k, no shared expert (the units
    are then the touched experts alone), renormalize off, and experts picked by every token
    (E = 1: one unit holds all T tokens, like the shared expert)."""
    _parity(Case(T, 256, 128, E, k, S=S, renorm=renorm))


@pytest.mark.parametrize("H,I", [(512, 1024), (2048, 32), (1024, 96), (64, 64)])
def test_few_shapes(H, I):
    """The K split over the 7 streaming waves with the most chunks (I = 1024: 5 per wave in
    the down pass), with fewer chunks than waves (I = 32, 96; H = 64), and blocks that end
    inside a unit."""
    _parity(Case(8, H, I, 64, 6))


def _full(T, fmt, layer=0):
    H, I, E, k = 2048, 768, 256, 6
    x = dg.normal_bf16((T, H), 0, dg.stream_id(layer, dg.KIND_X, 0), dg.X_STD)
    Wr = dg.normal_f32((E, H), 0, dg.stream_id(layer, dg.KIND_ROUTER, 0), dg.ROUTER_STD)
    ids = oracle.select(oracle.router(x, Wr), k)
    # only the experts the reference routing touches get weights (zeros elsewhere, on both
    # sides: a wrongly chosen expert still shows up as a mismatch)
    return Case(T, H, I, E, k, fmt=fmt, layer=layer, experts=sorted(set(ids.reshape(-1).tolist())))


@pytest.mark.parametrize("fmt", [fm.WFMT_BF16, fm.WFMT_NVFP4, fm.WFMT_INT4])
@pytest.mark.parametrize("T", [2, 8, 16])
def test_few_full_size(T, fmt):
    _parity(_full(T, fmt))


def test_few_shares_a_workspace_with_other_paths():
    """Small-batch launches between single-token launches and the four-launch path on one
    workspace: every call correct, the launch counters count the persistent launches (one
    per call here: the four-launch path at T = 32 routes in one)."""
    ws = None
    n = 0
    for T in (8, 1, 16, 32, 3, 1, 8):
        c = Case(T, 256, 128, 256, 6, layer=T)
        c.upload()
        ws = c.workspace(32) if ws is None else ws
        g = _layer(c, ws)
        n += 1
        assert _launches(ws) == n
        assert fm.workspace_status(ws) == 0
        w64 = check_routing(c, g, {})
        check_forward(c, g, w64)
        _say("  T=%d ok" % T)


def test_few_repeated_calls_bitwise():
    """The same batch twice on one workspace: identical bits (a fixed summation order; the
    second call's words carry a new tag)."""
    c = Case(8, 256, 128, 256, 6).upload()
    ws = c.workspace()
    a = _layer(c, ws)
    b = _layer(c, ws)
    assert _launches(ws) == 2
    for key in ("y", "topk_ids", "topk_w", "logits", "sorted_assign", "assign_pos", "counts", "offsets"):
        assert np.array_equal(a[key], b[key]), key
