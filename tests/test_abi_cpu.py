"""The C-ABI library loads, exports every symbol include/flint_moe.h declares, and
rejects invalid arguments with the documented status codes before touching the device
(no GPU is needed: every call here fails validation, so no kernel is launched)."""
import ctypes
import os
import re

import pytest

import sparse_moe_transformer_wave_amd as fm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flint_moe.h")


def declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(flint_moe_\w+)\s*\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    names = declared()
    assert set(names) == set(fm.EXPORTED)
    L = ctypes.CDLL(fm.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for s in range(7):
        assert isinstance(fm.status_string(s), str) and fm.status_string(s)
    assert fm.status_string(99) == "unknown status"


A = 1 << 20          # a fake, 16-byte aligned address (never dereferenced)
MIS = A + 8          # misaligned


def _route(d, T, x=A, wr=A, bias=None, logits=None, ids=A, w=A, flags=0, ws=None, nb=0):
    L = fm.lib()
    return L.flint_moe_route(None if d is None else ctypes.byref(d), T, x, wr, bias, logits,
                             ids, w, flags, ws, nb, None)


def test_route_validation():
    d = fm.desc(2048, 768)
    assert _route(None, 1) == fm.ERR_NULL
    assert _route(fm.desc(2048, 768, n_experts=0), 1) == fm.ERR_SHAPE
    assert _route(fm.desc(2048, 768, n_experts=300), 1) == fm.ERR_SHAPE
    assert _route(fm.desc(2048, 768, top_k=9), 1) == fm.ERR_SHAPE
    assert _route(fm.desc(2048, 768, n_experts=4, top_k=5), 1) == fm.ERR_SHAPE
    assert _route(fm.desc(2000, 768), 1) == fm.ERR_SHAPE
    assert _route(fm.desc(2048, 700), 1) == fm.ERR_SHAPE
    assert _route(fm.desc(2048, 768, n_shared=2), 1) == fm.ERR_SHAPE
    assert _route(d, -1) == fm.ERR_SHAPE
    assert _route(d, 70000) == fm.ERR_SHAPE
    assert _route(d, 0) == fm.OK
    assert _route(d, 1, x=None) == fm.ERR_NULL
    assert _route(d, 1, ids=None) == fm.ERR_NULL
    assert _route(d, 1, x=MIS) == fm.ERR_ALIGN
    assert _route(d, 1, flags=4) == fm.ERR_FORMAT
    assert _route(d, 1, flags=fm.ROUTE_LOGITS_IN) == fm.ERR_NULL   # logits missing
    assert _route(d, 1) == fm.ERR_NULL                              # no logits, no workspace
    assert _route(d, 1, ws=A, nb=16) == fm.ERR_WORKSPACE


def _weights(fmt=fm.WFMT_BF16, shared=True, scales=False, **kw):
    w = fm.Weights(fmt, A, A, A, *( (A, A, A) if shared else (None, None, None)))
    if scales:
        for n in ("gate_sf", "up_sf", "down_sf", "gate_ts", "up_ts", "down_ts"):
            setattr(w, n, A)
        if shared:
            for n in ("sh_gate_sf", "sh_up_sf", "sh_down_sf", "sh_ts"):
                setattr(w, n, A)
    for k, v in kw.items():
        setattr(w, k, v)
    return w.c_struct()


def _forward(d, w, T, ws=A, nb=0, **kw):
    args = dict(x=A, ids=A, tw=A, off=A, sa=A, ap=A, y=A)
    args.update(kw)
    return fm.lib().flint_moe_forward(ctypes.byref(d), ctypes.byref(w), T, args["x"], args["ids"],
                                      args["tw"], args["off"], args["sa"], args["ap"], args["y"],
                                      ws, nb, None)


def test_forward_and_layer_validation():
    d = fm.desc(2048, 768)
    need = fm.workspace_bytes(d, 8)
    assert need > 0 and fm.workspace_bytes(d, 16) > need
    assert fm.workspace_bytes(d, -1) == 0 and fm.workspace_bytes(fm.desc(100, 768), 1) == 0
    assert fm.workspace_bytes(d, 8, 7) == 0
    assert _forward(d, _weights(), 0) == fm.OK
    assert _forward(d, _weights(), 8, nb=need - 1) == fm.ERR_WORKSPACE
    assert _forward(d, _weights(), 8, nb=need, y=None) == fm.ERR_NULL
    assert _forward(d, _weights(), 8, nb=need, sa=MIS) == fm.ERR_ALIGN
    assert _forward(d, _weights(fmt=3), 8, nb=need) == fm.ERR_FORMAT
    assert _forward(d, _weights(shared=False), 8, nb=need) == fm.ERR_NULL
    assert _forward(fm.desc(2048, 768, n_shared=0), _weights(), 8, nb=need) == fm.ERR_FORMAT
    assert _forward(d, _weights(scales=True), 8, nb=need) == fm.ERR_FORMAT   # bf16 with scales
    assert _forward(d, _weights(fmt=fm.WFMT_NVFP4), 8, nb=need) == fm.ERR_FORMAT  # nvfp4 without
    assert _forward(d, _weights(fmt=fm.WFMT_NVFP4, scales=True, gate_ts=MIS), 8, nb=need) == fm.ERR_ALIGN
    assert _forward(d, _weights(gate=MIS), 8, nb=need) == fm.ERR_ALIGN
    L = fm.lib()
    w = _weights()
    assert L.flint_moe_layer(ctypes.byref(d), ctypes.byref(w), 0, A, A, None, A, None, A, 0, None) == fm.OK
    assert L.flint_moe_layer(ctypes.byref(d), ctypes.byref(w), 4, A, None, None, A, None, A, need, None) == fm.ERR_NULL
    assert L.flint_moe_layer(ctypes.byref(d), ctypes.byref(w), 4, A, A, None, A, None, A, 16, None) == fm.ERR_WORKSPACE
    assert L.flint_moe_permute(ctypes.byref(d), 4, A, A, None, A, A, None, 0, None) == fm.ERR_NULL
    assert L.flint_moe_permute(ctypes.byref(d), 0, None, None, None, None, None, None, 0, None) == fm.OK


def test_dense_layer_validation():
    """n_experts = 0, top_k = 0, n_shared = 1 is a dense SwiGLU layer: the shared expert
    alone, no router.  Route and permute reject it; forward and layer take it with the
    routed weight pointers NULL and no router weights."""
    L = fm.lib()
    dd = fm.desc(2048, 4096, n_experts=0, top_k=0, n_shared=1)
    need = fm.workspace_bytes(dd, 8)
    assert need > 0 and fm.workspace_bytes(dd, 32) > need
    assert fm.workspace_bytes(fm.desc(2048, 4096, n_experts=0, top_k=1), 1) == 0
    assert fm.workspace_bytes(fm.desc(2048, 4096, n_experts=0, top_k=0, n_shared=0), 1) == 0
    assert _route(dd, 1, ws=A, nb=need) == fm.ERR_SHAPE
    assert L.flint_moe_permute(ctypes.byref(dd), 4, A, A, A, A, A, None, 0, None) == fm.ERR_SHAPE
    dense_w = fm.Weights(fm.WFMT_BF16, None, None, None, A, A, A).c_struct()
    routed_w = _weights()
    # routing arguments may be NULL; routed weights must be absent
    assert _forward(dd, dense_w, 8, nb=need - 1, ids=None, tw=None, off=None, sa=None,
                    ap=None) == fm.ERR_WORKSPACE
    assert _forward(dd, routed_w, 8, nb=need) == fm.ERR_FORMAT
    assert _forward(dd, dense_w, 8, nb=need, y=None) == fm.ERR_NULL
    assert _forward(dd, fm.Weights(fm.WFMT_BF16, None, None, None).c_struct(), 8, nb=need) == fm.ERR_NULL
    nv = fm.Weights(fm.WFMT_NVFP4, None, None, None, A, A, A, sh_gate_sf=A, sh_up_sf=A,
                    sh_down_sf=A, sh_ts=A, gate_ts=A).c_struct()
    assert _forward(dd, nv, 8, nb=need) == fm.ERR_FORMAT
    assert L.flint_moe_layer(ctypes.byref(dd), ctypes.byref(dense_w), 8, A, None, None, A, None,
                             A, 16, None) == fm.ERR_WORKSPACE
    assert L.flint_moe_layer(ctypes.byref(dd), ctypes.byref(dense_w), 8, A, None, None, None,
                             None, A, need, None) == fm.ERR_NULL


def test_decode_chain_validation():
    """flint_moe_decode_chain checks every layer's weights before any HIP call."""
    L = fm.lib()
    d = fm.desc(2048, 768)
    need = fm.workspace_bytes(d, 1)

    def chain(layers, n=None, flags=0, T=1, x=A, y=A, ids=None, tw=None, ws=A, nb=need, dd=d):
        refs = fm.layer_refs(layers)
        return L.flint_moe_decode_chain(ctypes.byref(dd), refs if layers else None,
                                        len(layers) if n is None else n, flags, T, x, y, ids, tw,
                                        None, ws, nb, None)

    good = (fm.Weights(fm.WFMT_BF16, A, A, A, A, A, A), A, None)
    assert chain([], n=0) == fm.OK
    assert chain([good], n=-1) == fm.ERR_SHAPE
    assert chain([good], n=5000) == fm.ERR_SHAPE
    assert chain([good], T=0) == fm.ERR_SHAPE and chain([good], T=17) == fm.ERR_SHAPE
    assert chain([good], dd=fm.desc(2048, 768, n_experts=0, top_k=0)) == fm.ERR_SHAPE
    assert chain([good], flags=2) == fm.ERR_FORMAT
    assert chain([], n=1) == fm.ERR_NULL
    assert chain([good], x=None) == fm.ERR_NULL
    assert chain([good], y=MIS) == fm.ERR_ALIGN
    assert chain([good, (fm.Weights(fm.WFMT_BF16, A, A, None, A, A, A), A, None)]) == fm.ERR_NULL
    assert chain([good, (good[0], None, None)]) == fm.ERR_NULL
    assert chain([good, (good[0], A, MIS)]) == fm.ERR_ALIGN
    nv = fm.Weights(fm.WFMT_NVFP4, A, A, A, A, A, A, A, A, A, A, A, A, A, A, A, A)
    assert chain([good, (nv, A, None)]) == fm.ERR_FORMAT  # formats differ
    assert chain([good], nb=need - 1) == fm.ERR_WORKSPACE


def test_int4_weight_validation():
    """INT4: group scales required (shared ones iff n_shared), tensor scales forbidden."""
    d = fm.desc(2048, 768)
    need = fm.workspace_bytes(d, 8, fm.WFMT_INT4)
    assert need > 0
    ok = fm.Weights(fm.WFMT_INT4, A, A, A, A, A, A, A, A, A, A, A, A)
    assert _forward(d, ok.c_struct(), 8, nb=need - 1) == fm.ERR_WORKSPACE
    bad_ts = fm.Weights(fm.WFMT_INT4, A, A, A, A, A, A, A, A, A, A, A, A, gate_ts=A)
    assert _forward(d, bad_ts.c_struct(), 8, nb=need) == fm.ERR_FORMAT
    bad_sh_ts = fm.Weights(fm.WFMT_INT4, A, A, A, A, A, A, A, A, A, A, A, A, sh_ts=A)
    assert _forward(d, bad_sh_ts.c_struct(), 8, nb=need) == fm.ERR_FORMAT
    no_sf = fm.Weights(fm.WFMT_INT4, A, A, A, A, A, A, None, A, A, A, A, A)
    assert _forward(d, no_sf.c_struct(), 8, nb=need) == fm.ERR_FORMAT
    no_sh_sf = fm.Weights(fm.WFMT_INT4, A, A, A, A, A, A, A, A, A, None, A, A)
    assert _forward(d, no_sh_sf.c_struct(), 8, nb=need) == fm.ERR_FORMAT
    mis = fm.Weights(fm.WFMT_INT4, A, A, A, A, A, A, A, MIS, A, A, A, A)
    assert _forward(d, mis.c_struct(), 8, nb=need) == fm.ERR_ALIGN
    d0 = fm.desc(2048, 768, n_shared=0)
    sh_sf_without_shared = fm.Weights(fm.WFMT_INT4, A, A, A, None, None, None, A, A, A, A, None, None)
    assert _forward(d0, sh_sf_without_shared.c_struct(), 8, nb=need) == fm.ERR_FORMAT


def test_shape_contract_h64_i32():
    """hidden % 64 and inter % 32 (bf16, NVFP4); INT4 also needs hidden % 128 and inter % 128
    (its scale groups are 128 columns)."""
    for H, I in ((64, 32), (320, 96), (2048, 96), (192, 160), (8192, 4096)):
        d = fm.desc(H, I)
        assert fm.workspace_bytes(d, 8, fm.WFMT_BF16) > 0
        assert fm.workspace_bytes(d, 8, fm.WFMT_NVFP4) > 0
        assert (fm.workspace_bytes(d, 8, fm.WFMT_INT4) > 0) == (H % 128 == 0 and I % 128 == 0)
    for H, I in ((32, 32), (96, 32), (2048, 16), (2048, 48), (8256, 32), (2048, 4128)):
        assert fm.workspace_bytes(fm.desc(H, I), 8) == 0, (H, I)
    d = fm.desc(2048, 96)
    need = fm.workspace_bytes(d, 8, fm.WFMT_NVFP4)
    int4 = fm.Weights(fm.WFMT_INT4, A, A, A, A, A, A, A, A, A, A, A, A)
    assert _forward(d, int4.c_struct(), 8, nb=need) == fm.ERR_SHAPE
    assert _forward(fm.desc(384, 128), int4.c_struct(), 8, nb=fm.workspace_bytes(fm.desc(384, 128), 8, 2) - 1) \
        == fm.ERR_WORKSPACE


def test_workspace_status_validation():
    L = fm.lib()
    assert L.flint_moe_workspace_status(None, 1 << 20, A, None) == fm.ERR_NULL
    assert L.flint_moe_workspace_status(A, 1 << 20, None, None) == fm.ERR_NULL
    assert L.flint_moe_workspace_status(MIS, 1 << 20, A, None) == fm.ERR_ALIGN
    assert L.flint_moe_workspace_status(A, 1 << 20, A + 2, None) == fm.ERR_ALIGN
    assert L.flint_moe_workspace_status(A, 1024, A, None) == fm.ERR_WORKSPACE


def test_layer_noalloc_validation():
    """flint_moe_layer_noalloc validates like flint_moe_layer, and rejects a T whose
    workspace would exceed its 16 MiB array, before any HIP call."""
    L = fm.lib()
    d = fm.desc(2048, 768)
    w = _weights()
    call = lambda T, dd=d, ww=w, x=A, wr=A, y=A: L.flint_moe_layer_noalloc(
        None if dd is None else ctypes.byref(dd), ctypes.byref(ww), T, x, wr, None, y, None, None)
    assert call(0) == fm.OK
    assert call(1, dd=None) == fm.ERR_NULL
    assert call(-1) == fm.ERR_SHAPE
    assert call(4, wr=None) == fm.ERR_NULL
    assert call(4, y=MIS) == fm.ERR_ALIGN
    assert fm.workspace_bytes(d, 150) <= 16 << 20 < fm.workspace_bytes(d, 256)
    assert call(256) == fm.ERR_WORKSPACE
    assert call(65536) == fm.ERR_WORKSPACE
