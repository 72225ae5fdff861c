"""Shared helpers for the GPU parity tests: build seeded layer inputs on the host, run
the HIP library through the C ABI, run the reference on the same bytes and compare.

Parity protocol (two stages):
  R  routing:  fp32 logits within the a-priori bound of an fp32 dot product
               (|dl| <= 2 (H + 2) 2^-24 sum_h |x_h Wr_eh| + 2^-23 |bias_e|); ids equal to the
               reference selection run on the GPU's own fp32 logits (bit-exact, same order);
               weights within 1e-6 of sigmoid/sum recomputed in fp64 from those logits; tokens
               whose fp64 k-th/k+1-th gap exceeds twice the bound also match the reference's
               own fp64 selection.  Permutation arrays: exactly equal.
  F  forward:  y against the reference evaluated with the GPU's ids and the fp64 weights:
               max|dy| <= 2e-2 max|y_ref| and sum|dy| / sum|y_ref| <= 5e-3.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import sparse_moe_transformer_wave_amd as fm
from sparse_moe_transformer_wave_amd import datagen as dg

MAX_REL = 2e-2
MEAN_REL = 5e-3
U = 2.0 ** -24


class Case:
    """Seeded layer: host arrays, reference descriptors and device tensors."""

    def __init__(self, T, H, I, E, k, S=1, seed=0, layer=0, fmt=fm.WFMT_BF16, bias_c=None,
                 renorm=1, experts=None, x=None, logits_in=None, wscale=None):
        self.T, self.H, self.I, self.E, self.k, self.S = T, H, I, E, k, S
        self.fmt, self.renorm = fmt, renorm
        self.desc = fm.desc(H, I, E, k, S, renorm)
        self.x = dg.normal_bf16((T, H), seed, dg.stream_id(layer, dg.KIND_X, 0), dg.X_STD) if x is None else x
        self.Wr = dg.normal_f32((E, H), seed, dg.stream_id(layer, dg.KIND_ROUTER, 0), dg.ROUTER_STD)
        self.bias = None if bias_c is None else dg.zipf_bias(E, bias_c, seed, layer)
        ex = list(range(E)) if experts is None else list(experts)
        self.seed, self.layer = seed, layer
        if fmt == fm.WFMT_BF16:
            g = np.zeros((E, I, H), np.uint16)
            u = np.zeros((E, I, H), np.uint16)
            d = np.zeros((E, H, I), np.uint16)
            for e in ex:
                g[e], u[e], d[e] = self._bf16(e)
            if wscale is not None:
                d = dg.f32_to_bf16_bits(dg.bf16_bits_to_f32(d) * wscale)
            self.host = {"gate": g, "up": u, "down": d}
            if S:
                sg, su, sd = self._bf16(E)
                if wscale is not None:
                    sd = dg.f32_to_bf16_bits(dg.bf16_bits_to_f32(sd) * wscale)
                self.host_sh = {"gate": sg[None], "up": su[None], "down": sd[None]}
        elif fmt == fm.WFMT_NVFP4:
            self.host = self._nvfp4_set(ex, E)
            if S:
                self.host_sh = self._nvfp4_set([E], 1, offset=E)
        else:
            self.host = self._int4_set(ex, E)
            if S:
                self.host_sh = self._int4_set([E], 1, offset=E)
        ofmt = {fm.WFMT_BF16: oracle.FMT_BF16, fm.WFMT_NVFP4: oracle.FMT_NVFP4, fm.WFMT_INT4: oracle.FMT_INT4}[fmt]
        self.routed = oracle.Experts(ofmt, H, I, self.host)
        self.shared = oracle.Experts(ofmt, H, I, self.host_sh) if S else None
        self.logits_in = logits_in

    def _bf16(self, e):
        H, I, s, L = self.H, self.I, self.seed, self.layer
        return (dg.normal_bf16((I, H), s, dg.stream_id(L, dg.KIND_GATE, e), dg.W_STD),
                dg.normal_bf16((I, H), s, dg.stream_id(L, dg.KIND_UP, e), dg.W_STD),
                dg.normal_bf16((H, I), s, dg.stream_id(L, dg.KIND_DOWN, e), dg.W_STD))

    def _nvfp4_set(self, ex, n, offset=0):
        H, I, s, L = self.H, self.I, self.seed, self.layer
        out = {}
        for name, kind, (N, K) in (("gate", dg.KIND_GATE, (I, H)), ("up", dg.KIND_UP, (I, H)),
                                   ("down", dg.KIND_DOWN, (H, I))):
            q = np.zeros((n, N, K // 2), np.uint8)
            sb = np.zeros((n, N, K // 16), np.uint8)
            st = np.ones(n, np.float32)
            for e in ex:
                W = dg.normal_f64((N, K), s, dg.stream_id(L, kind, e), dg.W_STD)
                q[e - offset], sb[e - offset], st[e - offset] = oracle.nvfp4_quantize(W)
            out["q_" + name], out["sb_" + name], out["st_" + name] = q, sb, st
        return out

    def _int4_set(self, ex, n, offset=0):
        H, I, s, L = self.H, self.I, self.seed, self.layer
        out = {}
        for name, kind, (N, K) in (("gate", dg.KIND_GATE, (I, H)), ("up", dg.KIND_UP, (I, H)),
                                   ("down", dg.KIND_DOWN, (H, I))):
            q = np.zeros((n, N, K // 2), np.uint8)
            sb = np.zeros((n, N, K // 128), np.uint16)
            for e in ex:
                W = dg.normal_f64((N, K), s, dg.stream_id(L, kind, e), dg.W_STD)
                q[e - offset], sb[e - offset] = oracle.int4_quantize(W)
            out["q_" + name], out["sb_" + name] = q, sb
        return out

    # ------------------------------------------------------------------ device side
    def upload(self):
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.d_x = dev(self.x.view(np.int16))
        self.d_Wr = dev(self.Wr)
        self.d_bias = None if self.bias is None else dev(self.bias)
        if self.fmt == fm.WFMT_BF16:
            h = {k: dev(v.view(np.int16)) for k, v in self.host.items()}
            hs = {k: dev(v.view(np.int16)) for k, v in self.host_sh.items()} if self.S else {}
            self.weights = fm.Weights(fm.WFMT_BF16, h["gate"], h["up"], h["down"],
                                      hs.get("gate"), hs.get("up"), hs.get("down"))
            self._keep = (h, hs)
        elif self.fmt == fm.WFMT_INT4:
            h = {k: dev(v.view(np.int16) if v.dtype == np.uint16 else v) for k, v in self.host.items()}
            hs = {k: dev(v.view(np.int16) if v.dtype == np.uint16 else v) for k, v in self.host_sh.items()} if self.S else {}
            self.weights = fm.Weights(
                fm.WFMT_INT4, h["q_gate"], h["q_up"], h["q_down"],
                hs.get("q_gate"), hs.get("q_up"), hs.get("q_down"),
                h["sb_gate"], h["sb_up"], h["sb_down"],
                hs.get("sb_gate"), hs.get("sb_up"), hs.get("sb_down"))
            self._keep = (h, hs)
        else:
            h = {k: dev(v) for k, v in self.host.items()}
            hs = {k: dev(v) for k, v in self.host_sh.items()} if self.S else {}
            sh_ts = dev(np.array([self.host_sh["st_gate"][0], self.host_sh["st_up"][0],
                                  self.host_sh["st_down"][0]], np.float32)) if self.S else None
            self.weights = fm.Weights(
                fm.WFMT_NVFP4, h["q_gate"], h["q_up"], h["q_down"],
                hs.get("q_gate"), hs.get("q_up"), hs.get("q_down"),
                h["sb_gate"], h["sb_up"], h["sb_down"],
                hs.get("sb_gate"), hs.get("sb_up"), hs.get("sb_down"),
                h["st_gate"], h["st_up"], h["st_down"], sh_ts)
            self._keep = (h, hs, sh_ts)
        return self

    def alloc_out(self):
        T, E, k, H = self.T, self.E, self.k, self.H
        z = lambda *s, dt=torch.int32: torch.zeros(s, dtype=dt, device="cuda")
        return {"logits": z(max(T, 1), E, dt=torch.float32), "topk_ids": z(max(T, 1), k),
                "topk_w": z(max(T, 1), k, dt=torch.float32), "counts": z(E),
                "offsets": z(E + 4), "sorted_assign": z(max(T * k, 1)),
                "assign_pos": z(max(T * k, 1)), "y": z(max(T, 1), H, dt=torch.int16)}

    def workspace(self, T=None):
        return fm.workspace(self.desc, self.T if T is None else T, self.fmt)

    def run_layer(self):
        out = self.alloc_out()
        ws = self.workspace()
        routing = {k: out[k] for k in ("logits", "topk_ids", "topk_w", "counts", "offsets",
                                       "sorted_assign", "assign_pos")}
        fm.layer(self.desc, self.weights, self.T, self.d_x, self.d_Wr, self.d_bias, out["y"], ws,
                 routing)
        torch.cuda.synchronize()
        return to_host(out, self)

    def run_steps(self):
        """route -> permute -> forward as three separate C-ABI calls."""
        out = self.alloc_out()
        ws = self.workspace()
        T = self.T
        fm.route(self.desc, T, self.d_x, self.d_Wr, self.d_bias, out["topk_ids"], out["topk_w"],
                 ws, logits=out["logits"])
        fm.permute(self.desc, T, out["topk_ids"], out["counts"], out["offsets"],
                   out["sorted_assign"], out["assign_pos"], ws)
        fm.forward(self.desc, self.weights, T, self.d_x, out["topk_ids"], out["topk_w"],
                   out["offsets"], out["sorted_assign"], out["assign_pos"], out["y"], ws)
        torch.cuda.synchronize()
        return to_host(out, self)


def to_host(out, c):
    T, E, k = c.T, c.E, c.k
    h = {kk: v.cpu().numpy() for kk, v in out.items()}
    h["logits"] = h["logits"][:T]
    h["topk_ids"] = h["topk_ids"][:T]
    h["topk_w"] = h["topk_w"][:T]
    h["offsets"] = h["offsets"][:E + 1]
    h["sorted_assign"] = h["sorted_assign"][:T * k]
    h["assign_pos"] = h["assign_pos"][:T * k]
    h["y"] = h["y"][:T].view(np.uint16)
    return h


def logit_bound(c: Case):
    """A-priori bound of an fp32 sum of n exact products plus the bias: 2 (n + 2) u sum|x w|.
    The streaming path (T <= 32) sums n = H products; the batched path splits each fp32
    weight into three exact bf16 parts and sums n = 3H exact products."""
    xa = np.abs(dg.bf16_bits_to_f32(c.x).astype(np.float64))
    sa = xa @ np.abs(c.Wr.astype(np.float64)).T
    b = 0.0 if c.bias is None else np.abs(c.bias.astype(np.float64))[None, :]
    n = c.H if c.T <= 32 else 3 * c.H
    return 2.0 * (n + 2) * U * sa + 2.0 * U * b


def check_routing(c: Case, g, report=None):
    """Stage R; returns the fp64 weights recomputed from the GPU logits."""
    T, k = c.T, c.k
    ref_l = oracle.router(c.x, c.Wr, c.bias)
    beta = logit_bound(c)
    gl = g["logits"].astype(np.float64)
    fin = np.isfinite(ref_l)  # an infinite bias gives that infinite logit exactly
    np.testing.assert_array_equal(gl[~fin], ref_l[~fin])
    dl = np.abs(gl[fin] - ref_l[fin])
    assert np.all(dl <= beta[fin]), "logits outside the fp32 bound: max excess %g" % (dl - beta[fin]).max()
    ids_ref_on_gpu = oracle.select(gl, k)
    np.testing.assert_array_equal(g["topk_ids"], ids_ref_on_gpu)
    w64 = oracle.weights(gl, g["topk_ids"], bool(c.renorm))
    assert np.abs(g["topk_w"] - w64).max() <= 1e-6
    if c.renorm:
        assert np.abs(g["topk_w"].astype(np.float64).sum(1) - 1).max() <= 1e-6
    own = oracle.select(ref_l, k)
    srt = -np.sort(-ref_l, axis=1)
    if k < c.E:
        with np.errstate(invalid="ignore"):
            gap = srt[:, k - 1] - srt[:, k]
            clear = gap > 2 * np.where(fin, beta, 0).max(axis=1)
        # a clear k-th / k+1-th gap fixes the selected set (the order inside it may follow
        # near-equal logits either way)
        np.testing.assert_array_equal(np.sort(g["topk_ids"][clear], 1), np.sort(own[clear], 1))
        if report is not None:
            report["near_ties"] = int((~clear).sum())
    if "counts" not in g:  # a call that returns no grouping tensors
        return w64
    counts, offsets, sa, ap = oracle.permute(g["topk_ids"], c.E)
    np.testing.assert_array_equal(g["counts"], counts)
    np.testing.assert_array_equal(g["offsets"], offsets)
    np.testing.assert_array_equal(g["sorted_assign"], sa)
    np.testing.assert_array_equal(g["assign_pos"], ap)
    return w64


def check_forward(c: Case, g, w64, tokens=None):
    ids = g["topk_ids"]
    y_ref = oracle.moe_tokens(c.routed, c.shared, c.x, ids, w64, tokens)
    y = dg.bf16_bits_to_f32(g["y"] if tokens is None else g["y"][tokens]).astype(np.float64)
    d = np.abs(y - y_ref)
    assert np.all(np.isfinite(y))
    mx = np.abs(y_ref).max()
    rel_max = d.max() / mx
    rel_l1 = d.sum() / np.abs(y_ref).sum()
    assert rel_max <= MAX_REL, "max|dy| / max|y| = %g" % rel_max
    assert rel_l1 <= MEAN_REL, "sum|dy| / sum|y| = %g" % rel_l1
    return rel_max, rel_l1
