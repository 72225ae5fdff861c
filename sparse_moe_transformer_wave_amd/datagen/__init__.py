"""Seeded synthetic inputs for the MoE layer.

This module draws numbers and nothing else: it holds none of the layer's arithmetic.
Both the GPU library and the reference read the bytes it produces.  The generator's
definition is in gen_host.c; gen_device.hip draws the same streams on the GPU for the
large benchmark pools (host and device may differ in the last bit of a transcendental,
so tests take their inputs from the host side).

Workload recipe (what the benchmark and tests draw):
  x      bf16  N(0, 1)      [T][H]           stream (layer, KIND_X, 0)
  Wr     fp32  N(0, 0.02)   [E][H]           stream (layer, KIND_ROUTER, 0)
  gate   bf16  N(0, 0.02)   [I][H] / expert  stream (layer, KIND_GATE, e)   e = E is shared
  up     bf16  N(0, 0.02)   [I][H] / expert  stream (layer, KIND_UP, e)
  down   bf16  N(0, 0.02)   [H][I] / expert  stream (layer, KIND_DOWN, e)
  Zipf logit bias  bias_e = -c * s * ln(rank_e), s = 1.1, rank from a seeded permutation
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libflint_gen_host.so")
_SRC = os.path.join(_HERE, "gen_host.c")

KIND_X = 1
KIND_ROUTER = 2
KIND_GATE = 3
KIND_UP = 4
KIND_DOWN = 5
KIND_ZIPF = 6

X_STD = 1.0
W_STD = 0.02
ROUTER_STD = 0.02
ZIPF_S = 1.1
# Zipf strength c for the 8192-token prefill workload at H=2048, E=256, k=6, seed 0:
# the value at which the 16 hottest experts receive 50 % of the assignments.  Written by
# tests/golden/calibrate_zipf.py (tests/golden/zipf_c.txt holds the value and the share).
ZIPF_C = 0.4284


def stream_id(layer: int, kind: int, index: int = 0) -> int:
    return (int(layer) << 40) | (int(kind) << 32) | int(index)


def build(force: bool = False) -> str:
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def _L():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_SO)
        vp, i64, u64, d = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double
        for name in ("gen_normal_bf16", "gen_normal_f32", "gen_normal_f64"):
            getattr(L, name).argtypes = [vp, i64, u64, u64, d]
            getattr(L, name).restype = None
        L.gen_uint64.argtypes = [vp, i64, u64, u64]
        L.gen_uint64.restype = None
        L.gen_rank_permutation.argtypes = [vp, ctypes.c_int32, u64, u64]
        L.gen_rank_permutation.restype = None
        L.gen_key.argtypes = [u64, u64]
        L.gen_key.restype = u64
        _lib = L
    return _lib


def _fill(name, dtype, shape, seed, stream, std):
    a = np.empty(shape, dtype)
    getattr(_L(), name)(a.ctypes.data, a.size, seed, stream, float(std))
    return a


def normal_bf16(shape, seed: int, stream: int, std: float) -> np.ndarray:
    """uint16 bf16 bits of round-to-nearest-even(std * N(0,1))."""
    return _fill("gen_normal_bf16", np.uint16, shape, seed, stream, std)


def normal_f32(shape, seed: int, stream: int, std: float) -> np.ndarray:
    return _fill("gen_normal_f32", np.float32, shape, seed, stream, std)


def normal_f64(shape, seed: int, stream: int, std: float) -> np.ndarray:
    return _fill("gen_normal_f64", np.float64, shape, seed, stream, std)


def raw_u64(n: int, seed: int, stream: int) -> np.ndarray:
    a = np.empty(n, np.uint64)
    _L().gen_uint64(a.ctypes.data, n, seed, stream)
    return a


def rank_permutation(n: int, seed: int, stream: int) -> np.ndarray:
    r = np.empty(n, np.int32)
    _L().gen_rank_permutation(r.ctypes.data, n, seed, stream)
    return r


def zipf_bias(E: int, c: float, seed: int = 0, layer: int = 0, s: float = ZIPF_S) -> np.ndarray:
    """Per-expert logit bias -c * s * ln(rank): rank 1 is the hottest expert."""
    rank = rank_permutation(E, seed, stream_id(layer, KIND_ZIPF, 0)).astype(np.float64)
    return (-c * s * np.log(rank)).astype(np.float32)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bf16 bits (finite inputs)."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


class LayerInputs:
    """Host-side bf16 layer of the recipe above (routed experts 0..E-1, shared = E)."""

    def __init__(self, T, H, I, E, k, seed=0, layer=0, n_shared=1, bias_c=None,
                 experts=None):
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, k
        self.seed, self.layer, self.n_shared = seed, layer, n_shared
        self.x = normal_bf16((T, H), seed, stream_id(layer, KIND_X, 0), X_STD)
        self.Wr = normal_f32((E, H), seed, stream_id(layer, KIND_ROUTER, 0), ROUTER_STD)
        self.bias = None if bias_c is None else zipf_bias(E, bias_c, seed, layer)
        ex = range(E) if experts is None else experts
        self.gate = np.zeros((E, I, H), np.uint16)
        self.up = np.zeros((E, I, H), np.uint16)
        self.down = np.zeros((E, H, I), np.uint16)
        for e in ex:
            self.gate[e], self.up[e], self.down[e] = self.expert_bf16(e)
        if n_shared:
            g, u, d = self.expert_bf16(E)
            self.sh_gate, self.sh_up, self.sh_down = g[None], u[None], d[None]
        else:
            self.sh_gate = self.sh_up = self.sh_down = None

    def expert_bf16(self, e):
        H, I, s, L = self.H, self.I, self.seed, self.layer
        return (normal_bf16((I, H), s, stream_id(L, KIND_GATE, e), W_STD),
                normal_bf16((I, H), s, stream_id(L, KIND_UP, e), W_STD),
                normal_bf16((H, I), s, stream_id(L, KIND_DOWN, e), W_STD))

    def expert_f64(self, e):
        H, I, s, L = self.H, self.I, self.seed, self.layer
        return (normal_f64((I, H), s, stream_id(L, KIND_GATE, e), W_STD),
                normal_f64((I, H), s, stream_id(L, KIND_UP, e), W_STD),
                normal_f64((H, I), s, stream_id(L, KIND_DOWN, e), W_STD))


# ----------------------------------------------------------------------------- device side
_dev = None
_DEV_SO = os.path.join(_HERE, "libflint_gen_device.so")


def _D():
    global _dev
    if _dev is None:
        if not os.path.exists(_DEV_SO):
            raise RuntimeError("libflint_gen_device.so is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(_DEV_SO)
        vp, i64, u64, d = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_double
        L.flint_gen_normal_bf16.argtypes = [vp, i64, i64, u64, u64, d, vp]
        L.flint_gen_normal_f32.argtypes = [vp, i64, u64, u64, d, vp]
        L.flint_gen_nvfp4.argtypes = [vp, vp, vp, vp, i64, i64, i64, u64, u64, d, vp]
        L.flint_gen_int4.argtypes = [vp, vp, i64, i64, i64, u64, u64, d, vp]
        for f in ("flint_gen_normal_bf16", "flint_gen_normal_f32", "flint_gen_nvfp4", "flint_gen_int4"):
            getattr(L, f).restype = ctypes.c_int
        _dev = L
    return _dev


def _cur_stream():
    import torch
    return torch.cuda.current_stream().cuda_stream


def device_normal_bf16(t, n_mat: int, per_mat: int, seed: int, stream0: int, std: float):
    """Fill device tensor t (>= n_mat * per_mat bf16) with matrices of streams stream0 + m."""
    assert t.numel() * t.element_size() >= n_mat * per_mat * 2
    rc = _D().flint_gen_normal_bf16(t.data_ptr(), n_mat, per_mat, seed, stream0, std, _cur_stream())
    if rc:
        raise RuntimeError("flint_gen_normal_bf16 failed: %d" % rc)


def device_normal_f32(t, seed: int, stream: int, std: float):
    rc = _D().flint_gen_normal_f32(t.data_ptr(), t.numel(), seed, stream, std, _cur_stream())
    if rc:
        raise RuntimeError("flint_gen_normal_f32 failed: %d" % rc)


def device_int4(q, sc, n_mat: int, N: int, K: int, seed: int, stream0: int, std: float):
    """INT4 pool on the device: codes q uint8 [n_mat][N][K/2], bf16 group scales sc
    (int16 tensor) [n_mat][N][K/128]."""
    rc = _D().flint_gen_int4(q.data_ptr(), sc.data_ptr(), n_mat, N, K, seed, stream0, std, _cur_stream())
    if rc:
        raise RuntimeError("flint_gen_int4 failed: %d" % rc)


def device_nvfp4(q, sf, ts, scratch, n_mat: int, N: int, K: int, seed: int, stream0: int,
                 std: float):
    rc = _D().flint_gen_nvfp4(q.data_ptr(), sf.data_ptr(), ts.data_ptr(), scratch.data_ptr(),
                              n_mat, N, K, seed, stream0, std, _cur_stream())
    if rc:
        raise RuntimeError("flint_gen_nvfp4 failed: %d" % rc)
