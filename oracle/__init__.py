"""Python access to the reference MoE layer in oracle.c.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the CPU-baseline
leg of bench.py may import this module.  The GPU product path never does.

The C library is plain single-threaded fp64 code (see oracle.h for the definitions and
their sources on the pages).  This module only marshals numpy arrays into it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

FMT_BF16 = 0
FMT_NVFP4 = 1
FMT_INT4 = 2


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (single-threaded, -O2, no fast-math)."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall",
                               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _SO)
    return _SO


class _Matrix(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("data", ctypes.c_void_p),
                ("block_scale", ctypes.c_void_p), ("tensor_scale", ctypes.c_float)]


class _Expert(ctypes.Structure):
    _fields_ = [("gate", _Matrix), ("up", _Matrix), ("down", _Matrix)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_SO)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e2m1_value.argtypes = [ctypes.c_uint32]
        L.oracle_e4m3_value.restype = ctypes.c_double
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint32]
        L.oracle_e4m3_encode.restype = ctypes.c_uint32
        L.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        L.oracle_e2m1_encode.restype = ctypes.c_uint32
        L.oracle_e2m1_encode.argtypes = [ctypes.c_double]
        L.oracle_router.argtypes = [i64, i32, i32, vp, vp, vp, vp]
        L.oracle_router.restype = None
        L.oracle_select.argtypes = [i64, i32, i32, vp, vp]
        L.oracle_select.restype = ctypes.c_int
        L.oracle_weights.argtypes = [i64, i32, i32, i32, vp, vp, vp]
        L.oracle_weights.restype = None
        L.oracle_permute.argtypes = [i64, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_permute.restype = ctypes.c_int
        L.oracle_expert_ffn.argtypes = [i32, i32, ctypes.POINTER(_Expert), vp, vp, vp]
        L.oracle_expert_ffn.restype = None
        L.oracle_moe_tokens.argtypes = [i32, i32, i32, i32, ctypes.POINTER(_Expert),
                                        ctypes.POINTER(_Expert), vp, vp, vp, i64, vp, vp]
        L.oracle_moe_tokens.restype = None
        L.oracle_nvfp4_quantize.argtypes = [i64, i64, vp, vp, vp, ctypes.POINTER(ctypes.c_float)]
        L.oracle_nvfp4_quantize.restype = None
        L.oracle_int4_value.restype = ctypes.c_double
        L.oracle_int4_value.argtypes = [ctypes.c_uint32]
        L.oracle_int4_quantize.argtypes = [i64, i64, vp, vp, vp]
        L.oracle_int4_quantize.restype = None
        L.oracle_matrix_at.restype = ctypes.c_double
        L.oracle_matrix_at.argtypes = [ctypes.POINTER(_Matrix), i64, i64, i64]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


# ----------------------------------------------------------------------------- codecs
def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(code)


def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(code)


def e2m1_encode(v: float) -> int:
    return lib().oracle_e2m1_encode(float(v))


def e4m3_encode(v: float) -> int:
    return lib().oracle_e4m3_encode(float(v))


def nvfp4_quantize(W: np.ndarray):
    """W [N][K] (float64) -> (q uint8 [N][K/2], sb uint8 [N][K/16], st float)."""
    W = np.ascontiguousarray(W, dtype=np.float64)
    N, K = W.shape
    assert K % 16 == 0
    q = np.empty((N, K // 2), np.uint8)
    sb = np.empty((N, K // 16), np.uint8)
    st = ctypes.c_float(0.0)
    lib().oracle_nvfp4_quantize(N, K, _p(W), _p(q), _p(sb), ctypes.byref(st))
    return q, sb, float(st.value)


def int4_value(code: int) -> float:
    return lib().oracle_int4_value(code)


def int4_quantize(W: np.ndarray):
    """W [N][K] (float64) -> (q uint8 [N][K/2], s bf16 bits uint16 [N][K/128])."""
    W = np.ascontiguousarray(W, dtype=np.float64)
    N, K = W.shape
    assert K % 128 == 0
    q = np.empty((N, K // 2), np.uint8)
    sc = np.empty((N, K // 128), np.uint16)
    lib().oracle_int4_quantize(N, K, _p(W), _p(q), _p(sc))
    return q, sc


def matrix_at(fmt: int, data: np.ndarray, scale, K: int, n: int, k: int, tensor_scale=1.0) -> float:
    """Element (n, k) of one matrix as the reference reads it."""
    m = _Matrix(fmt, data.ctypes.data, None if scale is None else scale.ctypes.data,
                float(tensor_scale))
    return lib().oracle_matrix_at(ctypes.byref(m), K, n, k)


# ------------------------------------------------------------------------ layer steps
def router(x_bits: np.ndarray, Wr: np.ndarray, bias: np.ndarray | None = None) -> np.ndarray:
    """x bf16 bits uint16 [T][H], Wr float32 [E][H] -> logits float64 [T][E]."""
    x_bits = np.ascontiguousarray(x_bits, np.uint16)
    Wr = np.ascontiguousarray(Wr, np.float32)
    T, H = x_bits.shape
    E = Wr.shape[0]
    out = np.empty((T, E), np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    lib().oracle_router(T, H, E, _p(x_bits), _p(Wr), None if b is None else _p(b), _p(out))
    return out


def select(logits: np.ndarray, k: int) -> np.ndarray:
    logits = np.ascontiguousarray(logits, np.float64)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    rc = lib().oracle_select(T, E, k, _p(logits), _p(ids))
    if rc != 0:
        raise ValueError("oracle_select: NaN logit or k out of range")
    return ids


def weights(logits: np.ndarray, ids: np.ndarray, renormalize: bool = True) -> np.ndarray:
    logits = np.ascontiguousarray(logits, np.float64)
    ids = np.ascontiguousarray(ids, np.int32)
    T, E = logits.shape
    k = ids.shape[1]
    w = np.empty((T, k), np.float64)
    lib().oracle_weights(T, E, k, int(bool(renormalize)), _p(logits), _p(ids), _p(w))
    return w


def permute(ids: np.ndarray, E: int):
    """-> counts [E], offsets [E+1], sorted_assign [T*k], assign_pos [T*k] (int32)."""
    ids = np.ascontiguousarray(ids, np.int32)
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sa = np.empty(T * k, np.int32)
    ap = np.empty(T * k, np.int32)
    rc = lib().oracle_permute(T, E, k, _p(ids), _p(counts), _p(offsets), _p(sa), _p(ap))
    if rc != 0:
        raise ValueError("oracle_permute: expert id out of range")
    return counts, offsets, sa, ap


# ------------------------------------------------------------------------ weights
class Experts:
    """Holds the numpy arrays behind the ctypes expert descriptors (keeps them alive).

    bf16:  gate [n][I][H], up [n][I][H], down [n][H][I] as uint16 bits.
    nvfp4: dict of q/sb/st triples per matrix:  q_gate [n][I][H/2], sb_gate [n][I][H/16],
           st_gate [n] float32, and likewise for up and down ([n][H][I/2], [n][H][I/16]).
    int4:  q/sb pairs per matrix: q_gate [n][I][H/2] packed nibbles, sb_gate [n][I][H/128]
           bf16 scale bits (uint16), likewise for up and down.
    """

    def __init__(self, fmt: int, H: int, I: int, arrays: dict):
        self.fmt, self.H, self.I = fmt, H, I
        self.arrays = {k: np.ascontiguousarray(v) for k, v in arrays.items()}
        key = "gate" if fmt == FMT_BF16 else "q_gate"
        self.n = self.arrays[key].shape[0]
        self.desc = (_Expert * max(self.n, 1))()
        for e in range(self.n):
            self.desc[e] = self._expert(e)

    def _matrix(self, name: str, e: int, N: int, K: int) -> _Matrix:
        if self.fmt == FMT_BF16:
            a = self.arrays[name]
            assert a.dtype == np.uint16 and a.shape[1:] == (N, K)
            return _Matrix(FMT_BF16, a[e].ctypes.data, None, 0.0)
        if self.fmt == FMT_INT4:
            q, sb = self.arrays["q_" + name], self.arrays["sb_" + name]
            assert q.dtype == np.uint8 and q.shape[1:] == (N, K // 2) and sb.dtype == np.uint16
            assert sb.shape[1:] == (N, K // 128)
            return _Matrix(FMT_INT4, q[e].ctypes.data, sb[e].ctypes.data, 1.0)
        q, sb, st = self.arrays["q_" + name], self.arrays["sb_" + name], self.arrays["st_" + name]
        assert q.dtype == np.uint8 and q.shape[1:] == (N, K // 2) and sb.shape[1:] == (N, K // 16)
        return _Matrix(FMT_NVFP4, q[e].ctypes.data, sb[e].ctypes.data, float(st[e]))

    def _expert(self, e: int) -> _Expert:
        H, I = self.H, self.I
        return _Expert(self._matrix("gate", e, I, H), self._matrix("up", e, I, H),
                       self._matrix("down", e, H, I))

    def ptr(self, e: int = 0):
        return ctypes.cast(ctypes.byref(self.desc, e * ctypes.sizeof(_Expert)),
                           ctypes.POINTER(_Expert))


def expert_ffn(ex: Experts, e: int, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float64)
    out = np.empty(ex.H, np.float64)
    scratch = np.empty(2 * ex.I, np.float64)
    lib().oracle_expert_ffn(ex.H, ex.I, ex.ptr(e), _p(x), _p(scratch), _p(out))
    return out


def moe_tokens(routed: Experts, shared: Experts | None, x_bits: np.ndarray, ids: np.ndarray,
               w: np.ndarray, tokens=None) -> np.ndarray:
    """Combine for the listed tokens (all tokens if None) given routing ids and weights."""
    x_bits = np.ascontiguousarray(x_bits, np.uint16)
    ids = np.ascontiguousarray(ids, np.int32)
    w = np.ascontiguousarray(w, np.float64)
    T, H = x_bits.shape
    k = ids.shape[1]
    tok = np.arange(T, dtype=np.int64) if tokens is None else np.ascontiguousarray(tokens, np.int64)
    y = np.empty((tok.shape[0], H), np.float64)
    lib().oracle_moe_tokens(H, routed.I, routed.n, k, routed.ptr(0),
                            None if shared is None else shared.ptr(0),
                            _p(x_bits), _p(ids), _p(w), tok.shape[0], _p(tok), _p(y))
    return y


def moe_layer(x_bits, Wr, routed: Experts, shared: Experts | None, k: int,
              bias=None, renormalize: bool = True):
    """Whole layer: returns dict(logits, ids, w, y)."""
    logits = router(x_bits, Wr, bias)
    ids = select(logits, k)
    w = weights(logits, ids, renormalize)
    y = moe_tokens(routed, shared, x_bits, ids, w)
    return {"logits": logits, "ids": ids, "w": w, "y": y}
