"""The seeded generators follow their published definition (SplitMix64 + Box-Muller).

A pure-Python rendering of the definition in gen_host.c checks the C generator on a
few hundred elements of several streams; bf16 rounding is checked against numpy's
float32 path where no double rounding can occur.
"""
import math

import numpy as np

from sparse_moe_transformer_wave_amd import datagen as dg

M64 = (1 << 64) - 1
G = 0x9E3779B97F4A7C15


def mix(z):
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def key(seed, stream):
    return mix(mix((stream + G) & M64) ^ ((seed * 0xD1B54A32D192ED03) & M64))


def draw(k, i):
    return mix((k + (i + 1) * G) & M64)


def normal(k, i):
    p = i >> 1
    u1 = ((draw(k, 2 * p) >> 11) + 0.5) * 2.0**-53
    u2 = ((draw(k, 2 * p + 1) >> 11) + 0.5) * 2.0**-53
    r = math.sqrt(-2.0 * math.log(u1))
    th = 2 * math.pi * u2
    return r * math.sin(th) if i & 1 else r * math.cos(th)


def test_draws_follow_definition():
    for seed, stream in [(0, 0), (0, dg.stream_id(3, dg.KIND_GATE, 256)), (7, 12345)]:
        raw = dg.raw_u64(64, seed, stream)
        k = key(seed, stream)
        assert [int(v) for v in raw] == [draw(k, i) for i in range(64)]
        f64 = dg.normal_f64((300,), seed, stream, 0.02)
        ref = np.array([0.02 * normal(k, i) for i in range(300)])
        np.testing.assert_allclose(f64, ref, rtol=1e-15, atol=0)


def test_bf16_rounding_and_determinism():
    a = dg.normal_bf16((4096,), 0, 99, 1.0)
    b = dg.normal_bf16((4096,), 0, 99, 1.0)
    np.testing.assert_array_equal(a, b)
    d = dg.normal_f64((4096,), 0, 99, 1.0)
    # nearest bf16: the error is at most half a bf16 ulp of the value
    v = dg.bf16_bits_to_f32(a).astype(np.float64)
    ulp = 2.0 ** (np.floor(np.log2(np.abs(d))) - 7)
    assert np.all(np.abs(v - d) <= ulp / 2)
    assert abs(d.mean()) < 0.05 and abs(d.std() - 1) < 0.05


def test_rank_permutation_is_a_permutation():
    r = dg.rank_permutation(256, 0, dg.stream_id(0, dg.KIND_ZIPF, 0))
    assert sorted(r) == list(range(1, 257))


def _digest_script():
    import importlib.util
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "make_input_digests.py")
    spec = importlib.util.spec_from_file_location("make_input_digests", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_parity_inputs_match_recorded_digests():
    """The parity tests' seeded inputs (tiny and full-size tokens, router weights, Zipf bias,
    experts in bf16 and as the reference quantisers' NVFP4 / INT4 codes) are the bytes whose
    SHA-256 digests tests/golden/input_digests.json records."""
    import json
    mod = _digest_script()
    rec = json.load(open(mod.OUT))
    assert rec["seed"] == 0 and rec["zipf_c"] == dg.ZIPF_C
    now = mod.compute()
    assert sorted(now) == sorted(rec["tensors"])
    bad = [k for k in now if now[k] != rec["tensors"][k]]
    assert not bad, bad


def test_recorded_digests_describe_the_parity_cases():
    """The tiny parity case builds its inputs from the same draws the digests cover."""
    import hashlib
    import json
    import os
    import sys
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from moe_cases import Case
    import sparse_moe_transformer_wave_amd as fm
    rec = json.load(open(_digest_script().OUT))["tensors"]
    sha = lambda a: hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
    c = Case(32, 256, 128, 256, 6)
    assert sha(c.x) == rec["tiny/x"]["sha256"]
    assert sha(c.Wr) == rec["tiny/Wr"]["sha256"]
    for name in ("gate", "up", "down"):
        both = np.concatenate([c.host[name], c.host_sh[name]])
        assert sha(both) == rec["tiny/bf16/all_experts/" + name]["sha256"]
    c4 = Case(32, 256, 128, 256, 6, fmt=fm.WFMT_INT4, experts=[0, 255])
    for name in ("q_gate", "sb_down"):
        assert sha(c4.host[name][0]) == rec["tiny/int4/expert0/" + name]["sha256"]
        assert sha(c4.host[name][255]) == rec["tiny/int4/expert255/" + name]["sha256"]
        assert sha(c4.host_sh[name][0]) == rec["tiny/int4/expert256/" + name]["sha256"]
