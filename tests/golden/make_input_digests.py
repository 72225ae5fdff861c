"""Writes tests/golden/input_digests.json: SHA-256 digests of the seeded inputs the parity
tests feed both the reference and the GPU library (seed 0, layer 0).

The tensors are drawn by the host generator (sparse_moe_transformer_wave_amd.datagen) and,
for the 4-bit formats, quantised by the reference's quantisers (oracle/), exactly as the
parity cases draw them: the tiny layer (T = 32, H = 256, I = 128, E = 256, top-6 + shared)
in bf16 with every expert, NVFP4 and INT4 for experts 0 and 255 and the shared expert; and
the full-size layer (H = 2048, I = 768) tokens for T = 1, 8, 32, its router weights, the
Zipf logit bias, and expert 0 and the shared expert in all three formats.  A digest is taken
over the array's bytes (C order, little-endian) and stored with its dtype and shape, so the
record shows that the inputs are the same bytes on every machine.
Run:  python tests/golden/make_input_digests.py
"""
import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402
from sparse_moe_transformer_wave_amd import datagen as dg  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "input_digests.json")
SEED, LAYER, E = 0, 0, 256
MATS = (("gate", dg.KIND_GATE, True), ("up", dg.KIND_UP, True), ("down", dg.KIND_DOWN, False))


def digest(a):
    a = np.ascontiguousarray(a)
    return {"dtype": str(a.dtype), "shape": list(a.shape), "sha256": hashlib.sha256(a.tobytes()).hexdigest()}


def expert_tensors(H, I, e, fmt):
    """Expert e's matrices as the parity cases build them (e = E is the shared expert)."""
    out = {}
    for name, kind, gate_like in MATS:
        N, K = (I, H) if gate_like else (H, I)
        sid = dg.stream_id(LAYER, kind, e)
        if fmt == "bf16":
            out[name] = dg.normal_bf16((N, K), SEED, sid, dg.W_STD)
            continue
        W = dg.normal_f64((N, K), SEED, sid, dg.W_STD)
        if fmt == "nvfp4":
            q, sb, st = oracle.nvfp4_quantize(W)
            out["q_" + name], out["sb_" + name] = q, sb
            out["st_" + name] = np.array([st], np.float32)
        else:
            q, sb = oracle.int4_quantize(W)
            out["q_" + name], out["sb_" + name] = q, sb
    return out


def compute():
    d = {}
    H, I = 256, 128
    d["tiny/x"] = digest(dg.normal_bf16((32, H), SEED, dg.stream_id(LAYER, dg.KIND_X, 0), dg.X_STD))
    d["tiny/Wr"] = digest(dg.normal_f32((E, H), SEED, dg.stream_id(LAYER, dg.KIND_ROUTER, 0), dg.ROUTER_STD))
    stacks = {}
    for e in range(E + 1):
        for name, a in expert_tensors(H, I, e, "bf16").items():
            stacks.setdefault(name, []).append(a)
    for name, arrs in stacks.items():
        d["tiny/bf16/all_experts/" + name] = digest(np.stack(arrs))
    for fmt in ("nvfp4", "int4"):
        for e in (0, 255, E):
            for name, a in expert_tensors(H, I, e, fmt).items():
                d["tiny/%s/expert%d/%s" % (fmt, e, name)] = digest(a)
    H, I = 2048, 768
    for T in (1, 8, 32):
        d["full/x_T%d" % T] = digest(dg.normal_bf16((T, H), SEED, dg.stream_id(LAYER, dg.KIND_X, 0), dg.X_STD))
    d["full/Wr"] = digest(dg.normal_f32((E, H), SEED, dg.stream_id(LAYER, dg.KIND_ROUTER, 0), dg.ROUTER_STD))
    d["full/zipf_bias"] = digest(dg.zipf_bias(E, dg.ZIPF_C, SEED, LAYER))
    for fmt in ("bf16", "nvfp4", "int4"):
        for e in (0, E):
            for name, a in expert_tensors(H, I, e, fmt).items():
                d["full/%s/expert%d/%s" % (fmt, e, name)] = digest(a)
    return d


def main():
    with open(OUT, "w") as fh:
        json.dump({"seed": SEED, "layer": LAYER, "zipf_c": dg.ZIPF_C, "tensors": compute()}, fh, indent=1,
                  sort_keys=True)
        fh.write("\n")
    print("wrote", OUT)


if __name__ == "__main__":
    main()
