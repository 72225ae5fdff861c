#!/usr/bin/env python3
"""MoE-layer benchmark on one MI355X.

Default workload: decode, T = 1 token per step through a stack of 47 distinct Flint-style
MoE layers (H=2048, I=768, 256 routed experts, top-6 sigmoid routing + 1 shared expert,
SwiGLU, bf16 weights N(0, 0.02), x ~ N(0, 1)).  The 47 layers hold 114 GB of expert
weights, so every layer streams its experts from HBM.  One step = the whole hot path
(router, top-k, grouping, experts, combine) for every layer of the stack, replayed from a
HIP graph.  Inputs are seeded synthetic data drawn on the device before timing.

Prints one JSON line: MoE-layer tokens/s, the roofline of the dominant kernel (bytes or
flops per launch over its measured duration) and the reference's single-core CPU rate on
a bounded sample.  --config picks another workload: decode_t8, decode_t32, prefill,
prefill_zipf, nvfp4_t1, nvfp4_t8, nvfp4_t32, nvfp4_prefill, int4_t1, int4_t8, int4_t32, int4_prefill, and the dense SwiGLU layer
(no router, I = 4096) at dense_t1, dense_t32, dense_prefill (and nvfp4_dense_t1, int4_dense_t1
with 4-bit weights); chain_t1 and nvfp4_chain_t1
run the single token through all 47 layers with one flint_moe_decode_chain call (token of
layer l + 1 = bf16(x_l + y_l), formed in the kernel of layer l).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

H, I, E, TOPK, S = 2048, 768, 256, 6, 1
DENSE_I = 4096  # intermediate size of the dense SwiGLU layers (not given by the pages)
CONFIGS = {
    "decode_t1": dict(T=1, fmt=0, layers=47, zipf=False),
    "decode_t8": dict(T=8, fmt=0, layers=47, zipf=False),
    "decode_t32": dict(T=32, fmt=0, layers=47, zipf=False),
    "prefill": dict(T=8192, fmt=0, layers=1, zipf=False),
    "prefill_zipf": dict(T=8192, fmt=0, layers=1, zipf=True),
    "nvfp4_t1": dict(T=1, fmt=1, layers=47, zipf=False),
    "nvfp4_t8": dict(T=8, fmt=1, layers=47, zipf=False),
    "nvfp4_t32": dict(T=32, fmt=1, layers=47, zipf=False),
    "nvfp4_prefill": dict(T=8192, fmt=1, layers=1, zipf=False),
    # INT4 W4A16 (signed nibbles, one bf16 scale per 128 columns), same shapes
    "int4_t1": dict(T=1, fmt=2, layers=47, zipf=False),
    "int4_t8": dict(T=8, fmt=2, layers=47, zipf=False),
    "int4_t32": dict(T=32, fmt=2, layers=47, zipf=False),
    "int4_prefill": dict(T=8192, fmt=2, layers=1, zipf=False),
    # one token through the 47 layers in one flint_moe_decode_chain call, each layer's token =
    # bf16(previous token + previous layer's output) formed by the previous layer's kernel
    "chain_t1": dict(T=1, fmt=0, layers=47, zipf=False, chain=True),
    "nvfp4_chain_t1": dict(T=1, fmt=1, layers=47, zipf=False, chain=True),
    # dense SwiGLU layers (E = 0, k = 0, the shared expert alone; 16 distinct layers cycled)
    "dense_t1": dict(T=1, fmt=0, layers=16, zipf=False, dense=True),
    "dense_t32": dict(T=32, fmt=0, layers=16, zipf=False, dense=True),
    "dense_prefill": dict(T=8192, fmt=0, layers=1, zipf=False, dense=True),
    # the same dense layer's single token with 4-bit weights (48 layers: 680 MB, more than
    # the last-level cache)
    "nvfp4_dense_t1": dict(T=1, fmt=1, layers=48, zipf=False, dense=True),
    "int4_dense_t1": dict(T=1, fmt=2, layers=48, zipf=False, dense=True),
}


def shape_of(cfg):
    """(H, I, E, k, S) of a workload."""
    if cfg.get("dense"):
        return H, DENSE_I, 0, 0, 1
    return H, I, E, TOPK, S


def expert_bytes(fmt, H_, I_):
    if fmt == 0:
        return 3 * I_ * H_ * 2
    if fmt == 1:
        return 3 * (I_ * H_ // 2 + I_ * H_ // 16) + 3 * 4
    return 3 * (I_ * H_ // 2 + I_ * H_ // 64)
METRIC = "MoE-layer tokens/s at T=1/8/32/8192; achieved HBM GB/s or MFMA % of peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "sparse_moe_transformer_wave_amd", "csrc")
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def csrc_digest():
    """sha256 over the HIP sources: counter-derived traffic is reported only while the
    kernels it was measured on are unchanged."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            h.update(open(os.path.join(CSRC, name), "rb").read())
    return h.hexdigest()


def measured_traffic(config):
    """HBM bytes per layer call from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    (scaled by the copy-kernel calibration), or None if absent or stale."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("csrc_sha256") != csrc_digest():
        return None
    entry = t.get("configs", {}).get(config)
    return None if entry is None else entry.get("bytes_per_layer_call")


def copy_calibration():
    """A plain 1 GiB device-to-device copy, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "launches": 3}))


def build_layer(torch, fm, dg, l, fmt, zipf, shp):
    """Layer l of the seeded pool, drawn on the device."""
    H, I, E, _, S = shp
    d = {"Wr": None, "bias": None}
    if E:
        d["Wr"] = torch.empty((E, H), dtype=torch.float32, device="cuda")
        dg.device_normal_f32(d["Wr"], 0, dg.stream_id(l, dg.KIND_ROUTER, 0), dg.ROUTER_STD)
        d["bias"] = torch.from_numpy(dg.zipf_bias(E, dg.ZIPF_C, 0, l)).cuda() if zipf else None
    kinds = (("gate", dg.KIND_GATE, I, H), ("up", dg.KIND_UP, I, H), ("down", dg.KIND_DOWN, H, I))
    if fmt == 0:
        for name, kind, N, K in kinds:
            t = torch.empty((E + S, N, K), dtype=torch.int16, device="cuda")
            dg.device_normal_bf16(t, E + S, N * K, 0, dg.stream_id(l, kind, 0), dg.W_STD)
            d[name] = t
        if E == 0:  # dense layer: the shared expert's pointers only
            d["weights"] = fm.Weights(0, None, None, None, d["gate"][0], d["up"][0], d["down"][0])
        else:
            d["weights"] = fm.Weights(0, d["gate"], d["up"], d["down"], d["gate"][E], d["up"][E],
                                      d["down"][E])
    elif fmt == 2:
        for name, kind, N, K in kinds:
            q = torch.empty((E + S, N, K // 2), dtype=torch.uint8, device="cuda")
            sc = torch.empty((E + S, N, K // 128), dtype=torch.int16, device="cuda")
            dg.device_int4(q, sc, E + S, N, K, 0, dg.stream_id(l, kind, 0), dg.W_STD)
            d["q_" + name], d["sc_" + name] = q, sc
        if E == 0:  # dense layer: the shared expert's pointers only
            d["weights"] = fm.Weights(2, None, None, None, d["q_gate"][0], d["q_up"][0], d["q_down"][0],
                                      None, None, None, d["sc_gate"][0], d["sc_up"][0], d["sc_down"][0])
        else:
            d["weights"] = fm.Weights(
                2, d["q_gate"], d["q_up"], d["q_down"], d["q_gate"][E], d["q_up"][E], d["q_down"][E],
                d["sc_gate"], d["sc_up"], d["sc_down"], d["sc_gate"][E], d["sc_up"][E], d["sc_down"][E])
    else:
        scratch = torch.empty(E + S, dtype=torch.int32, device="cuda")
        for name, kind, N, K in kinds:
            q = torch.empty((E + S, N, K // 2), dtype=torch.uint8, device="cuda")
            sf = torch.empty((E + S, N, K // 16), dtype=torch.uint8, device="cuda")
            ts = torch.empty(E + S + 3, dtype=torch.float32, device="cuda")
            dg.device_nvfp4(q, sf, ts, scratch, E + S, N, K, 0, dg.stream_id(l, kind, 0), dg.W_STD)
            d["q_" + name], d["sf_" + name], d["ts_" + name] = q, sf, ts
        sh_ts = torch.stack([d["ts_gate"][E], d["ts_up"][E], d["ts_down"][E]]).contiguous()
        sh_ts = torch.cat([sh_ts, torch.zeros(1, device="cuda")])
        d["sh_ts"] = sh_ts
        if E == 0:  # dense layer: the shared expert's pointers only
            d["weights"] = fm.Weights(
                1, None, None, None, d["q_gate"][0], d["q_up"][0], d["q_down"][0], None, None, None,
                d["sf_gate"][0], d["sf_up"][0], d["sf_down"][0], None, None, None, sh_ts)
        else:
            d["weights"] = fm.Weights(
                1, d["q_gate"], d["q_up"], d["q_down"], d["q_gate"][E], d["q_up"][E], d["q_down"][E],
                d["sf_gate"], d["sf_up"], d["sf_down"], d["sf_gate"][E], d["sf_up"][E],
                d["sf_down"][E], d["ts_gate"], d["ts_up"], d["ts_down"], sh_ts)
    return d


def cpu_baseline(cfg, budget_s):
    """The reference (single-threaded C, fp64) on a bounded sample of the same workload:
    the whole layer (router, selection, weights, experts, combine) for cfg's T tokens
    through layers 0..7 of the stack, cycled until budget_s of reference time."""
    import numpy as np

    import oracle
    from sparse_moe_transformer_wave_amd import datagen as dg
    H, I, E, TOPK, S = shape_of(cfg)
    nvfp4 = cfg["fmt"] == 1
    int4 = cfg["fmt"] == 2
    # host quantisation costs ~1 s per expert: NVFP4 samples 2 tokens of one layer
    T = min(cfg["T"], 2) if nvfp4 else cfg["T"] if cfg["T"] <= 32 else 4
    n_layers = min(1 if nvfp4 else 8, cfg["layers"])
    x = dg.normal_bf16((cfg["T"], H), 0, dg.stream_id(0, dg.KIND_X, 0), dg.X_STD)[:T]
    x = np.ascontiguousarray(x)
    if E == 0:
        return cpu_baseline_dense(cfg, budget_s, x, H, I, n_layers)
    layers = []
    for l in range(n_layers):
        Wr = dg.normal_f32((E, H), 0, dg.stream_id(l, dg.KIND_ROUTER, 0), dg.ROUTER_STD)
        bias = dg.zipf_bias(E, dg.ZIPF_C, 0, l) if cfg["zipf"] else None
        ids = oracle.select(oracle.router(x, Wr, bias), TOPK)
        used = sorted(set(ids.reshape(-1).tolist()))
        local = {e: i for i, e in enumerate(used)}
        arrays = {}
        for e in used + [E]:
            for name, kind, shape in (("gate", dg.KIND_GATE, (I, H)), ("up", dg.KIND_UP, (I, H)),
                                      ("down", dg.KIND_DOWN, (H, I))):
                if nvfp4:
                    q, sb, st = oracle.nvfp4_quantize(dg.normal_f64(shape, 0, dg.stream_id(l, kind, e), dg.W_STD))
                    for pre, v in (("q_", q), ("sb_", sb), ("st_", np.float32(st))):
                        arrays.setdefault(pre + name, []).append(v)
                elif int4:
                    q, sb = oracle.int4_quantize(dg.normal_f64(shape, 0, dg.stream_id(l, kind, e), dg.W_STD))
                    for pre, v in (("q_", q), ("sb_", sb)):
                        arrays.setdefault(pre + name, []).append(v)
                else:
                    arrays.setdefault(name, []).append(dg.normal_bf16(shape, 0, dg.stream_id(l, kind, e), dg.W_STD))
        fmt_o = oracle.FMT_NVFP4 if nvfp4 else oracle.FMT_INT4 if int4 else oracle.FMT_BF16
        routed = oracle.Experts(fmt_o, H, I, {k: np.stack(v[:-1]) for k, v in arrays.items()})
        shared = oracle.Experts(fmt_o, H, I, {k: np.stack(v[-1:]) for k, v in arrays.items()})
        layers.append((Wr, bias, local, routed, shared))
    done, t_used = 0, 0.0
    while t_used < budget_s:
        Wr, bias, local, routed, shared = layers[done % n_layers]
        t0 = time.perf_counter()
        logits = oracle.router(x, Wr, bias)
        ids = oracle.select(logits, TOPK)
        w = oracle.weights(logits, ids, True)
        lid = np.vectorize(local.get)(ids).astype(np.int32)
        oracle.moe_tokens(routed, shared, x, lid, w)
        t_used += time.perf_counter() - t0
        done += 1
    return cpu_result(T, done, n_layers, t_used, "full layer, NVFP4 weights" if nvfp4 else
                      "full layer, INT4 weights" if int4 else "full layer")


def host_cpu():
    cpu = platform.processor() or platform.machine()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return cpu


def cpu_result(T, done, n_layers, t_used, what):
    return {"value": T * done / t_used, "unit": "MoE-layer tokens/s", "cores": 1, "kind": "oracle",
            "sample": "%d token(s) x %d layer evaluations (layers 0..%d cycled), %s, "
                      "single-threaded fp64 C reference, %.1f s; host CPU %s, %d logical cores"
                      % (T, done, n_layers - 1, what, t_used, host_cpu(), os.cpu_count() or 0)}


def cpu_baseline_dense(cfg, budget_s, x, H, I, n_layers):
    """The reference's SwiGLU expert (the dense layer) for each token, layers cycled; 4-bit
    weights are quantised on the host by the reference's own quantisers."""
    import numpy as np

    import oracle
    from sparse_moe_transformer_wave_amd import datagen as dg
    fmt = cfg["fmt"]
    layers = []
    for l in range(n_layers):
        arrays = {}
        for name, kind, shape in (("gate", dg.KIND_GATE, (I, H)), ("up", dg.KIND_UP, (I, H)),
                                  ("down", dg.KIND_DOWN, (H, I))):
            if fmt == 0:
                arrays[name] = dg.normal_bf16(shape, 0, dg.stream_id(l, kind, 0), dg.W_STD)[None]
            elif fmt == 1:
                q, sb, st = oracle.nvfp4_quantize(dg.normal_f64(shape, 0, dg.stream_id(l, kind, 0), dg.W_STD))
                arrays["q_" + name], arrays["sb_" + name] = q[None], sb[None]
                arrays["st_" + name] = np.array([st], dtype=np.float32)
            else:
                q, sb = oracle.int4_quantize(dg.normal_f64(shape, 0, dg.stream_id(l, kind, 0), dg.W_STD))
                arrays["q_" + name], arrays["sb_" + name] = q[None], sb[None]
        fmt_o = (oracle.FMT_BF16, oracle.FMT_NVFP4, oracle.FMT_INT4)[fmt]
        layers.append(oracle.Experts(fmt_o, H, I, arrays))
    xf = dg.bf16_bits_to_f32(x).astype(np.float64)
    done, t_used = 0, 0.0
    while t_used < budget_s:
        ex = layers[done % n_layers]
        t0 = time.perf_counter()
        for t in range(x.shape[0]):
            oracle.expert_ffn(ex, 0, xf[t])
        t_used += time.perf_counter() - t0
        done += 1
    return cpu_result(x.shape[0], done, n_layers, t_used, ("dense SwiGLU layer", "dense SwiGLU layer, NVFP4 weights",
                                                          "dense SwiGLU layer, INT4 weights")[fmt])


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="decode_t1", choices=sorted(CONFIGS))
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_moe_transformer_wave_amd as fm
    from sparse_moe_transformer_wave_amd import datagen as dg

    cfg = CONFIGS[args.config]
    T, fmt, L = cfg["T"], cfg["fmt"], cfg["layers"]
    shp = shape_of(cfg)
    H, I, E, TOPK, S = shp
    torch.cuda.init()
    log("config %s: T=%d fmt=%s layers=%d" % (args.config, T, ("bf16", "nvfp4", "int4")[fmt], L))
    t0 = time.time()
    layers = [build_layer(torch, fm, dg, l, fmt, cfg["zipf"], shp) for l in range(L)]
    x = torch.empty((T, H), dtype=torch.int16, device="cuda")
    dg.device_normal_bf16(x, 1, T * H, 0, dg.stream_id(0, dg.KIND_X, 0), dg.X_STD)
    y = torch.empty((T, H), dtype=torch.int16, device="cuda")
    desc = fm.desc(H, I, E, TOPK, S, 1)
    ws = fm.workspace(desc, T, fmt)
    torch.cuda.synchronize()
    xb = expert_bytes(fmt, H, I)
    log("pool ready (%.1f GB of expert weights) in %.1f s"
        % (L * (E + S) * xb / 1e9, time.time() - t0))

    # Routing of every layer (for the algorithmic byte count: distinct experts touched).
    touched = []
    if E:
        counts = torch.zeros(E, dtype=torch.int32, device="cuda")
        for d in layers:
            fm.layer(desc, d["weights"], T, x, d["Wr"], d["bias"], y, ws, {"counts": counts})
            touched.append(int((counts > 0).sum().item()))
    else:
        for d in layers:
            fm.layer(desc, d["weights"], T, x, None, None, y, ws)
            touched.append(0)
    chain = bool(cfg.get("chain"))
    if chain:  # a single token touches exactly k routed experts in every layer
        touched = [TOPK] * L
        ychain = torch.empty((L, H), dtype=torch.int16, device="cuda")
        refs = fm.layer_refs([(d["weights"], d["Wr"], d["bias"]) for d in layers])
    alg_bytes = [(u + S) * xb + E * H * 4 + 4 * T * H for u in touched]
    flops_layer = 2.0 * T * (TOPK + S) * 3 * H * I

    stream = torch.cuda.current_stream()
    L_lib = fm.lib()

    def capture(n_steps, with_events):
        ev = []
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            st = torch.cuda.current_stream().cuda_stream
            if chain:
                fn, name = L_lib.flint_moe_decode_chain, "flint_moe_decode_chain"
                calls = [((ctypes.byref(desc), refs, L, fm.CHAIN_RESIDUAL, x.data_ptr(), ychain.data_ptr(),
                           None, None, None, ws.data_ptr(), ws.numel(), st), refs)]
            else:
                fn, name = L_lib.flint_moe_layer, "flint_moe_layer"
                calls = [fm.layer_ptr_args(desc, d["weights"], T, x, d["Wr"], d["bias"], y,
                                           ws.data_ptr(), ws.numel(), st) for d in layers]
            for _ in range(n_steps):
                for a, _keep in calls:
                    if with_events:
                        e = torch.cuda.Event(enable_timing=True, external=True)
                        e.record()
                        ev.append(e)
                    rc = fn(*a)
                    if rc:
                        raise fm.FlintError(rc, name)
            if with_events:
                e = torch.cuda.Event(enable_timing=True, external=True)
                e.record()
                ev.append(e)
        return g, ev, calls

    g_warm, _, keep_w = capture(1, False)
    try:
        g_timed, evs, keep_t = capture(args.steps, True)
    except RuntimeError as exc:  # no event nodes in graphs: time whole replays only
        log("events inside the graph unavailable (%s); per-call time = replay / calls" % exc)
        torch.cuda.synchronize()
        g_timed, evs, keep_t = capture(args.steps, False)
    log("graphs captured (%d + %d layer calls)" % (L, L * args.steps))
    for _ in range(args.warmup):
        g_warm.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    g_timed.replay()
    end.record()
    torch.cuda.synchronize()
    elapsed_ms = start.elapsed_time(end)
    if evs:
        per_call = [evs[i].elapsed_time(evs[i + 1]) for i in range(len(evs) - 1)]
        if chain:  # one event interval per chain call of L layers
            per_call = [t / L for t in per_call for _ in range(L)]
    else:
        per_call = [elapsed_ms / (L * args.steps)] * (L * args.steps)
    log("timed %d steps: %.3f ms" % (args.steps, elapsed_ms))

    K = args.steps
    tokens = T * L * K
    value = tokens / (elapsed_ms / 1e3)
    avg_call_ms = sum(per_call) / len(per_call)
    if T <= 32:
        bytes_per_call = sum(alg_bytes) / L
        achieved = bytes_per_call / (avg_call_ms / 1e3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(args.config),
                "kernel": ("dense1_kernel (the whole dense layer in one persistent launch)" if E == 0 and T == 1 else
                           "flint_moe_layer (dense: gate/up and down kernels)" if E == 0 else
                           "decode1_kernel (one persistent launch per layer; chain call time / layers)"
                           if chain else
                           "decode1_kernel (the whole layer in one persistent launch)" if T == 1 else
                           "flint_moe_layer (router with selection, gate/up, down, combine kernels)"),
                "avg_launch_us": round(avg_call_ms * 1e3, 2),
                "alg_bytes_per_launch": int(bytes_per_call)}
    else:
        achieved = flops_layer / (avg_call_ms / 1e3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(args.config),
                "kernel": "flint_moe_layer (one layer: all kernels)",
                "avg_launch_us": round(avg_call_ms * 1e3, 2), "alg_flops_per_launch": flops_layer}
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "MoE-layer tokens/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(elapsed_ms / K, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("bf16" if fmt == 0 else "nvfp4-w4a16 (e2m1 weights x bf16 activations, fp32 accumulate)"
                  if fmt == 1 else "int4-w4a16 (int4 weights, bf16 scale per 128, x bf16 activations, fp32 accumulate)"),
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) tokens, drawn on device)",
        "config": {"workload": ("%s: T=%d tokens, H=%d, I=%d, E=%d routed, top-%d sigmoid + %d shared, "
                                "SwiGLU, %s, %d distinct layers cycled%s"
                                % (args.config, T, H, I, E, TOPK, S, ("bf16", "NVFP4", "INT4")[fmt],
                                   L, ", Zipf(1.1) logit bias" if cfg["zipf"] else
                                   ", chained: one flint_moe_decode_chain call per step, token of layer l + 1 = "
                                   "bf16(x_l + y_l)" if chain else "")) if E else
                               ("%s: T=%d tokens, dense SwiGLU FFN layer (no router), H=%d, I=%d, "
                                "%s, %d distinct layers cycled" % (args.config, T, H, I,
                                                                   "bf16" if fmt == 0 else "NVFP4", L)),
                   "tokens_per_layer_call": T, "layers": L, "touched_experts_mean": float(np.mean(touched))},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("timing the reference on the host (%.0f s budget)" % args.cpu_seconds)
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    del keep_w, keep_t


if __name__ == "__main__":
    main()
