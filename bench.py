#!/usr/bin/env python3
"""MoE-layer benchmark on one MI355X.

The layer: Flint-style MoE FFN (H=2048, I=768, 256 routed experts, top-6 sigmoid routing + 1
shared expert, SwiGLU), seeded synthetic weights N(0, 0.02) and tokens N(0, 1), drawn on the
device before timing.  A step is the whole hot path (router, top-k, grouping, experts,
combine) of every layer of a stack; decode workloads cycle 47 distinct layers (114 GB bf16,
32 GB NVFP4), so every layer streams its experts from HBM, and prefill runs one layer of
8192 tokens.  Steps are replayed from a HIP graph.

The default run measures the whole metric in one JSON line: decode T=1 (the headline `value`),
T=8, T=32, prefill T=8192 with uniform and with Zipf(1.1)-biased routing, and NVFP4 decode
T=1/8/32.  Each workload is timed as `trials` (default 5) replays of a graph of K steps after
W warm-up steps; the line reports the median trial (tokens/s, ms per step) with the IQR, the
roofline (algorithmic HBM bytes or MFMA flops per layer call over the median layer time),
and the reference timed single-threaded on the host on a bounded sample of the same
workload.  It also reports a measured device-to-device copy bandwidth, the seed, the Zipf
constant and SHA-256 digests of the input tokens and of the last layer's output.

Other workloads through --configs: int4_t1/8/32, nvfp4_prefill, int4_prefill, dense_t1/t32/
prefill (the dense SwiGLU layer, no router, I = 4096), nvfp4_dense_t1, int4_dense_t1, and
chain_t1 / nvfp4_chain_t1 / chain_t8 / nvfp4_chain_t8 (one flint_moe_decode_chain call per step
through the 47 layers, 1 or 8 tokens).

The timed trials of each workload sit between two flint_moe_workspace_status calls, whose
one-thread kernel (ws_status_kernel) marks them in a rocprofv3 kernel trace or counter
collection; --summarize-trace turns such a CSV into the markdown tables kept under
profiles/, counting only the dispatches between the markers.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

H, I, E, TOPK, S = 2048, 768, 256, 6, 1
DENSE_I = 4096  # intermediate size of the dense SwiGLU layers (not given by the pages)
SEED = 0
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
    # eight tokens through the 47 layers the same way
    "chain_t8": dict(T=8, fmt=0, layers=47, zipf=False, chain=True),
    "nvfp4_chain_t8": dict(T=8, fmt=1, layers=47, zipf=False, chain=True),
    # dense SwiGLU layers (E = 0, k = 0, the shared expert alone; 16 distinct layers cycled)
    "dense_t1": dict(T=1, fmt=0, layers=16, zipf=False, dense=True),
    "dense_t32": dict(T=32, fmt=0, layers=16, zipf=False, dense=True),
    "dense_prefill": dict(T=8192, fmt=0, layers=1, zipf=False, dense=True),
    # the same dense layer's single token with 4-bit weights (48 layers: 680 MB, more than
    # the last-level cache)
    "nvfp4_dense_t1": dict(T=1, fmt=1, layers=48, zipf=False, dense=True),
    "int4_dense_t1": dict(T=1, fmt=2, layers=48, zipf=False, dense=True),
}
# the metric's workloads: decode T = 1 / 8 / 32 and the 8192-token prefill (uniform and
# Zipf-biased routing) in bf16, and NVFP4 decode T = 1 / 8 / 32; the first is the headline
DEFAULT_CONFIGS = ["decode_t1", "decode_t8", "decode_t32", "prefill", "prefill_zipf",
                   "nvfp4_t1", "nvfp4_t8", "nvfp4_t32"]
FMT_NAME = ("bf16", "NVFP4", "INT4")
DTYPE = ("bf16",
         "nvfp4-w4a16 (e2m1 weights with e4m3 block scales x bf16 activations, fp32 accumulate)",
         "int4-w4a16 (int4 weights, bf16 scale per 128 columns, x bf16 activations, fp32 accumulate)")

METRIC = "MoE-layer tokens/s at T=1/8/32/8192; achieved HBM GB/s or MFMA % of peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "sparse_moe_transformer_wave_amd", "csrc")
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


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


def algorithmic_bytes(fmt, shp, T, touched):
    """HBM bytes one layer call must move: the weights of the `touched` routed experts and of
    the shared expert once each, the fp32 router matrix, the bf16 tokens read and the bf16
    outputs written."""
    H_, I_, E_, _, S_ = shp
    return (touched + S_) * expert_bytes(fmt, H_, I_) + E_ * H_ * 4 + 2 * T * H_ * 2


def layer_flops(shp, T):
    """Multiply-add flops of one layer call's expert FFNs: k routed + S shared experts per
    token, three H x I products each (gate, up, down)."""
    H_, I_, _, k_, S_ = shp
    return 2.0 * T * (k_ + S_) * 3 * H_ * I_


# ------------------------------------------------------------------ counter traffic
def csrc_digest():
    """sha256 over the HIP sources: counter-derived traffic is reported only while the
    kernels it was measured on are unchanged."""
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


def copy_bandwidth(torch, nbytes=4 << 30, reps=5):
    """Device-to-device copy of nbytes (read + write = 2 nbytes moved), median of reps."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b.copy_(a)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        b.copy_(a)
        e.record()
        torch.cuda.synchronize()
        ts.append(s.elapsed_time(e))
    ts.sort()
    ms = ts[len(ts) // 2]
    del a, b
    return {"bytes_moved": 2 * nbytes, "median_ms": round(ms, 4),
            "GB_per_s": round(2 * nbytes / (ms / 1e3) / 1e9, 1),
            "what": "torch device-to-device copy of %d GiB (read + write)" % (nbytes >> 30)}


# ------------------------------------------------------------------ pools
def build_layer(torch, fm, dg, l, fmt, shp):
    """Layer l of the seeded pool, drawn on the device."""
    H_, I_, E_, _, S_ = shp
    d = {"Wr": None}
    if E_:
        d["Wr"] = torch.empty((E_, H_), dtype=torch.float32, device="cuda")
        dg.device_normal_f32(d["Wr"], SEED, dg.stream_id(l, dg.KIND_ROUTER, 0), dg.ROUTER_STD)
    kinds = (("gate", dg.KIND_GATE, I_, H_), ("up", dg.KIND_UP, I_, H_), ("down", dg.KIND_DOWN, H_, I_))
    n = E_ + S_
    if fmt == 0:
        for name, kind, N, K in kinds:
            t = torch.empty((n, N, K), dtype=torch.int16, device="cuda")
            dg.device_normal_bf16(t, n, N * K, SEED, dg.stream_id(l, kind, 0), dg.W_STD)
            d[name] = t
        r = [d["gate"], d["up"], d["down"]] if E_ else [None, None, None]
        d["weights"] = fm.Weights(0, *r, d["gate"][E_], d["up"][E_], d["down"][E_])
    elif fmt == 2:
        for name, kind, N, K in kinds:
            q = torch.empty((n, N, K // 2), dtype=torch.uint8, device="cuda")
            sc = torch.empty((n, N, K // 128), dtype=torch.int16, device="cuda")
            dg.device_int4(q, sc, n, N, K, SEED, dg.stream_id(l, kind, 0), dg.W_STD)
            d["q_" + name], d["sc_" + name] = q, sc
        q = [d["q_gate"], d["q_up"], d["q_down"]] if E_ else [None] * 3
        sc = [d["sc_gate"], d["sc_up"], d["sc_down"]] if E_ else [None] * 3
        d["weights"] = fm.Weights(2, *q, d["q_gate"][E_], d["q_up"][E_], d["q_down"][E_],
                                  *sc, d["sc_gate"][E_], d["sc_up"][E_], d["sc_down"][E_])
    else:
        scratch = torch.empty(n, dtype=torch.int32, device="cuda")
        for name, kind, N, K in kinds:
            q = torch.empty((n, N, K // 2), dtype=torch.uint8, device="cuda")
            sf = torch.empty((n, N, K // 16), dtype=torch.uint8, device="cuda")
            ts = torch.empty(n + 3, dtype=torch.float32, device="cuda")
            dg.device_nvfp4(q, sf, ts, scratch, n, N, K, SEED, dg.stream_id(l, kind, 0), dg.W_STD)
            d["q_" + name], d["sf_" + name], d["ts_" + name] = q, sf, ts
        sh_ts = torch.stack([d["ts_gate"][E_], d["ts_up"][E_], d["ts_down"][E_]]).contiguous()
        d["sh_ts"] = torch.cat([sh_ts, torch.zeros(1, device="cuda")])
        q = [d["q_gate"], d["q_up"], d["q_down"]] if E_ else [None] * 3
        sf = [d["sf_gate"], d["sf_up"], d["sf_down"]] if E_ else [None] * 3
        ts = [d["ts_gate"], d["ts_up"], d["ts_down"]] if E_ else [None] * 3
        d["weights"] = fm.Weights(1, *q, d["q_gate"][E_], d["q_up"][E_], d["q_down"][E_], *sf,
                                  d["sf_gate"][E_], d["sf_up"][E_], d["sf_down"][E_], *ts, d["sh_ts"])
    return d


class Pools:
    """Device pools, built once per (format, dense) and shared by the workloads that use
    them (the prefill runs on layer 0 of the decode stack)."""

    def __init__(self, torch, fm, dg):
        self.torch, self.fm, self.dg = torch, fm, dg
        self.pools = {}

    def layers(self, cfg):
        key = (cfg["fmt"], bool(cfg.get("dense")))
        want = cfg["layers"]
        have = self.pools.get(key, [])
        if len(have) < want:
            t0 = time.time()
            shp = shape_of(cfg)
            have = have + [build_layer(self.torch, self.fm, self.dg, l, cfg["fmt"], shp)
                           for l in range(len(have), want)]
            self.torch.cuda.synchronize()
            self.pools[key] = have
            log("pool %s%s: %d layers, %.1f GB of expert weights, drawn in %.1f s"
                % (FMT_NAME[cfg["fmt"]], " dense" if key[1] else "", want,
                   want * (shp[2] + shp[4]) * expert_bytes(cfg["fmt"], shp[0], shp[1]) / 1e9, time.time() - t0))
        return have[:want]


# ------------------------------------------------------------------ reference on the host
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


def experts_to_host(torch, oracle, d, idx, fmt, H_, I_):
    """The listed experts of a device layer, copied back as the reference's expert arrays."""
    ix = torch.tensor(idx, dtype=torch.long, device="cuda")
    a = {}
    for name in ("gate", "up", "down"):
        if fmt == 0:
            a[name] = d[name][ix].cpu().numpy().view("uint16")
        elif fmt == 1:
            a["q_" + name] = d["q_" + name][ix].cpu().numpy()
            a["sb_" + name] = d["sf_" + name][ix].cpu().numpy()
            a["st_" + name] = d["ts_" + name][ix].cpu().numpy()
        else:
            a["q_" + name] = d["q_" + name][ix].cpu().numpy()
            a["sb_" + name] = d["sc_" + name][ix].cpu().numpy().view("uint16")
    return oracle.Experts((oracle.FMT_BF16, oracle.FMT_NVFP4, oracle.FMT_INT4)[fmt], H_, I_, a)


def cpu_baseline(torch, cfg, layers, x_host, budget_s):
    """The reference (single-threaded C, fp64) on a bounded sample of the same workload and
    the same bytes (the touched experts copied back from the device pool): the whole layer
    (router, selection, weights, experts, combine) for up to 32 of the tokens, layers cycled
    until budget_s of reference time."""
    import numpy as np

    import oracle
    H_, I_, E_, k_, S_ = shape_of(cfg)
    T = cfg["T"] if cfg["T"] <= 32 else 4
    x = np.ascontiguousarray(x_host[:T])
    n_layers = min(len(layers), 8 if T == 1 else 2 if T <= 8 else 1)
    prep = []
    for l in range(n_layers):
        d = layers[l]
        if E_ == 0:
            prep.append((None, None, None, experts_to_host(torch, oracle, d, [0], cfg["fmt"], H_, I_)))
            continue
        Wr = d["Wr"].cpu().numpy()
        bias = d.get("bias")
        bias = None if bias is None else bias.cpu().numpy()
        ids = oracle.select(oracle.router(x, Wr, bias), k_)
        used = sorted(set(ids.reshape(-1).tolist()))
        local = np.zeros(E_, np.int32)
        local[used] = np.arange(len(used), dtype=np.int32)
        routed = experts_to_host(torch, oracle, d, used, cfg["fmt"], H_, I_)
        shared = experts_to_host(torch, oracle, d, [E_], cfg["fmt"], H_, I_)
        prep.append((Wr, bias, local, (routed, shared)))
    xf = x.view(np.uint16)
    done, t_used = 0, 0.0
    while t_used < budget_s or done == 0:
        Wr, bias, local, ex = prep[done % n_layers]
        t0 = time.perf_counter()
        if E_ == 0:
            xd = (xf.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            for t in range(T):
                oracle.expert_ffn(ex, 0, xd[t])
        else:
            logits = oracle.router(x, Wr, bias)
            ids = oracle.select(logits, k_)
            w = oracle.weights(logits, ids, True)
            oracle.moe_tokens(ex[0], ex[1], x, local[ids], w)
        t_used += time.perf_counter() - t0
        done += 1
    what = ("dense SwiGLU layer" if E_ == 0 else "full layer") + (", %s weights" % FMT_NAME[cfg["fmt"]])
    tok_note = "" if cfg["T"] <= 32 else " (the first %d of the batch's %d tokens)" % (T, cfg["T"])
    return {"value": T * done / t_used, "unit": "MoE-layer tokens/s", "cores": 1, "kind": "oracle",
            "sample": "%d token(s)%s x %d layer evaluations (layers 0..%d cycled), %s, single-threaded "
                      "fp64 C reference on the device pool's bytes, %.1f s; host CPU %s, %d logical cores"
                      % (T, tok_note, done, n_layers - 1, what, t_used, host_cpu(), os.cpu_count() or 0)}


# ------------------------------------------------------------------ one workload
def sha256_of(t):
    return hashlib.sha256(t.contiguous().cpu().numpy().tobytes()).hexdigest()


def run_config(name, args, torch, fm, dg, pools):
    import numpy as np
    cfg = CONFIGS[name]
    T, fmt, L = cfg["T"], cfg["fmt"], cfg["layers"]
    shp = shape_of(cfg)
    H_, I_, E_, k_, S_ = shp
    chain = bool(cfg.get("chain"))
    log("config %s: T=%d %s, %d layer(s)%s" % (name, T, FMT_NAME[fmt], L, ", chained" if chain else ""))
    layers = pools.layers(cfg)
    bias = None
    if cfg["zipf"]:
        bias = torch.from_numpy(dg.zipf_bias(E_, dg.ZIPF_C, SEED, 0)).cuda()
    for d in layers:
        d["bias"] = bias
    x = torch.empty((T, H_), dtype=torch.int16, device="cuda")
    dg.device_normal_bf16(x, 1, T * H_, SEED, dg.stream_id(0, dg.KIND_X, 0), dg.X_STD)
    y = torch.empty((T, H_), dtype=torch.int16, device="cuda")
    desc = fm.desc(H_, I_, E_, k_, S_, 1)
    ws = fm.workspace(desc, T, fmt)

    # Routing of every layer (for the algorithmic bytes: distinct experts touched), outside
    # the timed region.
    touched = []
    ychain = None
    L_lib = fm.lib()
    if chain:
        ychain = torch.empty((L, T, H_), dtype=torch.int16, device="cuda")
        refs = fm.layer_refs([(d["weights"], d["Wr"], d["bias"]) for d in layers])
    if E_ and not chain:
        counts = torch.zeros(E_, dtype=torch.int32, device="cuda")
        for d in layers:
            fm.layer(desc, d["weights"], T, x, d["Wr"], d["bias"], y, ws, {"counts": counts})
            touched.append(int((counts > 0).sum().item()))
    elif chain and T > 1:  # each layer's routing from one untimed pass of the chain
        ids = torch.zeros((L, T, k_), dtype=torch.int32, device="cuda")
        fm.decode_chain(desc, [(d["weights"], d["Wr"], d["bias"]) for d in layers], x, ychain, ws,
                        topk_ids=ids, residual=True)
        touched = [len(set(r.reshape(-1).tolist())) for r in ids.cpu().numpy()]
    else:
        touched = [TOPK if E_ else 0] * L  # a single token touches exactly k routed experts
    alg_bytes = [algorithmic_bytes(fmt, shp, T, u) for u in touched]
    flops_layer = layer_flops(shp, T)

    def capture(n_steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            st = torch.cuda.current_stream().cuda_stream
            if chain:
                fn, fname = L_lib.flint_moe_decode_chain, "flint_moe_decode_chain"
                calls = [((ctypes.byref(desc), refs, L, fm.CHAIN_RESIDUAL, T, x.data_ptr(), ychain.data_ptr(),
                           None, None, None, ws.data_ptr(), ws.numel(), st), refs)]
            else:
                fn, fname = L_lib.flint_moe_layer, "flint_moe_layer"
                calls = [fm.layer_ptr_args(desc, d["weights"], T, x, d["Wr"], d["bias"], y,
                                           ws.data_ptr(), ws.numel(), st) for d in layers]
            for _ in range(n_steps):
                for a, _keep in calls:
                    rc = fn(*a)
                    if rc:
                        raise fm.FlintError(rc, fname)
        return g, calls

    g_warm, keep_w = capture(1)
    g_timed, keep_t = capture(args.steps)
    for _ in range(args.warmup):
        g_warm.replay()
    torch.cuda.synchronize()
    # the status call's kernel marks the start of the timed trials in a kernel trace (and
    # checks that no persistent launch timed out during the warm-up)
    assert fm.workspace_status(ws) == 0, "a persistent launch's wait ran out during the warm-up"
    times = []
    for _ in range(args.trials):
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        g_timed.replay()
        e.record()
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e))
    status = fm.workspace_status(ws)  # the end marker
    assert status == 0, "a persistent launch's wait ran out during the timed trials"
    q25, med, q75 = (float(v) for v in np.percentile(times, [25, 50, 75]))
    K = args.steps
    layer_ms = med / (K * L)
    out = {
        "value": round(T * L * K / (med / 1e3), 1), "unit": "MoE-layer tokens/s",
        "ms_per_step": round(med / K, 4), "dtype": DTYPE[fmt] if fmt else "bf16",
        "trials": {"n": args.trials, "median_ms": round(med, 4), "iqr_ms": round(q75 - q25, 4),
                   "all_ms": [round(t, 4) for t in times], "layer_us_median": round(layer_ms * 1e3, 2)},
        "config": {
            "workload": ("%s: T=%d tokens, H=%d, I=%d, E=%d routed, top-%d sigmoid + %d shared, SwiGLU, %s, "
                         "%d distinct layer(s)%s" % (name, T, H_, I_, E_, k_, S_, FMT_NAME[fmt], L,
                                                     ", Zipf(1.1) logit bias (c = %.4f)" % dg.ZIPF_C if cfg["zipf"] else
                                                     ", chained: one flint_moe_decode_chain call per step, token "
                                                     "of layer l + 1 = bf16(x_l + y_l)" if chain else ""))
            if E_ else ("%s: T=%d tokens, dense SwiGLU FFN layer (no router), H=%d, I=%d, %s, %d distinct layers"
                        % (name, T, H_, I_, FMT_NAME[fmt], L)),
            "tokens_per_layer_call": T, "layers": L, "touched_experts_mean": float(np.mean(touched))},
    }
    if T <= 32:
        bytes_per_call = sum(alg_bytes) / L
        achieved = bytes_per_call / (layer_ms / 1e3) / 1e9
        kernel = ("dense1_kernel (the whole dense layer in one persistent launch)" if E_ == 0 and T == 1 else
                  "the dense layer's gate/up and down kernels" if E_ == 0 else
                  "decode1_kernel (one persistent launch per layer; chain time / layers)" if chain and T == 1 else
                  "decode_few_kernel (one persistent launch per layer; chain time / layers)" if chain else
                  "decode1_kernel (the whole layer in one persistent launch)" if T == 1 else
                  "decode_few_kernel (the whole layer in one persistent launch)" if T <= 16 and fmt == 0 else
                  "one layer call: router with selection, gate/up, down and combine kernels")
        out["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(name),
                           "kernel": kernel, "avg_launch_us": round(layer_ms * 1e3, 2),
                           "alg_bytes_per_launch": int(bytes_per_call)}
    else:
        achieved = flops_layer / (layer_ms / 1e3) / 1e12
        out["roofline"] = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                           "traffic": measured_traffic(name),
                           "kernel": "one layer call: router, top-k, grouping, gate/up and down GEMMs, combine",
                           "avg_launch_us": round(layer_ms * 1e3, 2), "alg_flops_per_launch": flops_layer,
                           "alg_bytes_per_launch": int(sum(alg_bytes) / L),
                           "hbm_floor_us": round(sum(alg_bytes) / L / (HBM_PEAK_GBS * 1e9) * 1e6, 1)}
    out["sha256"] = {"x": sha256_of(x), "y_last_layer": sha256_of(ychain[-1] if chain else y)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(torch, cfg, layers, x.cpu().numpy().view("uint16"), args.cpu_seconds)
    log("  %s: %.1f tokens/s, %.2f us per layer (IQR %.4f ms over %d trials), %s %.3f of peak"
        % (name, out["value"], layer_ms * 1e3, q75 - q25, args.trials, out["roofline"]["unit"],
           out["roofline"]["frac"]))
    del keep_w, keep_t, g_warm, g_timed
    return out


# ------------------------------------------------------------------ profile summaries
MARKER = "ws_status_kernel"


def short_kernel_name(n):
    """A rocprofv3 kernel name without return type, namespaces and parameter list."""
    if n.startswith("void "):
        n = n[5:]
    n = n.replace("(anonymous namespace)::", "").replace("flint::", "")
    n = n.split("(")[0]
    return n if len(n) <= 60 else n[:57] + "..."


def summarize_trace(csv_path, title, command, note=""):
    """Markdown table of the kernels of a rocprofv3 kernel trace (kernel_trace.csv) or counter
    collection (counter_collection.csv) that ran between the first two ws_status_kernel
    dispatches, i.e. inside the timed trials of one workload.  For a counter collection the
    table gives each kernel's mean counter value per dispatch."""
    import csv
    rows = list(csv.DictReader(open(csv_path)))
    name_key = "Kernel_Name"
    start_key = "Start_Timestamp"
    end_key = "End_Timestamp"
    rows.sort(key=lambda r: int(r[start_key]))
    marks = [i for i, r in enumerate(rows) if MARKER in r[name_key]]
    if len(marks) < 2:
        raise SystemExit("%s: fewer than two %s dispatches" % (csv_path, MARKER))
    inside = rows[marks[0] + 1:marks[1]]
    counters = "Counter_Name" in rows[0]
    per = {}
    for r in inside:
        nm = r[name_key]
        if counters:
            nm = (nm, r["Counter_Name"])
        per.setdefault(nm, []).append(float(r["Counter_Value"]) if counters else
                                      (int(r[end_key]) - int(r[start_key])) / 1e3)
    window_us = (int(rows[marks[1]][start_key]) - int(rows[marks[0]][end_key])) / 1e3
    note_extra = ("The at::native fill and __amd_rocclr_copyBuffer dispatches in the window are the status "
                  "call's own (its output word is zeroed before and copied to the host after it).")
    note = (note + "\n\n" + note_extra) if note else note_extra
    lines = ["# %s" % title, "", "Command (from the repository root, on one MI355X):", "", "```", command, "```", ""]
    if note:
        lines += [note, ""]
    lines += ["Dispatches between the two %s markers (the timed trials only): %d, over %.1f us."
              % (MARKER, len(inside), window_us), ""]

    if counters:
        lines += ["| kernel | counter | dispatches | mean per dispatch (KiB) | total (KiB) |", "|---|---|---|---|---|"]
        for (nm, ctr), v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            lines.append("| %s | %s | %d | %.1f | %.1f |" % (short_kernel_name(nm), ctr, len(v), sum(v) / len(v), sum(v)))
    else:
        tot = sum(sum(v) for v in per.values())
        lines += ["| kernel | calls | avg us | min us | max us | % of kernel time |", "|---|---|---|---|---|---|"]
        for nm, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            lines.append("| %s | %d | %.2f | %.2f | %.2f | %.2f |" % (short_kernel_name(nm), len(v), sum(v) / len(v), min(v),
                                                                   max(v), 100.0 * sum(v) / tot))
    return "\n".join(lines) + "\n"


def _marked_rows(csv_path):
    """Rows of a rocprofv3 CSV between the first two marker dispatches, by start time."""
    import csv
    rows = sorted(csv.DictReader(open(csv_path)), key=lambda r: int(r["Start_Timestamp"]))
    marks = [i for i, r in enumerate(rows) if MARKER in r["Kernel_Name"]]
    if len(marks) < 2:
        raise SystemExit("%s: fewer than two %s dispatches" % (csv_path, MARKER))
    return rows[marks[0] + 1:marks[1]]


def traffic_json(copy_fetch_csv, copy_write_csv, entries):
    """HBM traffic per layer call from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs (KiB per
    dispatch), each counter scaled so that a plain 1 GiB device copy (bench.py
    --copy-calibration) reads and writes 1 GiB.  entries: NAME=FETCH_CSV,WRITE_CSV strings.
    The layer calls inside the marked window are counted as the fewest dispatches of any one
    of the library's kernels there (every kernel of a layer call runs once per call); the
    status call's own torch and runtime dispatches are left out."""
    import csv
    calib = {}
    for ctr, path in (("FETCH_SIZE", copy_fetch_csv), ("WRITE_SIZE", copy_write_csv)):
        vals = [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
                if "copy" in r["Kernel_Name"].lower() and r["Counter_Name"] == ctr]
        top = max(vals)
        calib[ctr] = {"copy_1GiB_counter_KiB": top, "scale": (1 << 20) / top}
    out = {"csrc_sha256": csrc_digest(),
           "made_by": [
               "rocprofv3 --pmc COUNTER --output-format csv -d gpurun_out/prof/pmc_copy_COUNTER -o run -- "
               "python3 bench.py --copy-calibration",
               "rocprofv3 --pmc COUNTER --output-format csv -d gpurun_out/prof/pmc_NAME_COUNTER -o run -- "
               "python3 bench.py --configs NAME --no-cpu-baseline --no-copy-bandwidth --steps 2 --warmup 1 --trials 1",
               "(COUNTER = FETCH_SIZE, then WRITE_SIZE, one run each), then python3 bench.py --traffic " +
               " ".join([copy_fetch_csv, copy_write_csv] + list(entries))],
           "calibration": calib, "configs": {}}
    for ent in entries:
        name, paths = ent.split("=", 1)
        per_kernel, calls, total = {}, None, 0.0
        for ctr, path in zip(("FETCH_SIZE", "WRITE_SIZE"), paths.split(",")):
            counts = {}
            for r in _marked_rows(path):
                if r["Counter_Name"] != ctr or "flint::" not in r["Kernel_Name"]:
                    continue
                b = float(r["Counter_Value"]) * calib[ctr]["scale"] * 1024.0
                k = short_kernel_name(r["Kernel_Name"])
                per_kernel.setdefault(k, {}).setdefault(ctr, 0.0)
                per_kernel[k][ctr] += b
                counts[k] = counts.get(k, 0) + 1
                total += b
            n = min(counts.values())
            calls = n if calls is None else min(calls, n)
        out["configs"][name] = {
            "layer_calls_counted": calls, "bytes_per_layer_call": int(round(total / calls)),
            "per_kernel_bytes_per_layer_call": {k: {c: int(round(v / calls)) for c, v in d.items()}
                                                for k, d in per_kernel.items()}}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--trials", type=int, default=5)
    ap.add_argument("--configs", default=",".join(DEFAULT_CONFIGS),
                    help="comma-separated workloads; the first is the headline (default: the metric's set)")
    ap.add_argument("--config", default=None, help="a single workload (same as --configs NAME)")
    ap.add_argument("--cpu-seconds", type=float, default=3.0, help="reference time budget per workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-copy-bandwidth", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--traffic", nargs="+", metavar="ARG",
                    help="COPY_FETCH_CSV COPY_WRITE_CSV NAME=FETCH_CSV,WRITE_CSV ...: print the counter "
                         "traffic JSON (profiles/traffic.json) and exit")
    ap.add_argument("--summarize-trace", nargs="+", metavar="ARG",
                    help="CSV TITLE COMMAND [NOTE]: print the markdown summary of the timed trials in a "
                         "rocprofv3 kernel_trace.csv or counter_collection.csv and exit")
    args = ap.parse_args()
    if args.traffic:
        print(json.dumps(traffic_json(args.traffic[0], args.traffic[1], args.traffic[2:]), indent=1))
        return
    if args.summarize_trace:
        print(summarize_trace(*args.summarize_trace), end="")
        return
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    names = [args.config] if args.config else [c for c in args.configs.split(",") if c]
    for n in names:
        if n not in CONFIGS:
            sys.exit("unknown workload %s (known: %s)" % (n, ", ".join(sorted(CONFIGS))))

    import torch

    import sparse_moe_transformer_wave_amd as fm
    from sparse_moe_transformer_wave_amd import datagen as dg

    torch.cuda.init()
    pools = Pools(torch, fm, dg)
    results = {}
    for n in names:
        results[n] = run_config(n, args, torch, fm, dg, pools)
    head = results[names[0]]
    out = {
        "metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": head["dtype"],
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) tokens, drawn on the device; seed %d)" % SEED,
        "config": head["config"], "roofline": head["roofline"], "trials": head["trials"],
    }
    if "cpu_baseline" in head:
        out["cpu_baseline"] = head["cpu_baseline"]
    out["seed"] = SEED
    out["zipf_c"] = dg.ZIPF_C
    prop = torch.cuda.get_device_properties(0)
    out["gpu"] = "%s%s, %d CUs, %.0f GB" % (torch.cuda.get_device_name() + " " if torch.cuda.get_device_name() else "",
                                            getattr(prop, "gcnArchName", "?"), prop.multi_processor_count,
                                            prop.total_memory / 1e9)
    if not args.no_copy_bandwidth:
        out["copy_bandwidth"] = copy_bandwidth(torch)
    out["configs"] = results
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
