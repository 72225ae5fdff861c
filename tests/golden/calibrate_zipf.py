"""Writes tests/golden/zipf_c.txt: the Zipf logit-bias strength c of the prefill workload.

The skewed prefill workload adds bias_e = -c * 1.1 * ln(rank_e) to the router logits so
that the 16 hottest experts receive about half of all assignments.  This script finds c
by bisection on the seeded 8192-token input (H=2048, E=256, k=6, seed 0, layer 0), using
only the reference router and selection from oracle/ and the seeded generators.
Run:  python tests/golden/calibrate_zipf.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402
from sparse_moe_transformer_wave_amd import datagen as dg  # noqa: E402

T, H, E, K, SEED, LAYER = 8192, 2048, 256, 6, 0, 0


def hot16_share(logits, c):
    bias = dg.zipf_bias(E, c, SEED, LAYER).astype(np.float64)
    ids = oracle.select(logits + bias[None, :], K)
    counts = np.bincount(ids.reshape(-1), minlength=E)
    return np.sort(counts)[::-1][:16].sum() / (T * K), counts


def main():
    x = dg.normal_bf16((T, H), SEED, dg.stream_id(LAYER, dg.KIND_X, 0), dg.X_STD)
    Wr = dg.normal_f32((E, H), SEED, dg.stream_id(LAYER, dg.KIND_ROUTER, 0), dg.ROUTER_STD)
    logits = oracle.router(x, Wr)
    lo, hi = 0.0, 2.0
    for _ in range(40):
        mid = 0.5 * (lo + hi)
        share, _ = hot16_share(logits, mid)
        lo, hi = (mid, hi) if share < 0.5 else (lo, mid)
    c = round(0.5 * (lo + hi), 4)
    share, counts = hot16_share(logits, c)
    out = os.path.join(os.path.dirname(os.path.abspath(__file__)), "zipf_c.txt")
    with open(out, "w") as f:
        f.write("# Zipf(s=1.1) logit-bias strength for the 8192-token prefill workload\n")
        f.write("# (H=2048, E=256, k=6, seed 0, layer 0); written by calibrate_zipf.py\n")
        f.write("c %.4f\nhot16_share %.6f\nmin_count %d\nmax_count %d\n"
                % (c, share, counts.min(), counts.max()))
    print(open(out).read())


if __name__ == "__main__":
    main()
