"""flint_moe_layer_noalloc (the layer on the library's own per-GPU scratch array, for callers
that cannot allocate) against flint_moe_layer with a workspace of the caller's: the same
kernels, so y and every routing output must be bit-identical, and y meets the reference's
parity bar.  Two calls in a row, the second with fewer tokens, so the second call runs on an
array that still holds the first call's contents; once on the streaming and grouped paths
(T = 64 then 5) and once on the single-token launch, whose exchange words live in the
array's head (T = 8 then 1, at H = 2048)."""
import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(__file__))

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import sparse_moe_transformer_wave_amd as fm  # noqa: E402
from moe_cases import Case, check_forward, check_routing, to_host  # noqa: E402

_ROUTING = ("logits", "topk_ids", "topk_w", "counts", "offsets", "sorted_assign", "assign_pos")


def _pair(c):
    """(flint_moe_layer outputs, flint_moe_layer_noalloc outputs), both on the host."""
    c.upload()
    outs = []
    for noalloc in (False, True):
        out = c.alloc_out()
        routing = {k: out[k] for k in _ROUTING}
        if noalloc:
            fm.layer_noalloc(c.desc, c.weights, c.T, c.d_x, c.d_Wr, c.d_bias, out["y"], routing)
        else:
            fm.layer(c.desc, c.weights, c.T, c.d_x, c.d_Wr, c.d_bias, out["y"], c.workspace(), routing)
        torch.cuda.synchronize()
        outs.append(to_host(out, c))
    return outs


@pytest.mark.parametrize("H,I,T1,T2", [(256, 128, 64, 5), (2048, 768, 8, 1)])
def test_noalloc_matches_layer(H, I, T1, T2):
    for layer, T in ((0, T1), (1, T2)):
        print("noalloc: H=%d I=%d T=%d layer=%d" % (H, I, T, layer), flush=True)
        c = Case(T, H, I, 256, 6, layer=layer)
        ref, got = _pair(c)
        for k in _ROUTING + ("y",):
            np.testing.assert_array_equal(got[k], ref[k], err_msg=k)
        w64 = check_routing(c, got)
        check_forward(c, got, w64)
