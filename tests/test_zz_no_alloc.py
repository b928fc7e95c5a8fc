"""csa2_sparse_attend_noalloc (the attention with the library's own scratch, for
callers that cannot allocate) against csa2_sparse_attend with a caller
workspace: the same kernels on the same inputs give the same bits. Two calls
in a row on one GPU, the second smaller than the first, so the second runs on
scratch the first left full of its partials; both also within the oracle bars."""

import math
import os
import sys

import numpy as np
import pytest
import torch

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu

import compressed_sparse_attention_06_amd as csa2  # noqa: E402
import oracle  # noqa: E402
from devutil import assert_attention_close, dev_cache, dev_window, t  # noqa: E402
from synth import make_small_decode  # noqa: E402

TAU = 1.0 / math.sqrt(512.0)

CALLS = [
    # 8 rows of 2048 entries + 128 window rows: every row cut between 17 workgroups
    dict(contexts=[4 * 2500] * 8, k=2048, page_size=64, shuffle=True),
    # then a smaller call: 3 rows, k 300, ragged contexts (one shorter than k)
    dict(contexts=[4 * 700, 4 * 150, 4 * 1500 + 3], k=300, page_size=16, shuffle=True, row_scale=True),
]


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.lib()


def test_noalloc_attend_matches_workspace_attend():
    for i, case in enumerate(CALLS):
        print(f"noalloc call {i}: {case}", flush=True)
        wl = make_small_decode(layers="F", **case)
        L, c = wl.layers[0], wl.caches[0]
        r = oracle.layer_step("F", c, L.win, L.q, L.qix_codes, L.qix_scales, L.w, k=wl.k)
        dc, dw, idx, q = dev_cache(c), dev_window(L.win), t(r["idx"]), t(L.q)
        ref_out, ref_lse = csa2.sparse_attend(dc, idx, q, dw)
        out = torch.full_like(ref_out, float("nan"))
        lse = torch.full_like(ref_lse, float("nan"))
        csa2.sparse_attend_noalloc(dc, idx, q, dw, out, lse)
        torch.cuda.synchronize()
        g_out, g_lse = out.cpu().numpy(), lse.cpu().numpy()
        w_out, w_lse = ref_out.cpu().numpy(), ref_lse.cpu().numpy()
        assert np.array_equal(g_out, w_out), f"call {i}: out differs from the workspace entry point"
        assert np.array_equal(g_lse, w_lse), f"call {i}: lse differs from the workspace entry point"
        assert_attention_close(g_out, g_lse, r["out"], r["lse"], f"noalloc call {i}")


def test_noalloc_rejects_missing_outputs():
    wl = make_small_decode([4 * 300], layers="F", k=16)
    L, c = wl.layers[0], wl.caches[0]
    idx = t(np.zeros((1, 1, 16), np.int32))
    with pytest.raises(csa2.CSA2Error):
        csa2.sparse_attend_noalloc(dev_cache(c), idx, t(L.q), dev_window(L.win), None, None)
