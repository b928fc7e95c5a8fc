"""The benchmark workloads at full size on the GPU, checked against the oracle on
sampled requests (decode) or sampled query rows (prefill chunk).

The GPU runs every request / query row of the workload in one pass, in the
same launch configuration the benchmark times; the oracle recomputes only the
sampled ones (every layer, in fp64) and both are compared with the same bar as
the small parity tests: top-K sets equal outside the near-tie band, ascending
ids, attention within 2e-3 max-abs / 1e-3 mean-abs, lse within 1e-4.
"""

import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
from devutil import _log, compare_workload, run_gpu, slice_queries, slice_requests  # noqa: E402
from synth import make_decode_workload, make_prefill_workload  # noqa: E402

pytestmark = pytest.mark.gpu


def _slice_res(res, reqs=None, qs=None):
    out = []
    for r in res:
        d = {}
        for k, v in r.items():
            if v is None:
                d[k] = None
            elif reqs is not None:
                d[k] = v[list(reqs)]
            else:
                d[k] = v[:, list(qs)]
        out.append(d)
    return out


def _check_requests(name, reqs):
    _log(f"{name}: generating")
    wl = make_decode_workload(name)
    _log(f"{name}: GPU, {wl.batch} requests x {len(wl.layers)} layers")
    res_g = run_gpu(wl)
    sub = slice_requests(wl, reqs)
    _log(f"{name}: oracle on requests {list(reqs)}")
    res_o = oracle.run_workload(sub, want_scores=True)
    compare_workload(sub, _slice_res(res_g, reqs=reqs), res_o, f"{name} req {list(reqs)}")


def test_full_size_b32_128k():
    """32 requests x 131072 tokens, [Full, Reuse x5], top-2048."""
    _check_requests("b32_128k_full_reuse5", [0, 31])


def test_full_size_b8_1m():
    """8 requests x 1,048,576 tokens, [Full, Reindex (pool 16384), Reuse x4], top-2048."""
    _check_requests("b8_1m_full_reindex_reuse4", [0, 7])


def test_full_size_spec6_1m():
    """8 requests x 1,048,576 tokens with 6 query rows each (5 drafts + 1 of a
    speculative step): per-query positions, block-causal visibility among the
    newest entries, causal windows, [Full, Reindex, Reuse x4]."""
    _check_requests("b8_1m_spec6", [2])


def test_full_size_ragged_paged():
    """64 ragged requests (log-uniform 4K..1M tokens) in shuffled 64-entry pages, 20 layers."""
    name = "ragged64_paged_20layer"
    _log(f"{name}: generating")
    wl = make_decode_workload(name)
    n = wl.caches[0].n_entries
    reqs = [int(np.argmin(n)), int(np.argmax(n))]
    _log(f"{name}: GPU, {wl.batch} requests x {len(wl.layers)} layers, entries {int(n.min())}..{int(n.max())}")
    res_g = run_gpu(wl)
    sub = slice_requests(wl, reqs)
    _log(f"{name}: oracle on requests {reqs}")
    res_o = oracle.run_workload(sub, want_scores=True)
    compare_workload(sub, _slice_res(res_g, reqs=reqs), res_o, f"{name} req {reqs}")


def test_full_size_prefill_chunk():
    """4096 query tokens at positions 126976..131071 of a 131072-token context:
    block-causal scoring of 32768 entries, per-query top-2048, causal window.
    The oracle recomputes 64 query rows spread evenly over the chunk (first and
    last included); the fused scoring + top-K kernel's selection is compared
    bit for bit with the materialised path (prefill scoring kernel, then
    csa2_topk) on every one of the 4096 rows."""
    import compressed_sparse_attention_06_amd as csa2
    from devutil import dev_cache, t

    _log("prefill: generating")
    wl = make_prefill_workload()
    _log(f"prefill: GPU, {wl.nq} query rows")
    res_g = run_gpu(wl)
    L, c = wl.layers[0], wl.caches[0]
    _log("prefill: materialised scores + csa2_topk on all rows")
    sc = csa2.index_score(dev_cache(c), t(L.qix_codes), t(L.qix_scales), t(L.w), q_pos=t(wl.q_pos))
    ref = csa2.topk(sc, wl.k).cpu().numpy()
    del sc
    g = res_g[0]["idx"]
    assert (g == ref).all(), f"fused and materialised selections differ in {int((g != ref).any(axis=-1).sum())} rows"
    qs = sorted(set(int(round(x)) for x in np.linspace(0, wl.nq - 1, 64)))
    assert len(qs) == 64
    sub = slice_queries(wl, qs)
    _log(f"prefill: oracle on {len(qs)} query rows")
    res_o = oracle.run_workload(sub, want_scores=True)
    compare_workload(sub, _slice_res(res_g, qs=qs), res_o, f"prefill {len(qs)} rows")
