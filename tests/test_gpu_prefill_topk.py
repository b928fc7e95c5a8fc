"""Prefill chunk with the indexer scoring fused into the per-query top-K (no
score matrix in memory): the selection and the attention that follows against
the oracle, and the selection bit for bit against the materialised path (the
prefill scoring kernel, then csa2_topk) on the same inputs.

The fused kernel runs for Full layers with no pool over at most 32768 entries
when a call has at least 1024 query rows and 64 per request; every case below
checks first that the workspace size says so (no score region), and the
host-side tests check the converse for shapes outside those limits."""

import os
import sys

import numpy as np
import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import compressed_sparse_attention_06_amd as csa2  # noqa: E402
import oracle  # noqa: E402
from devutil import _log, compare_workload, dev_cache, run_gpu, t  # noqa: E402
from synth import make_small_decode  # noqa: E402

pytestmark = pytest.mark.gpu

CASES = [
    # 65 workgroups of 16 rows, shuffled pages
    dict(contexts=[4 * 3000], nq=1040, k=256, page_size=32, shuffle=True),
    # positions 100..1199: the early rows see fewer than k entries (all taken)
    dict(contexts=[4 * 300], nq=1100, k=256, page_size=64),
    # 2500 pages of 8 entries: page ids read from the block table, not LDS
    dict(contexts=[4 * 20000], nq=1024, k=512, page_size=8, shuffle=True),
    # two requests, 520 rows each (the last workgroup of each holds 8 rows)
    dict(contexts=[4 * 2000, 4 * 2600], nq=520, k=128, page_size=16, shuffle=True),
]


def _is_fused(wl):
    """The Full layer's workspace is the attention's alone: no score region."""
    c = wl.caches[0]
    cap = c.block_table.shape[1] * c.page_size
    B, nq = wl.batch, wl.nq
    return csa2.workspace_bytes("F", B, nq, cap, wl.k, 0, 0) == csa2.workspace_bytes("U", B, nq, 0, wl.k, 0, 0)


def _materialised_topk(wl):
    L, c = wl.layers[0], wl.caches[0]
    sc = csa2.index_score(dev_cache(c), t(L.qix_codes), t(L.qix_scales), t(L.w), q_pos=t(wl.q_pos))
    return csa2.topk(sc, wl.k).cpu().numpy()


def _check(wl, what):
    assert _is_fused(wl), f"{what}: shape does not take the fused path"
    res_g = run_gpu(wl)
    g = res_g[0]["idx"]
    ref = _materialised_topk(wl)
    assert (g == ref).all(), f"{what}: fused and materialised selections differ in " \
                             f"{int((g != ref).any(axis=-1).sum())} rows"
    res_o = oracle.run_workload(wl, want_scores=True)
    compare_workload(wl, res_g, res_o, what)
    return g


@pytest.mark.parametrize("case", CASES, ids=["chunk_1040", "short_rows", "small_pages", "two_requests"])
def test_prefill_topk_fused(case):
    _log(f"fused prefill top-k {case}")
    wl = make_small_decode(layers="F", prefill=True, **case)
    _check(wl, "fused prefill")


def _visible(wl):
    c = wl.caches[0]
    return np.minimum(c.n_entries[:, None], (wl.q_pos.astype(np.int64) + 1) // 4)


def test_prefill_topk_fused_all_ties():
    """Every indexer key zero: every score is 0, so each query takes its lowest
    visible ids, reached through the deepest refinement (the composite's id
    part)."""
    _log("fused prefill top-k, all ties")
    wl = make_small_decode([4 * 3000], layers="F", k=300, nq=1024, prefill=True, page_size=64)
    wl.caches[0].ix_codes[:] = 0
    g = _check(wl, "all ties")
    V = _visible(wl)
    for r in range(wl.nq):
        n = min(wl.k, int(V[0, r]))
        assert (g[0, r, :n] == np.arange(n)).all() and (g[0, r, n:] == -1).all(), f"row {r}"


def test_prefill_topk_fused_few_positive():
    """95% of the keys zeroed: fewer positive scores than k, so the threshold is
    the tie at 0 and the rest of each row's k comes from its lowest-id zeros."""
    _log("fused prefill top-k, few positive scores")
    wl = make_small_decode([4 * 3000], layers="F", k=300, nq=1024, prefill=True, page_size=64,
                           shuffle=True)
    c = wl.caches[0]
    rng = np.random.default_rng(11)
    kill = rng.random(c.ix_codes.shape[0] * c.ix_codes.shape[1]) < 0.95
    c.ix_codes.reshape(-1, c.ix_codes.shape[-1])[kill] = 0
    _check(wl, "few positive")


def test_prefill_topk_fused_mixed_refinement():
    """Every third query's indexer vector zeroed: those rows score all entries
    0 and refine down to their lowest ids while the rows beside them (sharing
    LDS with them in pairs) collect after one histogram; both kinds must come
    out whole."""
    _log("fused prefill top-k, rows refining beside rows collecting")
    wl = make_small_decode([4 * 3000], layers="F", k=300, nq=1024, prefill=True, page_size=64,
                           shuffle=True)
    L = wl.layers[0]
    tied = np.arange(wl.nq) % 3 == 0
    L.qix_codes[:, tied] = 0
    g = _check(wl, "mixed refinement")
    V = _visible(wl)
    for r in np.nonzero(tied)[0]:
        n = min(wl.k, int(V[0, r]))
        assert (g[0, r, :n] == np.arange(n)).all() and (g[0, r, n:] == -1).all(), f"row {r}"
    assert ((g[0, ~tied] >= 0).sum(axis=-1) == wl.k).all()


@pytest.mark.parametrize("case", [
    dict(contexts=[4 * 20000, 4 * 9000], k=256, pool=2048, nq=1, prefill=False, page_size=64),
    dict(contexts=[4 * 3000], k=256, pool=0, nq=1040, prefill=True, page_size=32),
], ids=["decode_pool", "prefill_fused"])
def test_index_topk_matches_layer_step(case):
    """csa2_index_topk writes exactly the top-k (and pool) a Full csa2_layer_step
    selects before it attends."""
    from devutil import DevWorkload
    _log(f"index_topk vs layer_step {case}")
    wl = make_small_decode(layers="F", shuffle=True, **case)
    dw = DevWorkload(wl)
    call = dw.calls()[0]
    call()
    F = dw.layers[0]
    idx, pool = csa2.index_topk(dw.caches[0], F["qix_codes"], F["qix_scales"], F["w"], wl.k,
                                q_pos=dw.q_pos, pool=wl.pool)
    import torch
    torch.cuda.synchronize()
    assert torch.equal(idx, call.idx_out)
    if wl.pool:
        assert torch.equal(pool, call.pool_out)


def test_prefill_topk_fused_graph_replays():
    """The fused prefill layer (selection + attention) captured in a HIP graph
    replays to the eager result every time, with other work in between."""
    import torch
    from devutil import DevWorkload
    _log("fused prefill top-k, graph replays")
    wl = make_small_decode([4 * 3000], layers="F", k=256, nq=1040, prefill=True, page_size=32,
                           shuffle=True)
    dw = DevWorkload(wl)
    call = dw.calls()[0]
    call()
    torch.cuda.synchronize()
    ref = (call.out.clone(), call.lse.clone(), call.idx_out.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(3):
        call.out.fill_(float("nan"))
        call.lse.zero_()
        call.idx_out.fill_(-5)
        junk = torch.randn(1 << 20, device="cuda").sum()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(call.idx_out, ref[2]), f"replay {rep}"
        assert torch.equal(call.out, ref[0]) and torch.equal(call.lse, ref[1]), f"replay {rep}"
