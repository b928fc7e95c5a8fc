"""HIP path vs the CPU oracle (GPU required).

Tolerances (the bars every GPU parity test applies):
 * dequantised values: bit-exact (fp16 of the FP4 path, fp32 of E4M3);
 * index scores: |gpu - oracle| <= 1e-6 |oracle| + 1e-6 max|row| (the second
   term covers a head sum that cancels: fp32 rounding scales with the terms,
   not with the result);
 * top-K id sets: equal after dropping ids whose oracle score lies within
   1e-5 (relative) of the oracle's K-th score; exact when scores are exact;
 * attention, given the oracle's indices: out max-abs <= 2e-3, mean-abs <=
   1e-3, lse abs <= 1e-4 against fp64.
"""

import math

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import compressed_sparse_attention_06_amd as csa2  # noqa: E402
import oracle  # noqa: E402
from devutil import (SCORE_RTOL, DevWorkload, assert_attention_close, compare_workload,  # noqa: E402
                     assert_selection_matches, dev_cache, dev_window, run_gpu, t)
from helpers import hand_window  # noqa: E402
from synth import make_small_decode  # noqa: E402

TAU = 1.0 / math.sqrt(512.0)


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.lib()


@pytest.fixture(params=["seg", "pair"])
def attend_kernel(request):
    """The attention tests run once per attention kernel (the eight-wave and
    the paired-wave form; by default the library picks one by work size)."""
    csa2.set_attend_kernel(request.param)
    yield request.param
    csa2.set_attend_kernel("auto")


def _log(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------ dequantisation

def test_dequant_fp4_bit_exact():
    _log("dequant fp4: 16 codes x 256 scales")
    nib = np.tile(np.arange(16, dtype=np.uint8), (256, 2))  # 32 channels per row
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 2, axis=1)
    g = csa2.dequant_fp4(t(codes), t(scales)).cpu().numpy().astype(np.float64)
    o = oracle.dequant_fp4(codes, scales)
    nan = np.isnan(o)
    assert (np.isnan(g) == nan).all()
    assert (g[~nan] == o[~nan]).all()


def test_dequant_e4m3_bit_exact():
    b = np.arange(256, dtype=np.uint8)
    g = csa2.dequant_e4m3(t(b)).cpu().numpy().astype(np.float64)
    o = oracle.dequant_e4m3(b[None, :])[0]
    nan = np.isnan(o)
    assert (np.isnan(g) == nan).all()
    assert (g[~nan] == o[~nan]).all()
    assert (np.signbit(g[~nan]) == np.signbit(o[~nan])).all()


# ------------------------------------------------------------------ index scores

def _check_scores(g, o, what):
    g = np.asarray(g, np.float64)
    masked = np.isneginf(o)
    assert (np.isneginf(g) == masked).all(), f"{what}: masked columns differ"
    o0, g0 = np.where(masked, 0, o), np.where(masked, 0, g)  # no inf - inf
    rowmax = np.abs(o0).max(axis=-1, keepdims=True)
    tol = SCORE_RTOL * np.abs(o0) + SCORE_RTOL * rowmax
    d = np.abs(g0 - o0)
    assert (d <= tol).all(), f"{what}: score error {d.max():.3e}"


SCORE_CASES = [
    dict(contexts=[8192], page_size=64, shuffle=False),                 # 2048 entries, 1 row
    dict(contexts=[4 * 777 + 1, 1000, 64, 8], page_size=16, shuffle=True),  # ragged tails
    dict(contexts=[4 * 5000], page_size=128, shuffle=True, nq=3),        # several query rows
]


@pytest.mark.parametrize("case", SCORE_CASES, ids=["tiny", "ragged_paged", "multi_query"])
def test_index_score_full(case):
    _log(f"index_score full {case}")
    wl = make_small_decode(layers="F", k=16, **case)
    L, c = wl.layers[0], wl.caches[0]
    g = csa2.index_score(dev_cache(c), t(L.qix_codes), t(L.qix_scales), t(L.w)).cpu().numpy()
    o = oracle.index_score(c, L.qix_codes, L.qix_scales, L.w)
    _check_scores(g, o, "full")


@pytest.mark.parametrize("nq", [2, 3, 6, 8])
def test_index_score_rows_kernels_agree(nq):
    """Several query rows per request (the kernel that reads each key once
    for all of them) give, bit for bit, what one row at a time gives: both
    multiply the same FP4 codes on the matrix cores and apply scales, ReLU,
    weights and the head sum in the same fp32 order."""
    wl = make_small_decode([4 * 6000, 4 * 1500], layers="F", k=16, nq=nq, page_size=64, shuffle=True)
    L, c = wl.layers[0], wl.caches[0]
    dc = dev_cache(c)
    g = csa2.index_score(dc, t(L.qix_codes), t(L.qix_scales), t(L.w)).cpu().numpy()
    for q in range(nq):
        one = csa2.index_score(dc, t(L.qix_codes[:, q:q + 1]), t(L.qix_scales[:, q:q + 1]),
                               t(L.w[:, q:q + 1])).cpu().numpy()
        assert np.array_equal(g[:, q:q + 1].view(np.uint32), one.view(np.uint32)), f"row {q} of {nq}"


def test_index_score_histogram():
    """The optional histogram counts each finite score's top 12 order-key bits."""
    wl = make_small_decode([4 * 9000, 4 * 100], layers="F", k=16, page_size=64, shuffle=True)
    L, c = wl.layers[0], wl.caches[0]
    hist = torch.zeros(2, 1, 4096, dtype=torch.int32, device="cuda")
    g = csa2.index_score(dev_cache(c), t(L.qix_codes), t(L.qix_scales), t(L.w), hist=hist).cpu().numpy()
    h = hist.cpu().numpy()
    # expected from the oracle's scores rounded to fp32 (the key is defined on fp32 values)
    o = oracle.index_score(c, L.qix_codes, L.qix_scales, L.w).astype(np.float32)
    for b in range(2):
        v = o[b, 0][np.isfinite(o[b, 0])]
        u = v.view(np.uint32).copy()
        u[u == 0x80000000] = 0
        key = np.where(u & 0x80000000, ~u, u | 0x80000000).astype(np.uint32)
        ref = np.bincount(key >> 20, minlength=4096)
        # scores within fp32 rounding of a bin edge may land in the neighbouring bin
        assert np.abs(h[b, 0] - ref).sum() <= 2 * max(1, int(1e-4 * len(v)))
        assert h[b, 0].sum() == len(v) == np.isfinite(g[b, 0]).sum()


def test_index_score_causal_and_candidates():
    _log("index_score q_pos + candidates")
    wl = make_small_decode([4 * 3000], layers="F", k=16, nq=6, prefill=True, page_size=32, shuffle=True)
    L, c = wl.layers[0], wl.caches[0]
    qp = np.array([[3, 4, 7, 100, 8000, 11999]], np.int32)
    g = csa2.index_score(dev_cache(c), t(L.qix_codes), t(L.qix_scales), t(L.w), q_pos=t(qp)).cpu().numpy()
    o = oracle.index_score(c, L.qix_codes, L.qix_scales, L.w, q_pos=qp)
    _check_scores(g, o, "causal")
    rng = np.random.default_rng(5)
    cand = rng.integers(-5, 3100, size=(1, 6, 777)).astype(np.int32)
    g = csa2.index_score(dev_cache(c), t(L.qix_codes), t(L.qix_scales), t(L.w), q_pos=t(qp),
                         cand=t(cand)).cpu().numpy()
    o = oracle.index_score(c, L.qix_codes, L.qix_scales, L.w, q_pos=qp, cand=cand)
    _check_scores(g, o, "candidates")


@pytest.mark.parametrize("page_size", [16, 64])
def test_index_score_prefill_chunk(page_size):
    """Many queries per request (the matrix-core contraction path): 2 requests x 130
    queries at ragged positions, block-causal, with the score histogram."""
    _log(f"index_score prefill chunk page {page_size}")
    wl = make_small_decode([4 * 2500, 4 * 700], layers="F", k=16, nq=130, prefill=True,
                           page_size=page_size, shuffle=True)
    L, c = wl.layers[0], wl.caches[0]
    rng = np.random.default_rng(page_size)
    qp = np.stack([np.sort(rng.integers(0, 4 * 2500 + 40, size=130)),
                   np.sort(rng.integers(0, 4 * 700 + 40, size=130))]).astype(np.int32)
    qp[0, :3] = [0, 2, 3]  # nothing, nothing, entry 0 visible
    hist = torch.zeros(2, 130, 4096, dtype=torch.int32, device="cuda")
    g = csa2.index_score(dev_cache(c), t(L.qix_codes), t(L.qix_scales), t(L.w), q_pos=t(qp),
                         hist=hist).cpu().numpy()
    o = oracle.index_score(c, L.qix_codes, L.qix_scales, L.w, q_pos=qp)
    _check_scores(g, o, "prefill chunk")
    h = hist.cpu().numpy()
    fin = np.isfinite(g)
    assert (h.sum(axis=-1) == fin.sum(axis=-1)).all()
    assert h[0, 0].sum() == 0 and h[0, 2].sum() == 1


# ------------------------------------------------------------------ top-K

@pytest.mark.parametrize("n,k", [(100, 7), (2048 + 37, 256), (16384, 2048), (16385, 2048),
                                 (70000, 4096), (300000, 2048), (50, 100)])
def test_topk_exact_ties(n, k):
    """Integer scores (exact in fp32, many ties): the lowest-id rule decides, exact match."""
    _log(f"topk ties n={n} k={k}")
    rng = np.random.default_rng(n + k)
    s = rng.integers(0, 9, size=(2, 1, n)).astype(np.float64)
    s[rng.random(s.shape) < 0.1] = -np.inf
    s[1, 0, :] = 3.0  # one row where every score ties
    g = csa2.topk(t(s.astype(np.float32)), k).cpu().numpy()
    o = oracle.topk(s, k)
    assert (g == o).all()


@pytest.mark.parametrize("n,k", [(5000, 2048), (262144, 4096), (40000, 1), (524288, 4096)])
def test_topk_random_scores(n, k):
    _log(f"topk random n={n} k={k}")
    rng = np.random.default_rng(7)
    s = rng.standard_normal((3, 1, n)) * 10
    s32 = s.astype(np.float32)
    g = csa2.topk(t(s32), k).cpu().numpy()
    o = oracle.topk(s32.astype(np.float64), k)  # same fp32 values: exact ties only
    assert (g == o).all()


@pytest.mark.parametrize("dist", ["ties", "normal", "outliers"])
def test_topk_many_rows_one_workgroup_each(dist):
    """40 rows of 4097..16384 columns (the one-workgroup-per-row path): ties,
    plain normal scores, and a few large outliers that squeeze most keys into
    a narrow part of the row's range; -inf holes and a short last row."""
    _log(f"topk many rows {dist}")
    rng = np.random.default_rng({"ties": 11, "normal": 12, "outliers": 13}[dist])
    rows, n, k = 40, 12000, 2048
    if dist == "ties":
        s = rng.integers(0, 40, size=(rows, 1, n)).astype(np.float64)
    elif dist == "normal":
        s = rng.standard_normal((rows, 1, n))
    else:
        s = np.abs(rng.standard_normal((rows, 1, n))) + 1.0
        s[:, :, :5] = 1e6
    s[rng.random(s.shape) < 0.05] = -np.inf
    s[-1, 0, 3000:] = -np.inf  # fewer finite scores than k
    s32 = s.astype(np.float32)
    g = csa2.topk(t(s32), k).cpu().numpy()
    o = oracle.topk(s32.astype(np.float64), k)
    assert (g == o).all()
    # a candidate map in ascending order keeps ascending ids
    cand = np.sort(np.stack([rng.choice(10 ** 6, size=n, replace=False) for _ in range(rows)]), axis=1)
    cand = cand[:, None, :].astype(np.int32)
    g = csa2.topk(t(s32), k, cand=t(cand)).cpu().numpy()
    o = oracle.topk(s32.astype(np.float64), k, cand=cand)
    assert (g == o).all()
    # a permuted map: keys tied at the threshold are settled by the mapped id,
    # not by the column (the "ties" rows hold ~300 keys per value)
    cand = np.stack([rng.choice(10 ** 6, size=n, replace=False) for _ in range(rows)])[:, None, :]
    cand = cand.astype(np.int32)
    g = csa2.topk(t(s32), k, cand=t(cand)).cpu().numpy()
    o = oracle.topk(s32.astype(np.float64), k, cand=cand)
    assert (g == o).all(), f"{int((g != o).any(axis=-1).sum())} rows differ"


def test_reindex_shuffled_pool_many_rows():
    """A Reindex layer over 40 requests whose pools (5000 of each request's 6000
    entries, in random order, with -1 pads and ids past the entry count) are
    not ascending, so selection runs one workgroup per row with an id map; 70%
    of the indexer keys are zero, so about half of each selection is a tie at
    score 0 settled by entry id. Selected sets against the oracle (exact: the
    tied scores are exactly 0 on both sides; elsewhere outside the 1e-5 band),
    attention against the oracle's attention over the GPU's selection."""
    _log("reindex, shuffled pool, 40 rows")
    B, P, K = 40, 5000, 2048
    wl = make_small_decode([4 * 6000] * B, layers="FR", k=K, pool=P, page_size=64, shuffle=True)
    c, R = wl.caches[0], wl.layers[1]
    rng = np.random.default_rng(21)
    kill = rng.random(c.ix_codes.shape[0] * c.ix_codes.shape[1]) < 0.7
    c.ix_codes.reshape(-1, c.ix_codes.shape[-1])[kill] = 0
    pool = np.full((B, 1, P), -1, np.int32)
    for b in range(B):
        ids = rng.choice(6000, size=P - 40, replace=False)
        row = np.concatenate([ids, [6000, 6001, 10 ** 6, -3], np.full(36, -1)]).astype(np.int32)
        rng.shuffle(row)
        pool[b, 0] = row
    call = csa2.LayerCall("R", dev_cache(c), dev_window(R.win), t(R.q), K, pool=P, qix_codes=t(R.qix_codes),
                          qix_scales=t(R.qix_scales), w=t(R.w), idx_in=t(pool))
    call()
    torch.cuda.synchronize()
    g_idx = call.idx_out.cpu().numpy()
    o = oracle.layer_step("R", c, R.win, R.q, R.qix_codes, R.qix_scales, R.w, k=K, pool=P, idx_in=pool,
                          want_scores=True)
    n_exact = 0
    for b in range(B):
        id_to_col = {int(e): j for j, e in enumerate(pool[b, 0]) if e >= 0}
        n_exact += assert_selection_matches(o["scores"][b, 0], o["idx"][b, 0], g_idx[b, 0],
                                            id_to_col=id_to_col, what=f"reindex b{b}")
    _log(f"{n_exact}/{B} selections identical")
    o_out, o_lse, _ = oracle.sparse_attend(c, g_idx, R.q, R.win, sm_scale=TAU)
    assert_attention_close(call.out.cpu().numpy(), call.lse.cpu().numpy(), o_out, o_lse, "reindex attend")


def test_index_topk_many_ragged_rows():
    """Rows of very different lengths in grids sized by the longest: 128 rows
    of 1,000..40,960 entries (capacity 40,960), so most of the scoring,
    compaction and final workgroups hold no column of their row, and some
    rows are shorter than k. Every row's top-2048 and pool of 4096 against
    the oracle's scores: sets equal outside the near-tie band, ascending, -1
    past the visible entries."""
    rng = np.random.default_rng(11)
    ent = np.concatenate([[40960], rng.integers(1000, 40960, size=127)])
    _log(f"many ragged rows: {len(ent)} rows, {int(ent.sum())} entries")
    wl = make_small_decode(contexts=list(4 * ent), layers="F", k=2048, pool=4096, page_size=64, shuffle=True)
    c, L = wl.caches[0], wl.layers[0]
    g_idx, g_pool = csa2.index_topk(dev_cache(c), t(L.qix_codes), t(L.qix_scales), t(L.w), 2048, pool=4096)
    g_idx, g_pool = g_idx.cpu().numpy(), g_pool.cpu().numpy()
    o_sc = oracle.index_score(c, L.qix_codes, L.qix_scales, L.w)
    o_idx, o_pool = oracle.topk(o_sc, 2048), oracle.topk(o_sc, 4096)
    n_exact = 0
    for b in range(len(ent)):
        for g, o, tag in ((g_idx, o_idx, "top-k"), (g_pool, o_pool, "pool")):
            row = g[b, 0]
            v = row[row >= 0]
            assert (np.diff(v) > 0).all() and (row[len(v):] == -1).all(), f"row {b} {tag}: order or pads"
            n_exact += assert_selection_matches(o_sc[b, 0], o[b, 0], row, what=f"row {b} {tag}")
    _log(f"{n_exact}/{2 * len(ent)} selections identical")


def test_topk_candidate_map():
    rng = np.random.default_rng(9)
    n, k = 20000, 300
    s = np.round(rng.standard_normal((2, 1, n)) * 4)
    cand = np.stack([rng.permutation(10 ** 6)[:n] for _ in range(2)])[:, None, :].astype(np.int32)
    g = csa2.topk(t(s.astype(np.float32)), k, cand=t(cand)).cpu().numpy()
    o = oracle.topk(s, k, cand=cand)
    assert (g == o).all()


# ------------------------------------------------------------------ attention

ATT_CASES = [
    dict(contexts=[8192], k=256, page_size=64),
    dict(contexts=[4 * 700, 4 * 33, 4 * 1500 + 3], k=512, page_size=16, shuffle=True, row_scale=True),
    dict(contexts=[4 * 100, 40], k=300, page_size=8),   # N < K: pads
]


@pytest.mark.parametrize("case", ATT_CASES, ids=["tiny", "ragged_rowscale", "short"])
def test_sparse_attend_given_oracle_indices(case, attend_kernel):
    _log(f"sparse_attend {case}")
    wl = make_small_decode(layers="F", **case)
    L, c = wl.layers[0], wl.caches[0]
    r = oracle.layer_step("F", c, L.win, L.q, L.qix_codes, L.qix_scales, L.w, k=wl.k)
    g_out, g_lse = csa2.sparse_attend(dev_cache(c), t(r["idx"]), t(L.q), dev_window(L.win))
    torch.cuda.synchronize()
    assert_attention_close(g_out.cpu().numpy(), g_lse.cpu().numpy(), r["out"], r["lse"], "attend")


def test_sparse_attend_edge_cases(attend_kernel):
    _log("sparse_attend edges")
    wl = make_small_decode([4 * 64, 4 * 64], layers="F", k=8)
    c, L = wl.caches[0], wl.layers[0]
    # request 0: nothing at all (no entries, empty window) -> out 0, lse -inf
    # request 1: ids out of range / padding mixed with valid ones
    idx = np.array([[[-1] * 8], [[3, 99999, -1, 5, 64, 63, -7, 0]]], np.int32)
    win = hand_window(L.win.codes, length=[0, 17])
    g_out, g_lse = csa2.sparse_attend(dev_cache(c), t(idx), t(L.q), dev_window(win))
    o_out, o_lse, _ = oracle.sparse_attend(c, idx, L.q, win, sm_scale=TAU)
    assert_attention_close(g_out.cpu().numpy(), g_lse.cpu().numpy(), o_out, o_lse, "edges")
    # no window at all
    g_out, g_lse = csa2.sparse_attend(dev_cache(c), t(idx), t(L.q), None)
    o_out, o_lse, _ = oracle.sparse_attend(c, idx, L.q, None, sm_scale=TAU)
    assert_attention_close(g_out.cpu().numpy(), g_lse.cpu().numpy(), o_out, o_lse, "no window")


def test_sparse_attend_poisoned_unused_bytes(attend_kernel):
    """Bytes that no position of the attention set may use are NaN patterns
    (0xFF: an E4M3 NaN as a scale or window byte): a physical page no request
    maps (page 0, which a position without an entry addresses), the slots past
    each request's entry count, the window rows past each request's length and
    their row scales. Positions without a row (-1 pads, ids past the entry
    count, ids past the page table, positions k..k16-1) must still give the
    oracle's output."""
    _log("sparse_attend, poisoned unused bytes")
    wl = make_small_decode([4 * 700, 4 * 33, 4 * 5, 4 * 1500 + 3], layers="F", k=300, page_size=16,
                           shuffle=True, row_scale=True)
    c0, L = wl.caches[0], wl.layers[0]
    r = oracle.layer_step("F", c0, L.win, L.q, L.qix_codes, L.qix_scales, L.w, k=wl.k)
    # one extra physical page in front, mapped by no request
    bt = np.where(c0.block_table >= 0, c0.block_table + 1, -1).astype(np.int32)
    pad = lambda a: np.concatenate([np.full((1,) + a.shape[1:], 0xFF, np.uint8), a])  # noqa: E731
    c = type(c0)(kv_codes=pad(c0.kv_codes), kv_scales=pad(c0.kv_scales), ix_codes=pad(c0.ix_codes),
                 ix_scales=pad(c0.ix_scales), block_table=bt, n_entries=c0.n_entries, page_size=c0.page_size)
    ps = c.page_size
    for b, n in enumerate(c.n_entries):
        for s_ in range(int(n), (int(n) + ps - 1) // ps * ps):  # tail slots of the last page
            p = bt[b, s_ // ps]
            c.kv_codes[p, s_ % ps] = 0xFF
            c.kv_scales[p, s_ % ps] = 0xFF
    win = L.win
    for b, n in enumerate(win.length):
        win.codes[b, int(n):] = 0xFF
        win.row_scale[b, int(n):] = np.nan
    idx = r["idx"].copy()
    for b, n in enumerate(c.n_entries):  # pads of the short requests -> ids with no row
        row = idx[b, 0]
        free = np.nonzero(row < 0)[0]
        bad = [int(n), int(n) + 1, 10 ** 7, -9]
        for j, v in zip(free, bad):
            row[j] = v
    g_out, g_lse = csa2.sparse_attend(dev_cache(c), t(idx), t(L.q), dev_window(win))
    torch.cuda.synchronize()
    g_out, g_lse = g_out.cpu().numpy(), g_lse.cpu().numpy()
    assert np.isfinite(g_out).all(), "a masked position leaked a NaN"
    o_out, o_lse, _ = oracle.sparse_attend(c, idx, L.q, win, sm_scale=TAU)
    assert_attention_close(g_out, g_lse, o_out, o_lse, "poisoned")


# How the attention work is cut: each row's set (k entries, then the window from
# k rounded up to 16) in units of 128 positions, shared over at most 256
# workgroups. These cases cover k below, at and off a multiple of 16, sets of
# one unit, rows cut between workgroups at many offsets (T > 256 units, with
# 2..20 units per workgroup), workgroups that run through several rows with
# odd and even unit counts per row, several query rows per request with their
# own causal windows, no window, and rows cut into more partials (33) than
# the merge loads in one batch.
UNIT_CASES = [
    dict(contexts=[4 * 300, 4 * 40], k=1, nq=1, win=True),                       # U = 2
    dict(contexts=[4 * 300], k=13, nq=1, win=False),                              # one unit, tail lanes empty
    dict(contexts=[4 * 500, 4 * 200, 4 * 900], k=300, nq=1, win=True),            # k16 = 304
    dict(contexts=[4 * 700] * 20, k=256, nq=3, win=True, prefill=True),           # 60 rows x 3 units
    dict(contexts=[4 * 2200] * 30, k=2048, nq=1, win=True),                       # 30 x 17 units over 256
    dict(contexts=[4 * 3000] * 6, k=2048, nq=50, win=True, prefill=True),         # 300 rows x 17 units
    dict(contexts=[4 * 5000], k=4096, nq=1, win=True),                            # 33 partials of one row:
    dict(contexts=[4 * 5000, 4 * 4500, 4 * 6000], k=4096, nq=1, win=True),        # the merge takes two batches
    dict(contexts=[4 * 2200] * 16, k=2048, nq=1, win=True),                       # 9 workgroups per row
    dict(contexts=[4 * 2200] * 40, k=2048, nq=1, win=True),                       # 6 per row, 240 in all
    dict(contexts=[4 * 1500] * 6, k=512, nq=60, win=False, prefill=True),         # 360 rows x 4 units
    dict(contexts=[4 * 1500] * 4, k=640, nq=40, win=True, prefill=True),          # 160 rows x 6 units
]


@pytest.mark.parametrize("case", UNIT_CASES, ids=["k1", "k13_nowin", "k300", "nq3_prefill", "b30_k2048",
                                                 "nq50_k2048", "k4096_b1", "k4096_b3", "b16_k2048",
                                                 "b40_k2048", "nq60_k512_nowin", "nq40_k640"])
def test_sparse_attend_unit_geometry(case, attend_kernel):
    _log(f"sparse_attend geometry {case}")
    wl = make_small_decode(contexts=case["contexts"], layers="F", k=case["k"], nq=case["nq"],
                           prefill=case.get("prefill", False), page_size=32, shuffle=True, row_scale=True)
    c, L = wl.caches[0], wl.layers[0]
    rng = np.random.default_rng(len(case["contexts"]) * 7 + case["k"])
    B, nq, k = L.q.shape[0], L.q.shape[1], wl.k
    # ids: random visible entries, ascending, a few pads and out-of-range ids
    idx = np.full((B, nq, k), -1, np.int32)
    for b in range(B):
        n = int(c.n_entries[b])
        for q in range(nq):
            lim = n if wl.q_pos is None else min(n, (int(wl.q_pos[b, q]) + 1) // 4)
            m = min(k, lim)
            if m > 0:
                idx[b, q, :m] = np.sort(rng.choice(lim, size=m, replace=False))
            if k > 4 and m == k:
                idx[b, q, -1] = n + 5  # out of range: must be ignored
    win = L.win if case["win"] else None
    qp = wl.q_pos
    g_out, g_lse = csa2.sparse_attend(dev_cache(c), t(idx), t(L.q), dev_window(win), q_pos=t(qp))
    o_out, o_lse, _ = oracle.sparse_attend(c, idx, L.q, win, q_pos=qp, sm_scale=TAU)
    assert_attention_close(g_out.cpu().numpy(), g_lse.cpu().numpy(), o_out, o_lse, f"geometry {case}")


def test_sparse_attend_large_logits(attend_kernel):
    """Rows of 2688 and a large query: the running max keeps the softmax finite."""
    wl = make_small_decode([4 * 64], layers="F", k=4)
    c = wl.caches[0]
    c.kv_codes[...] = 0x77  # every channel 6.0
    c.kv_scales[...] = 0x7E  # x 448
    q = np.full((1, 1, 16, 512), 3.0, np.float32)
    idx = np.array([[[0, 1, 2, -1]]], np.int32)
    win = hand_window(np.zeros((1, 1, 512), np.uint8), length=[0])
    g_out, g_lse = csa2.sparse_attend(dev_cache(c), t(idx), t(q), dev_window(win))
    o_out, o_lse, _ = oracle.sparse_attend(c, idx, q, win, sm_scale=TAU)
    g_out, g_lse = g_out.cpu().numpy(), g_lse.cpu().numpy()
    assert np.isfinite(g_out).all() and np.isfinite(g_lse).all()
    assert np.abs(g_out - o_out).max() <= 2e-3 * 2688
    assert np.abs(g_lse - o_lse).max() / abs(o_lse).max() < 1e-6


def test_sparse_attend_prefill_windows(attend_kernel):
    _log("sparse_attend prefill windows")
    wl = make_small_decode([4 * 900], layers="F", k=64, nq=7, prefill=True, page_size=32)
    L, c = wl.layers[0], wl.caches[0]
    r = oracle.layer_step("F", c, L.win, L.q, L.qix_codes, L.qix_scales, L.w, q_pos=wl.q_pos, k=64)
    g_out, g_lse = csa2.sparse_attend(dev_cache(c), t(r["idx"]), t(L.q), dev_window(L.win), q_pos=t(wl.q_pos))
    torch.cuda.synchronize()
    assert_attention_close(g_out.cpu().numpy(), g_lse.cpu().numpy(), r["out"], r["lse"], "prefill")


# ------------------------------------------------------------------ layer steps

LAYER_CASES = [
    dict(contexts=[8192], layers="F", k=256, pool=0),
    dict(contexts=[4 * 3000, 4 * 1200], layers="FUU", k=128, pool=0, page_size=32, shuffle=True),
    dict(contexts=[4 * 20000, 4 * 9000, 4 * 600], layers="FRUU", k=256, pool=2048, page_size=64, shuffle=True),
    dict(contexts=[4 * 20000, 4 * 300], layers="FRU", k=512, pool=1024, page_size=64, row_scale=True),
    dict(contexts=[4 * 40], layers="FRU", k=64, pool=128, page_size=8),  # N < K < pool
    # Reindex over a pool long enough for the chunked selection; request 1 has
    # fewer entries than the pool, so its pool ends in -1 pads
    dict(contexts=[4 * 60000, 4 * 9000], layers="FRU", k=1024, pool=12000, page_size=64, shuffle=True),
    # 520 query rows of a prefill chunk: attention runs one workgroup per query row
    dict(contexts=[4 * 3000], layers="FRU", k=256, pool=1024, nq=520, prefill=True, page_size=32),
    # the largest k and pool the library takes (4096, 65536): 33 attention units per row
    dict(contexts=[4 * 70000, 4 * 20000], layers="FRU", k=4096, pool=65536, page_size=64, shuffle=True),
    # the page-size extremes: every entry its own page; whole requests in one or a few pages
    dict(contexts=[4 * 3000, 4 * 1000], layers="FRU", k=256, pool=1024, page_size=1, shuffle=True),
    dict(contexts=[4 * 20000, 4 * 5000], layers="FRU", k=512, pool=2048, page_size=4096, shuffle=True),
    # an empty request (no entries, no window rows) beside a full one and one shorter than k
    dict(contexts=[4 * 3000, 0, 4 * 10], layers="FRU", k=64, pool=256, page_size=16, shuffle=True),
]


@pytest.mark.parametrize("case", LAYER_CASES, ids=["tiny_full", "full_reuse", "full_reindex_reuse",
                                                   "rowscale", "short_ctx", "long_pool", "prefill_rows",
                                                   "max_k_pool", "page_1", "page_4096", "empty_request"])
def test_layer_step_chain(case, attend_kernel):
    _log(f"layer chain {case}")
    wl = make_small_decode(**case)
    res_g = run_gpu(wl)
    res_o = oracle.run_workload(wl, want_scores=True)
    compare_workload(wl, res_g, res_o, "chain")


def test_reuse_equals_full_given_same_indices(attend_kernel):
    wl = make_small_decode([4 * 5000], layers="FU", k=256, page_size=64)
    dw = DevWorkload(wl)
    calls = dw.calls()
    calls[0]()
    F = dw.layers[0]
    u = csa2.LayerCall("U", dw.caches[0], F["win"], F["q"], wl.k, idx_in=calls[0].idx_out)
    u()
    torch.cuda.synchronize()
    assert torch.equal(u.out, calls[0].out) and torch.equal(u.lse, calls[0].lse)


def test_layer_step_repeatable():
    """Same inputs, same outputs (selection is deterministic; attention sums in a fixed order)."""
    wl = make_small_decode([4 * 30000, 4 * 7000], layers="FRU", k=512, pool=2048, shuffle=True)
    a = run_gpu(wl)
    b = run_gpu(wl)
    for x, y in zip(a, b):
        if x["idx"] is not None:
            assert (x["idx"] == y["idx"]).all()
        assert (x["out"] == y["out"]).all() and (x["lse"] == y["lse"]).all()


def test_graph_capture_replays_match_eager(attend_kernel):
    """A captured Full/Reindex/Reuse chain replays to the eager result every time."""
    _log("graph capture")
    wl = make_small_decode([4 * 30000, 4 * 7000], layers="FRUU", k=512, pool=2048, shuffle=True)
    dw = DevWorkload(wl)
    calls = dw.calls()
    for c in calls:
        c()
    torch.cuda.synchronize()
    ref = [(c.out.clone(), c.lse.clone(), None if c.idx_out is None else c.idx_out.clone()) for c in calls]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for c in calls:
            c()
    for rep in range(4):
        for c in calls:  # scribble over the outputs, then replay
            c.out.fill_(float("nan"))
            c.lse.zero_()
            if c.idx_out is not None:
                c.idx_out.fill_(-5)
        junk = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work in between
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for c, (o, l, i) in zip(calls, ref):
            assert torch.equal(c.out, o) and torch.equal(c.lse, l), f"replay {rep}"
            if i is not None:
                assert torch.equal(c.idx_out, i), f"replay {rep}"


def test_full_size_tiny_config():
    """The tiny benchmark workload (1 request, 8192-token context, top-256) at full size."""
    from synth import make_decode_workload
    wl = make_decode_workload("tiny_b1_8k_full")
    res_g = run_gpu(wl)
    res_o = oracle.run_workload(wl, want_scores=True)
    compare_workload(wl, res_g, res_o, "tiny config")
