"""The cache's write side on the GPU vs the oracle: FP4 row quantisation, KV
append through the page table, window ring append. Bar: bit-exact bytes (and
bit-exact fp32 row scales), also for every byte the call must leave alone.
Then the appended entries are attended and compared like any other cache."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

import compressed_sparse_attention_06_amd as csa2  # noqa: E402
import oracle  # noqa: E402
from devutil import _log, assert_attention_close, assert_selection_matches, dev_cache, dev_window, t  # noqa: E402
from synth import make_small_decode  # noqa: E402


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.lib()


def _rows(rng, n, ch):
    """Values across magnitudes, with zero groups, exact midpoints, huge and tiny values."""
    x = rng.standard_normal((n, ch)) * np.exp(rng.standard_normal((n, 1)) * 4)
    x[0, :16] = 0.0
    x[1, :] = rng.integers(-24, 25, ch) * 0.25          # E2M1 midpoints at scale 0.5 or 1
    x[2, :16] = 1e6                                      # saturating scale
    x[3, :] = rng.standard_normal(ch) * 1e-5             # subnormal E4M3 scales
    x[4, ::3] = -0.0
    v = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    x[5, :16] = 6.0 * v[40:56]                           # amax/6 on the E4M3 grid
    return x.astype(np.float32)


@pytest.mark.parametrize("ch", [64, 512])
def test_quantize_fp4_bit_exact(ch):
    _log(f"quantize_fp4 ch={ch}")
    rng = np.random.default_rng(ch)
    x = _rows(rng, 300, ch)
    gc, gs = csa2.quantize_fp4(t(x))
    oc, os_ = oracle.quantize_fp4(x)
    assert (gs.cpu().numpy() == os_).all()
    assert (gc.cpu().numpy() == oc).all()


def test_window_append_encodes_like_the_oracle():
    """E4M3 of arbitrary values (every midpoint between neighbours, past 448, tiny),
    with and without a row scale; rows not named stay as they were."""
    _log("window_append")
    rng = np.random.default_rng(2)
    B, rows, n_new = 3, 16, 2
    v = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    mids = ((v[1:] + v[:-1]) / 2).astype(np.float32)
    x = (rng.standard_normal((B, n_new, 512)) * 50).astype(np.float32)
    x[0, 0, :126] = mids
    x[0, 0, 126:252] = -mids
    x[0, 0, 252:260] = [448.0, 449.0, 464.0, 1e9, -1e9, 2 ** -10, 3 * 2 ** -10, -(2 ** -11)]
    x[1, 1, :] = 0.0
    row = np.array([[3, 15], [-1, 0], [7, 16]], np.int32)  # -1 and 16 write nothing
    for with_scale in (False, True):
        oc = np.full((B, rows, 512), 0x5A, np.uint8)
        ors = np.full((B, rows), 9.0, np.float32) if with_scale else None
        oracle.window_append(oc, ors, x, row)
        gc = t(np.full((B, rows, 512), 0x5A, np.uint8))
        grs = t(np.full((B, rows), 9.0, np.float32)) if with_scale else None
        csa2.window_append(gc, t(x), t(row), row_scale=grs)
        assert (gc.cpu().numpy() == oc).all(), with_scale
        if with_scale:
            assert (grs.cpu().numpy() == ors).all()


def test_kv_append_through_page_table():
    """New entries of several requests (pages shuffled, one page missing, negative
    entries) land where the oracle puts them; every other byte is unchanged."""
    _log("kv_append")
    rng = np.random.default_rng(3)
    B, page, max_pages, n_new = 3, 16, 6, 5
    num_pages = B * max_pages
    bt = rng.permutation(num_pages).astype(np.int32).reshape(B, max_pages)
    bt[1, 2] = -1
    kvc = rng.integers(0, 256, (num_pages, page, 256), dtype=np.uint8)
    kvs = rng.integers(0, 256, (num_pages, page, 32), dtype=np.uint8)
    ixc = rng.integers(0, 256, (num_pages, page, 32), dtype=np.uint8)
    ixs = rng.integers(0, 256, (num_pages, page, 4), dtype=np.uint8)
    entry = np.array([[0, 17, 33, 95, -1], [40, 35, 2, -3, 95], [5, 6, 7, 80, 81]], np.int32)
    kv = _rows(rng, B * n_new, 512).reshape(B, n_new, 512)
    ix = _rows(rng, B * n_new, 64).reshape(B, n_new, 64)
    o = [a.copy() for a in (kvc, kvs, ixc, ixs)]
    oracle.kv_append(*o, bt, page, kv, ix, entry)
    cache = csa2.Cache(kv_codes=t(kvc), kv_scales=t(kvs), ix_codes=t(ixc), ix_scales=t(ixs),
                       block_table=t(bt), n_entries=t(np.full(B, 96, np.int32)))
    csa2.kv_append(cache, t(kv), t(entry), ix=t(ix))
    got = [cache.kv_codes, cache.kv_scales, cache.ix_codes, cache.ix_scales]
    for name, g, want in zip(("kv_codes", "kv_scales", "ix_codes", "ix_scales"), got, o):
        assert (g.cpu().numpy() == want).all(), name
    # main KV only (no indexer key): the indexer arrays stay untouched
    o2 = [a.copy() for a in o]
    oracle.kv_append(*o2[:2], np.empty((num_pages, page, 32), np.uint8), np.empty((num_pages, page, 4), np.uint8),
                     bt, page, kv[:, ::-1].copy(), None, entry)
    csa2.kv_append(cache, t(kv[:, ::-1].copy()), t(entry))
    assert (cache.kv_codes.cpu().numpy() == o2[0]).all() and (cache.kv_scales.cpu().numpy() == o2[1]).all()
    assert (cache.ix_codes.cpu().numpy() == o[2]).all() and (cache.ix_scales.cpu().numpy() == o[3]).all()


def test_appended_entries_are_attended():
    """Append a batch of new entries and window tokens, advance the counts, and run a
    Full layer on both sides: selection and attention see the new entries."""
    _log("append then attend")
    wl = make_small_decode(contexts=[4 * 600, 4 * 900], k=256, page_size=32, layers="F", row_scale=True)
    c, L = wl.caches[0], wl.layers[0]
    rng = np.random.default_rng(4)
    B, n_new = 2, 8
    n0 = c.n_entries.copy()
    entry = (n0[:, None] + np.arange(n_new)[None, :]).astype(np.int32)
    kv = (rng.standard_normal((B, n_new, 512)) * 3).astype(np.float32)
    ix = (rng.standard_normal((B, n_new, 64)) + 2.0).astype(np.float32)  # biased up: likely selected
    cache = dev_cache(c)
    csa2.kv_append(cache, t(kv), t(entry), ix=t(ix))
    oracle.kv_append(c.kv_codes, c.kv_scales, c.ix_codes, c.ix_scales, c.block_table, c.page_size, kv, ix, entry)
    c.n_entries[:] = n0 + n_new
    cache.n_entries.copy_(t(c.n_entries))
    # window: overwrite ring rows 0..3 with new tokens
    wx = (rng.standard_normal((B, 4, 512)) * 2).astype(np.float32)
    wrow = np.tile(np.arange(4, dtype=np.int32), (B, 1))
    win = dev_window(L.win)
    csa2.window_append(win.codes, t(wx), t(wrow), row_scale=win.row_scale)
    oracle.window_append(L.win.codes, L.win.row_scale, wx, wrow)
    r = oracle.layer_step("F", c, L.win, L.q, L.qix_codes, L.qix_scales, L.w, k=wl.k, want_scores=True)
    assert np.isin(entry, r["idx"]).any(), "no appended entry selected; the case proves nothing"
    call = csa2.LayerCall("F", cache, win, t(L.q), wl.k, qix_codes=t(L.qix_codes),
                          qix_scales=t(L.qix_scales), w=t(L.w))
    call()
    torch.cuda.synchronize()
    g_idx = call.idx_out.cpu().numpy()
    for b in range(B):
        assert_selection_matches(r["scores"][b, 0], r["idx"][b, 0], g_idx[b, 0], what=f"append b{b}")
    # attention compared on the GPU's own selection
    o_out, o_lse, _ = oracle.sparse_attend(c, g_idx, L.q, L.win)
    assert_attention_close(call.out.cpu().numpy(), call.lse.cpu().numpy(), o_out, o_lse, "append+attend")
