"""The C-ABI library on the host: it loads, exports every declared symbol, and
rejects bad arguments before launching anything (no GPU needed)."""

import ctypes as C
import glob
import os
import re

import pytest

import compressed_sparse_attention_06_amd as csa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

EINVAL, EUNSUPPORTED, EWORKSPACE = 1, 2, 3


def declared_functions():
    """Every csa2_* function declared in include/*.h."""
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = csa2.lib()
    decl = declared_functions()
    assert len(decl) >= 10
    for name in decl:
        assert hasattr(L, name), name
    assert set(csa2.EXPORTS) <= set(decl)


def test_version_and_status_strings():
    assert "gfx950" in csa2.version()
    L = csa2.lib()
    assert L.csa2_status_string(0) == b"ok"
    assert L.csa2_status_string(3) == b"workspace too small"


def _cache_struct(page_size=64, max_pages=4, num_pages=8, null_bt=False):
    s = csa2._Cache()
    dummy = 0x1000  # never dereferenced: validation reads no device memory
    s.kv_codes = s.kv_scales = s.ix_codes = s.ix_scales = dummy
    s.block_table = None if null_bt else dummy
    s.n_entries = dummy
    s.page_size, s.max_pages, s.num_pages = page_size, max_pages, num_pages
    return s


def _layer(mode=csa2.FULL, **over):
    cs = _cache_struct(**{k: over.pop(k) for k in list(over) if k in ("page_size", "max_pages", "num_pages", "null_bt")})
    a = csa2._LayerArgs()
    a.mode = mode
    a.cache = C.addressof(cs)
    a.q = a.qix_codes = a.qix_scales = a.w = a.out = a.lse = a.idx_out = a.idx_in = 0x2000
    a.batch, a.nq, a.k, a.pool = 2, 1, 16, 0
    a.sm_scale = 0.04
    a.ws, a.ws_bytes = 0x10000, 0
    for k, v in over.items():
        setattr(a, k, v)
    return a, cs


def _step(a):
    return csa2.lib().csa2_layer_step(C.byref(a), None)


def test_layer_step_validation():
    L = csa2.lib()
    assert L.csa2_layer_step(None, None) == EINVAL
    a, keep = _layer(k=0)
    assert _step(a) == EINVAL
    a, keep = _layer(k=5000)
    assert _step(a) == EINVAL
    a, keep = _layer(batch=0)
    assert _step(a) == EINVAL
    a, keep = _layer(q=None)
    assert _step(a) == EINVAL
    a, keep = _layer(mode=7)
    assert _step(a) == EINVAL
    a, keep = _layer(null_bt=True)
    assert _step(a) == EINVAL
    a, keep = _layer(page_size=48)
    assert _step(a) == EUNSUPPORTED
    a, keep = _layer(pool=8)  # pool < k
    assert _step(a) == EINVAL
    a, keep = _layer(pool=32, pool_out=None)
    assert _step(a) == EINVAL
    a, keep = _layer(mode=csa2.REINDEX, pool=32, idx_in=None)
    assert _step(a) == EINVAL
    a, keep = _layer(mode=csa2.REUSE, idx_in=None)
    assert _step(a) == EINVAL
    a, keep = _layer(sm_scale=float("inf"))
    assert _step(a) == EINVAL
    a, keep = _layer(mode=csa2.FULL, qix_codes=None)
    assert _step(a) == EINVAL
    # everything valid but the workspace: missing, misaligned, short
    a, keep = _layer(ws=None, ws_bytes=1 << 30)
    assert _step(a) == EWORKSPACE
    a, keep = _layer(ws=0x10010, ws_bytes=1 << 30)
    assert _step(a) == EWORKSPACE
    need = csa2.workspace_bytes(csa2.FULL, 2, 1, 4 * 64, 16)
    a, keep = _layer(ws_bytes=need - 1)
    assert _step(a) == EWORKSPACE
    assert b"needed" in L.csa2_last_error()


def test_other_entry_points_validation():
    L = csa2.lib()
    cs = _cache_struct()
    p = C.c_void_p(0x2000)
    assert L.csa2_index_score(None, p, p, p, None, None, 0, 1, 1, p, None, None) == EINVAL
    assert L.csa2_index_score(C.byref(cs), None, p, p, None, None, 0, 1, 1, p, None, None) == EINVAL
    assert L.csa2_index_score(C.byref(cs), p, p, p, None, p, 0, 1, 1, p, None, None) == EINVAL
    assert L.csa2_topk(p, None, 1, 1, 100, 0, p, p, C.c_size_t(1 << 30), None) == EINVAL
    assert L.csa2_topk(p, None, 1, 1, 100, 8, p, None, C.c_size_t(0), None) == EWORKSPACE
    assert L.csa2_sparse_attend(C.byref(cs), p, 0, p, None, None, C.c_float(0.04), 1, 1, p, p, p,
                                C.c_size_t(1 << 30), None) == EINVAL
    w = csa2._Window()
    w.rows, w.window = 16, 0
    assert L.csa2_sparse_attend(C.byref(cs), p, 8, p, C.byref(w), None, C.c_float(0.04), 1, 1, p, p,
                                p, C.c_size_t(1 << 30), None) == EINVAL
    assert L.csa2_dequant_fp4(p, p, 4, 48, p, None) == EINVAL
    assert L.csa2_dequant_e4m3(None, 4, p, None) == EINVAL
    # the write side: bad sizes, alignment and missing arrays are rejected on the host
    assert L.csa2_quantize_fp4(p, C.c_int64(4), 40, p, p, None) == EINVAL
    assert L.csa2_quantize_fp4(C.c_void_p(0x2004), C.c_int64(4), 64, p, p, None) == EINVAL
    assert L.csa2_quantize_fp4(None, C.c_int64(4), 64, p, p, None) == EINVAL
    cw = csa2._CacheW(0x2000, 0x2000, 0, 0, 0x2000, 64, 4, 4)
    assert L.csa2_kv_append(C.byref(cw), p, p, p, 1, 1, None) == EINVAL  # ix without indexer arrays
    cw = csa2._CacheW(0x2000, 0x2000, 0x2000, 0x2000, 0x2000, 48, 4, 4)
    assert L.csa2_kv_append(C.byref(cw), p, None, p, 1, 1, None) == EUNSUPPORTED
    assert L.csa2_window_append(p, None, 0, p, p, 1, 1, None) == EINVAL
    assert L.csa2_window_append(p, None, 8, C.c_void_p(0x2008), p, 1, 1, None) == EINVAL
    # scoring + selection without attention
    big = C.c_size_t(1 << 40)
    assert L.csa2_index_topk(C.byref(cs), None, p, p, None, 1, 1, 8, 0, p, None, p, big, None) == EINVAL
    assert L.csa2_index_topk(C.byref(cs), p, p, p, None, 1, 1, 0, 0, p, None, p, big, None) == EINVAL
    assert L.csa2_index_topk(C.byref(cs), p, p, p, None, 1, 1, 8, 4, p, p, p, big, None) == EINVAL  # pool < k
    assert L.csa2_index_topk(C.byref(cs), p, p, p, None, 1, 1, 8, 16, p, None, p, big, None) == EINVAL
    assert L.csa2_index_topk(C.byref(cs), p, p, p, None, 1, 1, 8, 0, p, None, None, C.c_size_t(0),
                             None) == EWORKSPACE
    # the attention-kernel choice: 0 (auto), 1 (eight waves), 2 (paired waves); nothing else
    for k in (3, -1):
        assert L.csa2_set_attend_kernel(k) == EINVAL
    for k in (1, 2, 0):
        assert L.csa2_set_attend_kernel(k) == 0


@pytest.mark.parametrize("mode,n_cols,k,pool,win", [
    (csa2.FULL, 262144, 2048, 16384, 128),
    (csa2.FULL, 2048, 256, 0, 128),
    (csa2.REINDEX, 16384, 2048, 16384, 128),
    (csa2.REUSE, 0, 2048, 0, 128),
])
def test_workspace_sizes(mode, n_cols, k, pool, win):
    nb = csa2.workspace_bytes(mode, 8, 1, n_cols, k, pool, win)
    assert nb % 256 == 0
    splits = -(-(k + win) // 256)
    assert nb >= 8 * splits * 16 * 514 * 4
    if mode != csa2.REUSE:
        assert nb >= 8 * n_cols * 4
    assert csa2.workspace_bytes(mode, 0, 1, n_cols, k, pool, win) == 0


@pytest.mark.parametrize("batch,nq,n_cols,pool,fused", [
    (1, 4096, 32768, 0, True),      # the 4096-query chunk of a 128K context
    (2, 512, 32768, 0, True),       # 1024 rows over two requests
    (1, 4096, 32768, 2048, False),  # a pool to select as well
    (1, 1000, 32768, 0, False),     # too few rows to fill the GPU 16 at a time
    (32, 32, 32768, 0, False),      # fewer than 64 query rows per request
    (1, 4096, 65536, 0, False),     # more entries than one row's bitmap covers
])
def test_fused_prefill_topk_workspace(batch, nq, n_cols, pool, fused):
    """The fused prefill selection keeps no score matrix: its Full-layer
    workspace is exactly the attention's; every other Full call reserves the
    score rows."""
    full = csa2.workspace_bytes(csa2.FULL, batch, nq, n_cols, 256, pool, 128)
    att = csa2.workspace_bytes(csa2.REUSE, batch, nq, 0, 256, 0, 128)
    if fused:
        assert full == att
    else:
        assert full >= att + batch * nq * n_cols * 4


@pytest.mark.parametrize("rows,groups", [
    (8, 136),    # 17 units per row, one workgroup each
    (32, 192),   # 6 workgroups per row: 2-3 units each, none spanning two rows
    (48, 240),   # 5 per row: 3-4 units each
    (64, 256),   # 4 per row: 4-5 units each
    (100, 256),  # a row-aligned split would give 9 units to some workgroup: plain split (6-7)
])
def test_attention_split_workgroups(rows, groups):
    """A Reuse call's workspace is the attention partials, two slots of
    16 x 516 floats per workgroup: it shows how many workgroups share the rows
    (2048 entries + a 128-row window = 17 units of 128 positions per row).
    When some multiple of the row count keeps the largest range as short as
    the plain split over 256 workgroups, whole rows are shared out (no range
    spans two rows), with the fewest workgroups per row that do so."""
    part = 2 * 16 * (512 + 4) * 4
    nb = csa2.workspace_bytes(csa2.REUSE, rows, 1, 0, 2048, 0, 128)
    assert nb == -(-groups * part // 256) * 256
