"""ctypes wrapper of the CSA2 CPU oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The HIP library never does, and the two
share no code: the oracle is a separate C file with its own decoders.
"""

from __future__ import annotations

import contextlib
import ctypes as C
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

MODE = {"F": 0, "R": 1, "U": 2}


def build(quiet: bool = True) -> str:
    """Compile the oracle with gcc (plain C11, -O2, OpenMP over independent rows)."""
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", _LIB, _SRC, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + r.stderr)
    if not quiet and r.stderr:
        print(r.stderr)
    return _LIB


def _open(path):
    L = C.CDLL(path)
    L.orc_e2m1.restype = C.c_double
    L.orc_e2m1.argtypes = [C.c_int]
    L.orc_e4m3.restype = C.c_double
    L.orc_e4m3.argtypes = [C.c_int]
    L.orc_num_threads.restype = C.c_int
    return L


_default = None


def lib():
    """The built oracle library (built on first use if missing or stale)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _default = _open(_LIB)
    return _default


def build_variant(source_text: str, out_path: str) -> str:
    """Compile a modified copy of the oracle source (used to plant mistakes in tests)."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(source_text)
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-I", _HERE,
           "-o", out_path, src, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("oracle variant build failed:\n" + r.stderr)
    return out_path


def source() -> str:
    with open(_SRC) as f:
        return f.read()


@contextlib.contextmanager
def using(path: str):
    """Route every call of this module to another build of the oracle."""
    global _default
    old = lib()
    _default = _open(path)
    try:
        yield
    finally:
        _default = old


class _Cache(C.Structure):
    _fields_ = [("kv_codes", C.c_void_p), ("kv_scales", C.c_void_p), ("ix_codes", C.c_void_p),
                ("ix_scales", C.c_void_p), ("block_table", C.c_void_p), ("n_entries", C.c_void_p),
                ("page_size", C.c_int32), ("max_pages", C.c_int32), ("num_pages", C.c_int32)]


class _Window(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("row_scale", C.c_void_p), ("length", C.c_void_p),
                ("pos0", C.c_void_p), ("rows", C.c_int32), ("window", C.c_int32)]


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


class _Keep:
    """Holds contiguous copies alive while a C struct points at them."""

    def __init__(self):
        self.items = []

    def __call__(self, a, dtype):
        a = _c(a, dtype)
        if a is not None:
            self.items.append(a)
        return a


def _cache_struct(cache, keep):
    s = _Cache()
    s.kv_codes = _p(keep(cache.kv_codes, np.uint8))
    s.kv_scales = _p(keep(cache.kv_scales, np.uint8))
    s.ix_codes = _p(keep(cache.ix_codes, np.uint8))
    s.ix_scales = _p(keep(cache.ix_scales, np.uint8))
    s.block_table = _p(keep(cache.block_table, np.int32))
    s.n_entries = _p(keep(cache.n_entries, np.int32))
    s.page_size = int(cache.page_size)
    s.max_pages = int(cache.block_table.shape[1])
    s.num_pages = int(cache.kv_codes.shape[0])
    return s


def _window_struct(win, keep):
    if win is None:
        return None
    s = _Window()
    s.codes = _p(keep(win.codes, np.uint8))
    s.row_scale = _p(keep(win.row_scale, np.float32))
    s.length = _p(keep(win.length, np.int32))
    s.pos0 = _p(keep(win.pos0, np.int32))
    s.rows = int(win.codes.shape[1])
    s.window = int(win.window)
    return s


def e2m1(code: int) -> float:
    return lib().orc_e2m1(int(code))


def e4m3(byte: int) -> float:
    return lib().orc_e4m3(int(byte))


def dequant_fp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    ch = codes.shape[-1] * 2
    n = codes.size // codes.shape[-1]
    out = np.empty(codes.shape[:-1] + (ch,), np.float64)
    lib().orc_dequant_fp4(C.c_void_p(codes.ctypes.data), C.c_void_p(scales.ctypes.data),
                          C.c_int64(n), C.c_int32(ch), C.c_void_p(out.ctypes.data))
    return out


def dequant_e4m3(b: np.ndarray, row_scale: Optional[np.ndarray] = None) -> np.ndarray:
    b = np.ascontiguousarray(b, np.uint8)
    ch = b.shape[-1]
    n = b.size // ch
    rs = _c(row_scale, np.float32)
    out = np.empty(b.shape, np.float64)
    lib().orc_dequant_e4m3(C.c_void_p(b.ctypes.data), None if rs is None else C.c_void_p(rs.ctypes.data),
                           C.c_int64(n), C.c_int32(ch), C.c_void_p(out.ctypes.data))
    return out


# ---- encoding: the write side of the cache (readings in csa2_oracle.h) ----

def e4m3_encode(x) -> np.ndarray:
    """E4M3 bytes of fp32 values: nearest finite value, ties to even, saturating."""
    x = np.ascontiguousarray(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().orc_e4m3_encode_n(C.c_void_p(x.ctypes.data), C.c_int64(x.size), C.c_void_p(out.ctypes.data))
    return out


def e2m1_encode(y: float) -> int:
    """E2M1 code (sign in bit 3) of a value already divided by its block scale."""
    L = lib()
    L.orc_e2m1_encode.argtypes = [C.c_float]
    return int(L.orc_e2m1_encode(C.c_float(y)))


def quantize_fp4(x: np.ndarray):
    """Rows [..., C] (C a multiple of 16) -> (codes [..., C/2], scales [..., C/16])."""
    x = np.ascontiguousarray(x, np.float32)
    ch = x.shape[-1]
    n = x.size // ch
    codes = np.empty(x.shape[:-1] + (ch // 2,), np.uint8)
    scales = np.empty(x.shape[:-1] + (ch // 16,), np.uint8)
    lib().orc_quantize_fp4(C.c_void_p(x.ctypes.data), C.c_int64(n), C.c_int32(ch),
                           C.c_void_p(codes.ctypes.data), C.c_void_p(scales.ctypes.data))
    return codes, scales


class _CacheW(C.Structure):
    _fields_ = [("kv_codes", C.c_void_p), ("kv_scales", C.c_void_p), ("ix_codes", C.c_void_p),
                ("ix_scales", C.c_void_p), ("block_table", C.c_void_p), ("page_size", C.c_int32),
                ("max_pages", C.c_int32), ("num_pages", C.c_int32)]


def kv_append(kv_codes, kv_scales, ix_codes, ix_scales, block_table, page_size, kv, ix, entry):
    """Quantise and write new entries into the (numpy) cache arrays in place.
    kv [B][n_new][512], ix [B][n_new][64] or None, entry [B][n_new] (< 0: none)."""
    for a in (kv_codes, kv_scales, ix_codes, ix_scales):
        assert a.flags["C_CONTIGUOUS"] and a.dtype == np.uint8
    bt = np.ascontiguousarray(block_table, np.int32)
    kv = np.ascontiguousarray(kv, np.float32)
    ixa = None if ix is None else np.ascontiguousarray(ix, np.float32)
    en = np.ascontiguousarray(entry, np.int32)
    B, n_new = en.shape
    num_pages = kv_codes.shape[0] // page_size if kv_codes.ndim == 2 else kv_codes.shape[0]
    cw = _CacheW(kv_codes.ctypes.data, kv_scales.ctypes.data, ix_codes.ctypes.data, ix_scales.ctypes.data,
                 bt.ctypes.data, page_size, bt.shape[-1], num_pages)
    lib().orc_kv_append(C.byref(cw), C.c_void_p(kv.ctypes.data),
                        None if ixa is None else C.c_void_p(ixa.ctypes.data),
                        C.c_void_p(en.ctypes.data), C.c_int32(B), C.c_int32(n_new))


def window_append(codes, row_scale, x, row):
    """Encode window rows into codes [B][rows][512] (and row_scale [B][rows]) in place.
    x [B][n_new][512], row [B][n_new] (< 0: none)."""
    assert codes.flags["C_CONTIGUOUS"] and codes.dtype == np.uint8
    if row_scale is not None:
        assert row_scale.flags["C_CONTIGUOUS"] and row_scale.dtype == np.float32
    x = np.ascontiguousarray(x, np.float32)
    rw = np.ascontiguousarray(row, np.int32)
    B, n_new = rw.shape
    lib().orc_window_append(C.c_void_p(codes.ctypes.data),
                            None if row_scale is None else C.c_void_p(row_scale.ctypes.data),
                            C.c_int32(codes.shape[1]), C.c_void_p(x.ctypes.data),
                            C.c_void_p(rw.ctypes.data), C.c_int32(B), C.c_int32(n_new))


def index_score(cache, qix_codes, qix_scales, w, q_pos=None, cand=None, n_cols=None):
    keep = _Keep()
    cs = _cache_struct(cache, keep)
    qc = keep(qix_codes, np.uint8)
    qs = keep(qix_scales, np.uint8)
    ww = keep(w, np.float32)
    B, nq = qc.shape[0], qc.shape[1]
    qp = keep(q_pos, np.int32)
    cd = keep(cand, np.int32)
    if cd is not None:
        n_cols = cd.shape[-1]
        cd = keep(np.broadcast_to(cd.reshape(B, -1, n_cols), (B, nq, n_cols)), np.int32)
    elif n_cols is None:
        n_cols = cache.block_table.shape[1] * cache.page_size
    out = np.empty((B, nq, n_cols), np.float64)
    lib().orc_index_score(C.byref(cs), C.c_void_p(qc.ctypes.data), C.c_void_p(qs.ctypes.data),
                          C.c_void_p(ww.ctypes.data), None if qp is None else C.c_void_p(qp.ctypes.data),
                          None if cd is None else C.c_void_p(cd.ctypes.data), C.c_int32(n_cols),
                          C.c_int32(B), C.c_int32(nq), C.c_int32(n_cols), C.c_void_p(out.ctypes.data))
    return out


def topk(scores: np.ndarray, k: int, cand: Optional[np.ndarray] = None) -> np.ndarray:
    s = np.ascontiguousarray(scores, np.float64)
    lead = s.shape[:-1]
    n = s.shape[-1]
    rows = int(np.prod(lead)) if lead else 1
    cd = None if cand is None else np.ascontiguousarray(np.broadcast_to(cand, s.shape), np.int32)
    out = np.empty(lead + (k,), np.int32)
    lib().orc_topk(C.c_void_p(s.ctypes.data), None if cd is None else C.c_void_p(cd.ctypes.data),
                   C.c_int32(rows), C.c_int32(1), C.c_int32(n), C.c_int32(k),
                   C.c_void_p(out.ctypes.data))
    return out


def sparse_attend(cache, idx, q, win, q_pos=None, sm_scale=1.0 / np.sqrt(512.0)):
    keep = _Keep()
    cs = _cache_struct(cache, keep)
    ws = _window_struct(win, keep)
    ix = keep(idx, np.int32)
    qq = keep(q, np.float32)
    B, nq = qq.shape[0], qq.shape[1]
    k = ix.shape[-1]
    qp = keep(q_pos, np.int32)
    out = np.empty((B, nq, 16, 512), np.float64)
    lse = np.empty((B, nq, 16), np.float64)
    psum = np.empty((B, nq, 16), np.float64)
    lib().orc_sparse_attend(C.byref(cs), C.c_void_p(ix.ctypes.data), C.c_int32(k),
                            C.c_void_p(qq.ctypes.data), None if ws is None else C.byref(ws),
                            None if qp is None else C.c_void_p(qp.ctypes.data),
                            C.c_double(sm_scale), C.c_int32(B), C.c_int32(nq),
                            C.c_void_p(out.ctypes.data), C.c_void_p(lse.ctypes.data),
                            C.c_void_p(psum.ctypes.data))
    return out, lse, psum


def layer_step(mode, cache, win, q, qix_codes=None, qix_scales=None, w=None, q_pos=None,
               k=2048, pool=0, idx_in=None, sm_scale=1.0 / np.sqrt(512.0), want_scores=False):
    """One layer; returns dict(out, lse, idx, pool, scores)."""
    m = MODE[mode] if isinstance(mode, str) else int(mode)
    keep = _Keep()
    cs = _cache_struct(cache, keep)
    ws = _window_struct(win, keep)
    qq = keep(q, np.float32)
    B, nq = qq.shape[0], qq.shape[1]
    qc = keep(qix_codes, np.uint8)
    qs = keep(qix_scales, np.uint8)
    ww = keep(w, np.float32)
    qp = keep(q_pos, np.int32)
    ii = keep(idx_in, np.int32)
    idx_out = np.full((B, nq, k), -1, np.int32)
    pool_out = np.full((B, nq, max(pool, 1)), -1, np.int32)
    out = np.empty((B, nq, 16, 512), np.float64)
    lse = np.empty((B, nq, 16), np.float64)
    scores = None
    if want_scores and m in (0, 1):
        n = cache.block_table.shape[1] * cache.page_size if m == 0 else pool
        scores = np.empty((B, nq, n), np.float64)

    def vp(a):
        return None if a is None else C.c_void_p(a.ctypes.data)

    rc = lib().orc_layer_step(C.c_int(m), C.byref(cs), None if ws is None else C.byref(ws),
                              vp(qq), vp(qc), vp(qs), vp(ww), vp(qp), C.c_int32(B), C.c_int32(nq),
                              C.c_int32(k), C.c_int32(pool), vp(ii), vp(idx_out),
                              vp(pool_out) if pool > 0 else None, C.c_double(sm_scale),
                              vp(out), vp(lse), vp(scores))
    if rc != 0:
        raise RuntimeError(f"oracle layer_step failed: {rc}")
    res = dict(out=out, lse=lse, scores=scores)
    if m in (0, 1):
        res["idx"] = idx_out
    else:
        res["idx"] = ii
    res["pool"] = pool_out if (m == 0 and pool > 0) else None
    return res


def run_workload(wl, layers=None, want_scores=False):
    """Run every layer of a synth workload through the oracle, in order.

    Full layers emit the pool (if the workload has one) and the top-K;
    Reindex layers rescore the most recent pool; Reuse layers inherit the
    most recent Full/Reindex top-K.
    """
    results = []
    last_idx = None
    last_pool = None
    sel = range(len(wl.layers)) if layers is None else layers
    for li in sel:
        L = wl.layers[li]
        cache = wl.caches[L.cache_id]
        idx_in = None
        if L.mode == "R":
            idx_in = last_pool
        elif L.mode == "U":
            idx_in = last_idx
        r = layer_step(L.mode, cache, L.win, L.q, L.qix_codes, L.qix_scales, L.w, wl.q_pos,
                       k=wl.k, pool=wl.pool if L.mode != "U" else 0, idx_in=idx_in,
                       sm_scale=wl.sm_scale, want_scores=want_scores)
        if L.mode in ("F", "R"):
            last_idx = r["idx"]
        if L.mode == "F" and wl.pool > 0:
            last_pool = r["pool"]
        results.append(r)
    return results


def num_threads() -> int:
    return lib().orc_num_threads()


def set_num_threads(n: int) -> None:
    """OpenMP threads for later calls (timing only: results do not depend on it)."""
    lib().orc_set_num_threads(int(n))
