"""Python binding of the CSA2 decode library for MI355X (gfx950).

A thin ctypes layer over ``libcsa2.so`` with the same entry points as
``include/csa2.h``: it checks tensor devices/dtypes/shapes, passes raw device
pointers and the current HIP stream, and raises on a non-OK status. Every
step of the computation runs in the library's HIP kernels; torch only owns
device memory and streams. There is no CPU fallback: without the built
library every call raises.
"""

from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass
from typing import Optional

import torch  # noqa: F401  (loaded first so the library binds to torch's HIP runtime)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

FULL, REINDEX, REUSE = 0, 1, 2
MODES = {"F": FULL, "R": REINDEX, "U": REUSE, FULL: FULL, REINDEX: REINDEX, REUSE: REUSE}
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small", 4: "HIP error"}
LATENT, HEADS, IX_HEADS, IX_DIM = 512, 16, 4, 64


class CSA2Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"csa2 status {status} ({STATUS.get(status, '?')}): {message}")
        self.status = status


class _Cache(C.Structure):
    _fields_ = [("kv_codes", C.c_void_p), ("kv_scales", C.c_void_p), ("ix_codes", C.c_void_p),
                ("ix_scales", C.c_void_p), ("block_table", C.c_void_p), ("n_entries", C.c_void_p),
                ("page_size", C.c_int32), ("max_pages", C.c_int32), ("num_pages", C.c_int32)]


class _Window(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("row_scale", C.c_void_p), ("length", C.c_void_p),
                ("pos0", C.c_void_p), ("rows", C.c_int32), ("window", C.c_int32)]


class _LayerArgs(C.Structure):
    _fields_ = [("mode", C.c_int), ("cache", C.c_void_p), ("win", C.c_void_p), ("q", C.c_void_p),
                ("qix_codes", C.c_void_p), ("qix_scales", C.c_void_p), ("w", C.c_void_p),
                ("q_pos", C.c_void_p), ("batch", C.c_int32), ("nq", C.c_int32), ("k", C.c_int32),
                ("pool", C.c_int32), ("idx_in", C.c_void_p), ("idx_out", C.c_void_p),
                ("pool_out", C.c_void_p), ("sm_scale", C.c_float), ("out", C.c_void_p),
                ("lse", C.c_void_p), ("ws", C.c_void_p), ("ws_bytes", C.c_size_t)]


_lib = None


def lib():
    """Load libcsa2.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise CSA2Error(4, f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = C.CDLL(LIB_PATH)
        L.csa2_workspace_bytes.restype = C.c_size_t
        L.csa2_workspace_bytes.argtypes = [C.c_int, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                           C.c_int32, C.c_int32]
        L.csa2_last_error.restype = C.c_char_p
        L.csa2_status_string.restype = C.c_char_p
        L.csa2_version.restype = C.c_char_p
        for name in ("csa2_index_score", "csa2_topk", "csa2_sparse_attend", "csa2_sparse_attend_noalloc",
                     "csa2_layer_step",
                     "csa2_index_topk", "csa2_dequant_fp4", "csa2_dequant_e4m3", "csa2_quantize_fp4", "csa2_kv_append",
                     "csa2_window_append", "csa2_stream_read", "csa2_set_attend_kernel"):
            getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


EXPORTS = ["csa2_index_score", "csa2_topk", "csa2_sparse_attend", "csa2_sparse_attend_noalloc", "csa2_layer_step",
           "csa2_index_topk", "csa2_workspace_bytes", "csa2_dequant_fp4", "csa2_dequant_e4m3",
           "csa2_quantize_fp4", "csa2_kv_append", "csa2_window_append", "csa2_stream_read",
           "csa2_set_attend_kernel",
           "csa2_status_string", "csa2_last_error", "csa2_version"]


def _check(status: int):
    if status != 0:
        raise CSA2Error(status, lib().csa2_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: Optional[torch.Tensor], dtype, name, shape=None):
    if t is None:
        return
    if not t.is_cuda:
        raise CSA2Error(1, f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise CSA2Error(1, f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise CSA2Error(1, f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise CSA2Error(1, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


@dataclass
class Cache:
    """Device tensors of one Full layer's paged cache."""

    kv_codes: torch.Tensor    # [num_pages, page, 256] uint8
    kv_scales: torch.Tensor   # [num_pages, page, 32] uint8
    ix_codes: torch.Tensor    # [num_pages, page, 32] uint8
    ix_scales: torch.Tensor   # [num_pages, page, 4] uint8
    block_table: torch.Tensor  # [B, max_pages] int32
    n_entries: torch.Tensor   # [B] int32

    @property
    def page_size(self) -> int:
        return int(self.kv_codes.shape[1])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def capacity(self) -> int:
        return self.max_pages * self.page_size

    def struct(self) -> _Cache:
        P, S = self.kv_codes.shape[0], self.kv_codes.shape[1]
        _dev(self.kv_codes, torch.uint8, "kv_codes", (P, S, 256))
        _dev(self.kv_scales, torch.uint8, "kv_scales", (P, S, 32))
        _dev(self.ix_codes, torch.uint8, "ix_codes", (P, S, 32))
        _dev(self.ix_scales, torch.uint8, "ix_scales", (P, S, 4))
        _dev(self.block_table, torch.int32, "block_table")
        _dev(self.n_entries, torch.int32, "n_entries")
        s = _Cache()
        s.kv_codes, s.kv_scales = self.kv_codes.data_ptr(), self.kv_scales.data_ptr()
        s.ix_codes, s.ix_scales = self.ix_codes.data_ptr(), self.ix_scales.data_ptr()
        s.block_table, s.n_entries = self.block_table.data_ptr(), self.n_entries.data_ptr()
        s.page_size, s.max_pages, s.num_pages = S, self.max_pages, P
        return s


@dataclass
class Window:
    codes: torch.Tensor                 # [B, rows, 512] uint8 (E4M3)
    length: torch.Tensor                # [B] int32
    row_scale: Optional[torch.Tensor] = None  # [B, rows] float32
    pos0: Optional[torch.Tensor] = None       # [B] int32
    window: int = 128

    def struct(self) -> _Window:
        B, rows = self.codes.shape[0], self.codes.shape[1]
        _dev(self.codes, torch.uint8, "window codes", (B, rows, 512))
        _dev(self.length, torch.int32, "window length", (B,))
        _dev(self.row_scale, torch.float32, "window row_scale", (B, rows))
        _dev(self.pos0, torch.int32, "window pos0", (B,))
        s = _Window()
        s.codes, s.length = self.codes.data_ptr(), self.length.data_ptr()
        s.row_scale = None if self.row_scale is None else self.row_scale.data_ptr()
        s.pos0 = None if self.pos0 is None else self.pos0.data_ptr()
        s.rows, s.window = rows, int(self.window)
        return s

    def span(self, q_pos) -> int:
        return int(self.window) if (self.pos0 is not None and q_pos is not None) else int(self.codes.shape[1])


def workspace_bytes(mode, batch: int, nq: int, n_cols: int, k: int, pool: int = 0,
                    win_cap: int = 0) -> int:
    return int(lib().csa2_workspace_bytes(MODES[mode], batch, nq, n_cols, k, pool, win_cap))


def alloc_workspace(nbytes: int, device=None) -> torch.Tensor:
    """A device byte buffer (torch's allocator hands out 256-byte aligned blocks)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device or "cuda")


def index_score(cache: Cache, qix_codes, qix_scales, w, q_pos=None, cand=None, out=None, hist=None):
    B, nq = qix_codes.shape[0], qix_codes.shape[1]
    _dev(qix_codes, torch.uint8, "qix_codes", (B, nq, 4, 32))
    _dev(qix_scales, torch.uint8, "qix_scales", (B, nq, 4, 4))
    _dev(w, torch.float32, "w", (B, nq, 4))
    _dev(q_pos, torch.int32, "q_pos", (B, nq))
    n_cand = 0
    if cand is not None:
        n_cand = cand.shape[-1]
        _dev(cand, torch.int32, "cand", (B, nq, n_cand))
    n_cols = n_cand if cand is not None else cache.capacity
    if out is None:
        out = torch.empty(B, nq, n_cols, dtype=torch.float32, device=qix_codes.device)
    _dev(out, torch.float32, "scores", (B, nq, n_cols))
    _dev(hist, torch.int32, "hist", (B, nq, 4096))
    cs = cache.struct()
    _check(lib().csa2_index_score(C.byref(cs), _ptr(qix_codes), _ptr(qix_scales), _ptr(w), _ptr(q_pos),
                                  _ptr(cand), C.c_int32(n_cand), C.c_int32(B), C.c_int32(nq),
                                  _ptr(out), _ptr(hist), _stream()))
    return out


class IndexTopkCall:
    """Pre-marshalled arguments of one csa2_index_topk call: a Full layer's
    scoring and selection without attention (reusable in a timed loop)."""

    def __init__(self, cache: Cache, qix_codes, qix_scales, w, k: int, q_pos=None, pool: int = 0,
                 idx_out=None, pool_out=None, ws=None):
        B, nq = qix_codes.shape[0], qix_codes.shape[1]
        _dev(qix_codes, torch.uint8, "qix_codes", (B, nq, 4, 32))
        _dev(qix_scales, torch.uint8, "qix_scales", (B, nq, 4, 4))
        _dev(w, torch.float32, "w", (B, nq, 4))
        _dev(q_pos, torch.int32, "q_pos", (B, nq))
        dev = qix_codes.device
        if idx_out is None:
            idx_out = torch.empty(B, nq, k, dtype=torch.int32, device=dev)
        _dev(idx_out, torch.int32, "idx_out", (B, nq, k))
        if pool > 0:
            if pool_out is None:
                pool_out = torch.empty(B, nq, pool, dtype=torch.int32, device=dev)
            _dev(pool_out, torch.int32, "pool_out", (B, nq, pool))
        need = workspace_bytes(FULL, B, nq, cache.capacity, k, pool, 0)
        if ws is None:
            ws = alloc_workspace(need, dev)
        self.keep = (cache, qix_codes, qix_scales, w, q_pos, ws)
        self.cs = cache.struct()
        self.args = (C.byref(self.cs), _ptr(qix_codes), _ptr(qix_scales), _ptr(w), _ptr(q_pos),
                     C.c_int32(B), C.c_int32(nq), C.c_int32(k), C.c_int32(pool), _ptr(idx_out),
                     _ptr(pool_out), _ptr(ws), C.c_size_t(ws.numel()))
        self.idx_out, self.pool_out = idx_out, pool_out

    def __call__(self, stream=None):
        st = _stream() if stream is None else C.c_void_p(stream)
        _check(lib().csa2_index_topk(*self.args, st))
        return self


def index_topk(cache: Cache, qix_codes, qix_scales, w, k: int, q_pos=None, pool: int = 0):
    """A Full layer's top-k (and pool) without attention -> (idx, pool or None)."""
    c = IndexTopkCall(cache, qix_codes, qix_scales, w, k, q_pos=q_pos, pool=pool)()
    return c.idx_out, c.pool_out


def topk(scores, k: int, cand=None, out=None, ws=None):
    """scores [B, nq, n] fp32 -> idx [B, nq, k] int32 (ascending ids, -1 padded)."""
    B, nq, n = scores.shape
    _dev(scores, torch.float32, "scores")
    _dev(cand, torch.int32, "cand", (B, nq, n))
    if out is None:
        out = torch.empty(B, nq, k, dtype=torch.int32, device=scores.device)
    _dev(out, torch.int32, "idx_out", (B, nq, k))
    need = workspace_bytes(REINDEX, B, nq, n, k)
    if ws is None:
        ws = alloc_workspace(need, scores.device)
    _check(lib().csa2_topk(_ptr(scores), _ptr(cand), C.c_int32(B), C.c_int32(nq), C.c_int32(n),
                           C.c_int32(k), _ptr(out), _ptr(ws), C.c_size_t(ws.numel()), _stream()))
    return out


def sparse_attend(cache: Cache, idx, q, win: Optional[Window], q_pos=None, sm_scale=None,
                  out=None, lse=None, ws=None):
    B, nq, k = idx.shape
    _dev(idx, torch.int32, "idx")
    _dev(q, torch.float32, "q", (B, nq, HEADS, LATENT))
    _dev(q_pos, torch.int32, "q_pos", (B, nq))
    if sm_scale is None:
        sm_scale = LATENT ** -0.5
    if out is None:
        out = torch.empty(B, nq, HEADS, LATENT, dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty(B, nq, HEADS, dtype=torch.float32, device=q.device)
    _dev(out, torch.float32, "out", (B, nq, HEADS, LATENT))
    _dev(lse, torch.float32, "lse", (B, nq, HEADS))
    wcap = 0 if win is None else win.span(q_pos)
    need = workspace_bytes(REUSE, B, nq, 0, k, 0, wcap)
    if ws is None:
        ws = alloc_workspace(need, q.device)
    cs = cache.struct()
    wsct = None if win is None else win.struct()
    _check(lib().csa2_sparse_attend(C.byref(cs), _ptr(idx), C.c_int32(k), _ptr(q),
                                    None if wsct is None else C.byref(wsct), _ptr(q_pos),
                                    C.c_float(sm_scale), C.c_int32(B), C.c_int32(nq), _ptr(out),
                                    _ptr(lse), _ptr(ws), C.c_size_t(ws.numel()), _stream()))
    return out, lse


ATTEND_KERNELS = {"auto": 0, "seg": 1, "pair": 2}


def set_attend_kernel(name: str):
    """csa2_set_attend_kernel: the attention kernel of the calls that follow
    ("auto", "seg": eight waves per unit, "pair": paired waves); process-wide."""
    if name not in ATTEND_KERNELS:
        raise CSA2Error(1, f"attend kernel {name!r} is not one of {sorted(ATTEND_KERNELS)}")
    _check(lib().csa2_set_attend_kernel(C.c_int32(ATTEND_KERNELS[name])))


def stream_read(x: torch.Tensor, sink: torch.Tensor, blocks: int = 2048):
    """Measurement probe: read every byte of the device tensor x once (csa2_stream_read)."""
    if not x.is_cuda or not sink.is_cuda or sink.dtype != torch.int32 or sink.numel() < 1024:
        raise CSA2Error(1, "x and sink (>= 1024 int32) must be device tensors")
    _check(lib().csa2_stream_read(_ptr(x), C.c_size_t(x.numel() * x.element_size()), _ptr(sink),
                                  C.c_int32(blocks), _stream()))


def sparse_attend_noalloc(cache: Cache, idx, q, win: Optional[Window], out, lse, q_pos=None, sm_scale=None):
    """csa2_sparse_attend_noalloc: the attention with the library's own scratch.
    Allocates nothing: the caller passes out [B, nq, 16, 512] and lse [B, nq, 16]."""
    B, nq, k = idx.shape
    _dev(idx, torch.int32, "idx")
    _dev(q, torch.float32, "q", (B, nq, HEADS, LATENT))
    _dev(q_pos, torch.int32, "q_pos", (B, nq))
    if out is None or lse is None:
        raise CSA2Error(1, "out and lse must be given (this entry point allocates nothing)")
    _dev(out, torch.float32, "out", (B, nq, HEADS, LATENT))
    _dev(lse, torch.float32, "lse", (B, nq, HEADS))
    if sm_scale is None:
        sm_scale = LATENT ** -0.5
    cs = cache.struct()
    wsct = None if win is None else win.struct()
    _check(lib().csa2_sparse_attend_noalloc(C.byref(cs), _ptr(idx), C.c_int32(k), _ptr(q),
                                            None if wsct is None else C.byref(wsct), _ptr(q_pos),
                                            C.c_float(sm_scale), C.c_int32(B), C.c_int32(nq), _ptr(out),
                                            _ptr(lse), _stream()))
    return out, lse


class LayerCall:
    """Pre-marshalled arguments of one csa2_layer_step call (reusable in a timed loop)."""

    def __init__(self, mode, cache: Cache, win: Optional[Window], q, k: int, pool: int = 0,
                 qix_codes=None, qix_scales=None, w=None, q_pos=None, idx_in=None, idx_out=None,
                 pool_out=None, out=None, lse=None, ws=None, sm_scale=None):
        m = MODES[mode]
        B, nq = q.shape[0], q.shape[1]
        _dev(q, torch.float32, "q", (B, nq, HEADS, LATENT))
        dev = q.device
        if m in (FULL, REINDEX):
            _dev(qix_codes, torch.uint8, "qix_codes", (B, nq, 4, 32))
            _dev(qix_scales, torch.uint8, "qix_scales", (B, nq, 4, 4))
            _dev(w, torch.float32, "w", (B, nq, 4))
            if idx_out is None:
                idx_out = torch.empty(B, nq, k, dtype=torch.int32, device=dev)
            _dev(idx_out, torch.int32, "idx_out", (B, nq, k))
        if m == FULL and pool > 0:
            if pool_out is None:
                pool_out = torch.empty(B, nq, pool, dtype=torch.int32, device=dev)
            _dev(pool_out, torch.int32, "pool_out", (B, nq, pool))
        if m == REINDEX:
            _dev(idx_in, torch.int32, "idx_in (pool)", (B, nq, pool))
        if m == REUSE:
            _dev(idx_in, torch.int32, "idx_in", (B, nq, k))
        _dev(q_pos, torch.int32, "q_pos", (B, nq))
        if out is None:
            out = torch.empty(B, nq, HEADS, LATENT, dtype=torch.float32, device=dev)
        if lse is None:
            lse = torch.empty(B, nq, HEADS, dtype=torch.float32, device=dev)
        n_cols = cache.capacity if m == FULL else (pool if m == REINDEX else 0)
        wcap = 0 if win is None else win.span(q_pos)
        need = workspace_bytes(m, B, nq, n_cols, k, pool, wcap)
        if ws is None:
            ws = alloc_workspace(need, dev)
        self.keep = (cache, win, q, qix_codes, qix_scales, w, q_pos, idx_in, ws)
        self.cache_s = cache.struct()
        self.win_s = None if win is None else win.struct()
        a = _LayerArgs()
        a.mode = m
        a.cache = C.addressof(self.cache_s)
        a.win = None if self.win_s is None else C.addressof(self.win_s)
        a.q = q.data_ptr()
        a.qix_codes = None if qix_codes is None else qix_codes.data_ptr()
        a.qix_scales = None if qix_scales is None else qix_scales.data_ptr()
        a.w = None if w is None else w.data_ptr()
        a.q_pos = None if q_pos is None else q_pos.data_ptr()
        a.batch, a.nq, a.k, a.pool = B, nq, k, pool
        a.idx_in = None if idx_in is None else idx_in.data_ptr()
        a.idx_out = None if idx_out is None else idx_out.data_ptr()
        a.pool_out = None if pool_out is None else pool_out.data_ptr()
        a.sm_scale = LATENT ** -0.5 if sm_scale is None else sm_scale
        a.out, a.lse = out.data_ptr(), lse.data_ptr()
        a.ws, a.ws_bytes = ws.data_ptr(), ws.numel()
        self.args = a
        self.out, self.lse, self.idx_out, self.pool_out = out, lse, idx_out, pool_out
        self.mode = m

    def __call__(self, stream=None):
        st = _stream() if stream is None else C.c_void_p(stream)
        _check(lib().csa2_layer_step(C.byref(self.args), st))
        return self


def layer_step(mode, cache, win, q, k, **kw) -> LayerCall:
    return LayerCall(mode, cache, win, q, k, **kw)()


def dequant_fp4(codes, scales):
    """codes [n, C/2], scales [n, C/16] uint8 -> fp16 [n, C] (exact)."""
    n, half = codes.shape
    _dev(codes, torch.uint8, "codes")
    _dev(scales, torch.uint8, "scales", (n, half * 2 // 16))
    out = torch.empty(n, half * 2, dtype=torch.float16, device=codes.device)
    _check(lib().csa2_dequant_fp4(_ptr(codes), _ptr(scales), C.c_int64(n), C.c_int32(half * 2),
                                  _ptr(out), _stream()))
    return out


def dequant_e4m3(b):
    _dev(b, torch.uint8, "bytes")
    out = torch.empty(b.shape, dtype=torch.float32, device=b.device)
    _check(lib().csa2_dequant_e4m3(_ptr(b), C.c_int64(b.numel()), _ptr(out), _stream()))
    return out


# ---- the write side of the cache ----

def quantize_fp4(x, codes=None, scales=None):
    """fp32 rows [..., C] (C a multiple of 16) -> (codes [..., C/2], scales [..., C/16]) uint8."""
    _dev(x, torch.float32, "x")
    ch = x.shape[-1]
    n = x.numel() // ch if ch else 0
    if codes is None:
        codes = torch.empty(*x.shape[:-1], ch // 2, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(*x.shape[:-1], ch // 16, dtype=torch.uint8, device=x.device)
    _dev(codes, torch.uint8, "codes", tuple(x.shape[:-1]) + (ch // 2,))
    _dev(scales, torch.uint8, "scales", tuple(x.shape[:-1]) + (ch // 16,))
    _check(lib().csa2_quantize_fp4(_ptr(x), C.c_int64(n), C.c_int32(ch), _ptr(codes), _ptr(scales),
                                   _stream()))
    return codes, scales


class _CacheW(C.Structure):
    _fields_ = [("kv_codes", C.c_void_p), ("kv_scales", C.c_void_p), ("ix_codes", C.c_void_p),
                ("ix_scales", C.c_void_p), ("block_table", C.c_void_p), ("page_size", C.c_int32),
                ("max_pages", C.c_int32), ("num_pages", C.c_int32)]


def kv_append(cache: Cache, kv, entry, ix=None):
    """Quantise new entries into the cache in place: kv [B, n_new, 512] fp32,
    ix [B, n_new, 64] fp32 or None, entry [B, n_new] int32 (entry index, < 0: none).
    The caller advances cache.n_entries."""
    B, n_new = entry.shape
    _dev(entry, torch.int32, "entry")
    _dev(kv, torch.float32, "kv", (B, n_new, LATENT))
    _dev(ix, torch.float32, "ix", (B, n_new, 64))
    cw = _CacheW(cache.kv_codes.data_ptr(), cache.kv_scales.data_ptr(), cache.ix_codes.data_ptr(),
                 cache.ix_scales.data_ptr(), cache.block_table.data_ptr(), cache.page_size,
                 cache.max_pages, cache.kv_codes.shape[0])
    _check(lib().csa2_kv_append(C.byref(cw), _ptr(kv), _ptr(ix), _ptr(entry), C.c_int32(B),
                                C.c_int32(n_new), _stream()))


def window_append(codes, x, row, row_scale=None):
    """Encode window tokens into the ring in place: codes [B, rows, 512] uint8,
    x [B, n_new, 512] fp32, row [B, n_new] int32 (ring row, < 0: none),
    row_scale [B, rows] fp32 or None."""
    B, rows = codes.shape[0], codes.shape[1]
    n_new = row.shape[1]
    _dev(codes, torch.uint8, "codes", (B, rows, LATENT))
    _dev(x, torch.float32, "x", (B, n_new, LATENT))
    _dev(row, torch.int32, "row", (B, n_new))
    _dev(row_scale, torch.float32, "row_scale", (B, rows))
    _check(lib().csa2_window_append(_ptr(codes), _ptr(row_scale), C.c_int32(rows), _ptr(x), _ptr(row),
                                    C.c_int32(B), C.c_int32(n_new), _stream()))


def version() -> str:
    return lib().csa2_version().decode()
