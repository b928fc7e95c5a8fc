"""Seeded synthetic CSA2 workloads.

Shapes follow the workloads described for DeepSeek V4.1 Flash's CSA2
(compressed sparse attention, second generation): a compressed main-KV latent
of 512 channels shared by 16 query heads, an FP4 lightning indexer of 4 heads
x 64 channels with one 64-channel key per compressed entry, 4 tokens per
compressed entry, a 128-token FP8 sliding window, top-K 2048 and a 16384-entry
candidate pool.

Value recipe (all seeded, numpy PCG64 via ``SeedSequence``):

* main-KV latent, indexer keys, indexer queries, window rows: N(0,1) before
  quantisation (FP4 blocks for the first three, E4M3 for the window);
* on round(1% of N) indexer keys per request, chosen uniformly, +3.0 is added
  to all 64 channels before quantisation, so the top-K is not degenerate;
* per-head indexer weights w ~ U[0.5, 1.5); main query fp32 N(0,1);
* window row scale absent (1.0).

Large caches draw their FP4 16-channel blocks from a pool of 2^20 blocks that
were themselves quantised from N(0,1) draws; each block of the cache is an
independent uniform pick from that pool (so every block still has the exact
quantised-N(0,1) distribution, but blocks repeat). Small caches quantise fresh
draws directly.

Nothing here decodes the formats or computes scores or attention.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

from .fp_encode import encode_e4m3, encode_fp4_blocks

D_LATENT = 512
N_HEADS = 16
IX_HEADS = 4
IX_DIM = 64
TOKENS_PER_ENTRY = 4
WINDOW = 128
POOL_BLOCKS = 1 << 20

# stream tags for SeedSequence
_T_KV, _T_IX, _T_BIAS, _T_PAGES, _T_CTX = 1, 2, 3, 4, 5
_T_Q, _T_QIX, _T_W, _T_WIN = 10, 11, 12, 13


def _rng(seed: int, *path: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, *path]))


@dataclass
class Cache:
    """One Full layer's compressed cache in a paged layout.

    Entry s of request b lives at page ``block_table[b, s // page_size]``,
    slot ``s % page_size``.
    """

    kv_codes: np.ndarray  # [num_pages, page, 256] uint8, E2M1 pairs
    kv_scales: np.ndarray  # [num_pages, page, 32] uint8, E4M3
    ix_codes: np.ndarray  # [num_pages, page, 32] uint8
    ix_scales: np.ndarray  # [num_pages, page, 4] uint8
    block_table: np.ndarray  # [B, max_pages] int32 (-1 where unused)
    n_entries: np.ndarray  # [B] int32
    page_size: int

    @property
    def num_pages(self) -> int:
        return int(self.kv_codes.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    def nbytes(self) -> int:
        return sum(a.nbytes for a in (self.kv_codes, self.kv_scales, self.ix_codes, self.ix_scales))


@dataclass
class Window:
    """Per-layer sliding-window rows (E4M3) of each request.

    Decode (``pos0 is None``): the ``length[b]`` valid rows are the last
    tokens and all of them are visible to the decode query. Prefill: row j
    holds token ``pos0[b] + j`` and a query at position p sees the rows with
    token position in ``(p - window, p]``.
    """

    codes: np.ndarray  # [B, rows, 512] uint8
    row_scale: Optional[np.ndarray]  # [B, rows] float32 or None (= 1)
    length: np.ndarray  # [B] int32
    pos0: Optional[np.ndarray] = None  # [B] int32
    window: int = WINDOW


@dataclass
class LayerInputs:
    mode: str  # "F" (Full), "R" (Reindex), "U" (Reuse)
    cache_id: int
    q: np.ndarray  # [B, nq, 16, 512] float32
    win: Window
    qix_codes: Optional[np.ndarray] = None  # [B, nq, 4, 32] uint8
    qix_scales: Optional[np.ndarray] = None  # [B, nq, 4, 4] uint8
    w: Optional[np.ndarray] = None  # [B, nq, 4] float32


@dataclass
class DecodeWorkload:
    name: str
    contexts: np.ndarray  # [B] tokens of context per request
    nq: int
    k: int
    pool: int
    caches: List[Cache]
    layers: List[LayerInputs]
    q_pos: Optional[np.ndarray] = None  # [B, nq] int32 absolute positions (prefill)
    sm_scale: float = 1.0 / math.sqrt(D_LATENT)
    window: int = WINDOW
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.contexts.shape[0])

    @property
    def modes(self) -> str:
        return "".join(l.mode for l in self.layers)


PrefillWorkload = DecodeWorkload


def _fp4_rows(rng: np.random.Generator, n_rows: int, channels: int, shift: float = 0.0):
    """FP4 rows of ``channels`` N(shift, 1) values: (codes [n, C/2], scales [n, C/16])."""
    nblk = channels // 16
    if n_rows * nblk <= POOL_BLOCKS:
        x = rng.standard_normal((n_rows, channels), dtype=np.float32)
        if shift:
            x += np.float32(shift)
        return encode_fp4_blocks(x)
    px = rng.standard_normal((POOL_BLOCKS, 16), dtype=np.float32)
    if shift:
        px += np.float32(shift)
    pc, ps = encode_fp4_blocks(px)  # [P, 8], [P, 1]
    ps = ps[:, 0]
    codes = np.empty((n_rows, channels // 2), np.uint8)
    scales = np.empty((n_rows, nblk), np.uint8)
    chunk = max(1, (1 << 24) // nblk)
    for r0 in range(0, n_rows, chunk):
        r1 = min(n_rows, r0 + chunk)
        ids = rng.integers(0, POOL_BLOCKS, size=(r1 - r0, nblk), dtype=np.uint32)
        codes[r0:r1] = pc[ids].reshape(r1 - r0, channels // 2)
        scales[r0:r1] = ps[ids]
    return codes, scales


def _page_layout(seed, stream, cache_idx, n_entries, page_size, shuffle):
    B = len(n_entries)
    npages = [max(1, -(-int(n) // page_size)) for n in n_entries]
    max_pages = max(npages)
    if shuffle:
        num_pages = sum(npages)
        perm = _rng(seed, stream, _T_PAGES, cache_idx).permutation(num_pages).astype(np.int32)
        bt = np.full((B, max_pages), -1, np.int32)
        off = 0
        for b, npg in enumerate(npages):
            bt[b, :npg] = perm[off:off + npg]
            off += npg
    else:
        num_pages = B * max_pages
        bt = (np.arange(B, dtype=np.int32)[:, None] * max_pages
              + np.arange(max_pages, dtype=np.int32)[None, :])
    return bt, num_pages


def make_cache(seed, stream, cache_idx, n_entries, page_size=64, shuffle=False,
               bias_frac=0.01, bias=3.0) -> Cache:
    n_entries = np.asarray(n_entries, np.int32)
    bt, num_pages = _page_layout(seed, stream, cache_idx, n_entries, page_size, shuffle)
    n_phys = num_pages * page_size
    kc, ks = _fp4_rows(_rng(seed, stream, _T_KV, cache_idx), n_phys, D_LATENT)
    ic, isc = _fp4_rows(_rng(seed, stream, _T_IX, cache_idx), n_phys, IX_DIM)
    rb = _rng(seed, stream, _T_BIAS, cache_idx)
    for b, n in enumerate(n_entries):
        nb = int(round(bias_frac * int(n)))
        if nb == 0:
            continue
        chosen = rb.choice(int(n), size=nb, replace=False)
        phys = bt[b, chosen // page_size].astype(np.int64) * page_size + chosen % page_size
        bc, bs = _fp4_rows(rb, nb, IX_DIM, shift=bias)
        ic[phys] = bc
        isc[phys] = bs
    return Cache(
        kv_codes=kc.reshape(num_pages, page_size, D_LATENT // 2),
        kv_scales=ks.reshape(num_pages, page_size, D_LATENT // 16),
        ix_codes=ic.reshape(num_pages, page_size, IX_DIM // 2),
        ix_scales=isc.reshape(num_pages, page_size, IX_DIM // 16),
        block_table=bt,
        n_entries=n_entries,
        page_size=page_size,
    )


def make_window(seed, stream, layer_idx, contexts, rows=WINDOW, pos0=None, window=WINDOW,
                row_scale=False) -> Window:
    B = len(contexts)
    r = _rng(seed, stream, _T_WIN, layer_idx)
    x = r.standard_normal((B, rows, D_LATENT), dtype=np.float32)
    codes = encode_e4m3(x).reshape(B, rows, D_LATENT)
    if pos0 is None:
        length = np.minimum(np.asarray(contexts, np.int64), rows).astype(np.int32)
    else:
        pos0 = np.asarray(pos0, np.int32)
        length = np.minimum(np.asarray(contexts, np.int64) - pos0, rows).astype(np.int32)
    rs = None
    if row_scale:
        rs = r.uniform(0.25, 2.0, size=(B, rows)).astype(np.float32)
    return Window(codes=codes, row_scale=rs, length=length, pos0=pos0, window=window)


def make_layer(seed, stream, layer_idx, mode, cache_id, contexts, nq, win_rows=WINDOW,
               win_pos0=None, window=WINDOW, row_scale=False) -> LayerInputs:
    B = len(contexts)
    q = _rng(seed, stream, _T_Q, layer_idx).standard_normal(
        (B, nq, N_HEADS, D_LATENT), dtype=np.float32)
    win = make_window(seed, stream, layer_idx, contexts, rows=win_rows, pos0=win_pos0,
                      window=window, row_scale=row_scale)
    li = LayerInputs(mode=mode, cache_id=cache_id, q=q, win=win)
    if mode in ("F", "R"):
        x = _rng(seed, stream, _T_QIX, layer_idx).standard_normal(
            (B, nq, IX_HEADS, IX_DIM), dtype=np.float32)
        li.qix_codes, li.qix_scales = encode_fp4_blocks(x)
        li.w = _rng(seed, stream, _T_W, layer_idx).uniform(
            0.5, 1.5, size=(B, nq, IX_HEADS)).astype(np.float32)
    return li


def build_workload(*, name, contexts, layers, k, pool=0, page_size=64, shuffle=False, nq=1,
                   prefill=False, seed=0, stream=0, row_scale=False, bias_frac=0.01,
                   window=WINDOW) -> DecodeWorkload:
    """Assemble a workload: one cache per Full layer, per-layer q / window / indexer query.

    ``layers`` is a string over {F, R, U}; the first must be F. Reindex and
    Reuse layers read the most recent Full layer's cache.
    """
    contexts = np.asarray(contexts, np.int64)
    if not layers or layers[0] != "F":
        raise ValueError("the first layer must be Full")
    n_entries = (contexts // TOKENS_PER_ENTRY).astype(np.int32)
    caches, lays = [], []
    q_pos = None
    win_rows, win_pos0 = window, None
    if prefill:
        q_pos = (contexts[:, None] - nq + np.arange(nq)[None, :]).astype(np.int32)
        win_pos0 = np.maximum(contexts - nq - (window - 1), 0).astype(np.int32)
        win_rows = int((contexts - win_pos0).max())
    for li, mode in enumerate(layers):
        if mode == "F":
            caches.append(make_cache(seed, stream, len(caches), n_entries, page_size, shuffle,
                                     bias_frac=bias_frac))
        lays.append(make_layer(seed, stream, li, mode, len(caches) - 1, contexts, nq,
                               win_rows=win_rows, win_pos0=win_pos0, window=window,
                               row_scale=row_scale))
    return DecodeWorkload(name=name, contexts=contexts, nq=nq, k=k, pool=pool, caches=caches,
                          layers=lays, q_pos=q_pos, window=window,
                          meta=dict(seed=seed, stream=stream, page_size=page_size,
                                    shuffle=shuffle))


def _ragged_contexts(seed, n=64, lo=4096, hi=1 << 20):
    r = _rng(seed, 5, _T_CTX)
    t = np.exp(r.uniform(math.log(lo), math.log(hi), size=n))
    return np.clip(np.floor(t), lo, hi).astype(np.int64)


def _pattern20():
    return ("FRUUUU" * 4)[:20]


# The five benchmark workloads, by name. Each entry builds the full-size inputs.
CONFIGS = {
    "tiny_b1_8k_full": dict(
        contexts=[8192], layers="F", k=256, pool=0, stream=1),
    "b32_128k_full_reuse5": dict(
        contexts=[131072] * 32, layers="FUUUUU", k=2048, pool=0, stream=2),
    "b8_1m_full_reindex_reuse4": dict(
        contexts=[1 << 20] * 8, layers="FRUUUU", k=2048, pool=16384, stream=3),
    "prefill_4096q_128k": dict(
        contexts=[131072], layers="F", k=2048, pool=0, nq=4096, prefill=True, stream=4),
    "ragged64_paged_20layer": dict(
        contexts=None, layers=_pattern20(), k=2048, pool=16384, shuffle=True, stream=5),
    # speculative verification: the last 6 tokens (5 drafts + 1) of each 1M-token
    # request are queries, each with its own position (block-causal visibility
    # among the newest entries, causal window)
    "b8_1m_spec6": dict(
        contexts=[1 << 20] * 8, layers="FRUUUU", k=2048, pool=16384, nq=6, prefill=True, stream=6),
}


def make_decode_workload(name: str, seed: int = 0, layers: Optional[str] = None,
                         batch: Optional[int] = None) -> DecodeWorkload:
    """Build one of the named full-size workloads (optionally fewer layers / requests)."""
    spec = dict(CONFIGS[name])
    if spec["contexts"] is None:
        spec["contexts"] = _ragged_contexts(seed)
    if batch is not None:
        spec["contexts"] = list(spec["contexts"])[:batch]
    if layers is not None:
        spec["layers"] = layers
    return build_workload(name=name, seed=seed, **spec)


def make_prefill_workload(seed: int = 0, nq: Optional[int] = None,
                          context: Optional[int] = None) -> DecodeWorkload:
    spec = dict(CONFIGS["prefill_4096q_128k"])
    if nq is not None:
        spec["nq"] = nq
    if context is not None:
        spec["contexts"] = [context]
    return build_workload(name="prefill_4096q_128k", seed=seed, **spec)


def make_small_decode(contexts, layers="F", k=16, pool=0, page_size=64, shuffle=False, nq=1,
                      prefill=False, seed=0, stream=100, row_scale=False, bias_frac=0.01,
                      window=WINDOW) -> DecodeWorkload:
    """Small workloads for tests (same recipe, arbitrary sizes)."""
    return build_workload(name="small", contexts=contexts, layers=layers, k=k, pool=pool,
                          page_size=page_size, shuffle=shuffle, nq=nq, prefill=prefill,
                          seed=seed, stream=stream, row_scale=row_scale,
                          bias_frac=bias_frac, window=window)


# ---- subsets (array slicing only) ---------------------------------------------

def take_requests(wl: DecodeWorkload, reqs) -> DecodeWorkload:
    """The same workload restricted to some requests (caches keep every page)."""
    reqs = list(reqs)

    def cs(c: Cache):
        return Cache(kv_codes=c.kv_codes, kv_scales=c.kv_scales, ix_codes=c.ix_codes,
                         ix_scales=c.ix_scales, block_table=c.block_table[reqs],
                         n_entries=c.n_entries[reqs], page_size=c.page_size)

    def ws(w: Window):
        return Window(codes=w.codes[reqs], row_scale=None if w.row_scale is None else w.row_scale[reqs],
                          length=w.length[reqs], pos0=None if w.pos0 is None else w.pos0[reqs],
                          window=w.window)

    layers = []
    for L in wl.layers:
        layers.append(LayerInputs(mode=L.mode, cache_id=L.cache_id, q=L.q[reqs], win=ws(L.win),
                                  qix_codes=None if L.qix_codes is None else L.qix_codes[reqs],
                                  qix_scales=None if L.qix_scales is None else L.qix_scales[reqs],
                                  w=None if L.w is None else L.w[reqs]))
    return DecodeWorkload(name=wl.name + "_slice", contexts=wl.contexts[reqs], nq=wl.nq, k=wl.k,
                          pool=wl.pool, caches=[cs(c) for c in wl.caches], layers=layers,
                          q_pos=None if wl.q_pos is None else wl.q_pos[reqs], sm_scale=wl.sm_scale,
                          window=wl.window, meta=dict(wl.meta))


def take_queries(wl: DecodeWorkload, qs) -> DecodeWorkload:
    """The same (single-request) workload restricted to some query rows."""
    qs = list(qs)
    layers = []
    for L in wl.layers:
        layers.append(LayerInputs(mode=L.mode, cache_id=L.cache_id, q=L.q[:, qs], win=L.win,
                                  qix_codes=None if L.qix_codes is None else L.qix_codes[:, qs],
                                  qix_scales=None if L.qix_scales is None else L.qix_scales[:, qs],
                                  w=None if L.w is None else L.w[:, qs]))
    return DecodeWorkload(name=wl.name + "_qslice", contexts=wl.contexts, nq=len(qs), k=wl.k,
                          pool=wl.pool, caches=wl.caches, layers=layers,
                          q_pos=None if wl.q_pos is None else wl.q_pos[:, qs], sm_scale=wl.sm_scale,
                          window=wl.window, meta=dict(wl.meta))
