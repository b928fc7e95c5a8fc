"""Small hand-built inputs shared by the oracle pins and the GPU parity tests."""

from __future__ import annotations

import json
import os

import numpy as np

from synth.workloads import Cache, Window

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name: str):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def pack_nibbles(nib: np.ndarray) -> np.ndarray:
    """[..., C] codes 0..15 -> [..., C/2] bytes, even channel in the low nibble."""
    nib = np.asarray(nib, np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def hand_cache(n_entries_per_req, page_size=4, ix_nib=None, ix_scales=None, kv_nib=None,
               kv_scales=None, block_table=None, num_pages=None):
    """A cache whose logical entry s of request b holds given codes.

    ``ix_nib`` [B][N][64] nibbles, ``ix_scales`` [B][N][4] bytes, ``kv_nib``
    [B][N][512], ``kv_scales`` [B][N][32]. Entries are placed by the documented
    layout rule: page ``block_table[b][s // page_size]``, slot ``s % page_size``.
    """
    n_entries = np.asarray(n_entries_per_req, np.int32)
    B = len(n_entries)
    Nmax = int(n_entries.max())
    max_pages = max(1, -(-Nmax // page_size))
    if block_table is None:
        block_table = (np.arange(B)[:, None] * max_pages + np.arange(max_pages)[None, :]).astype(np.int32)
    block_table = np.asarray(block_table, np.int32)
    if num_pages is None:
        num_pages = int(block_table.max()) + 1
    kvc = np.zeros((num_pages, page_size, 256), np.uint8)
    kvs = np.zeros((num_pages, page_size, 32), np.uint8)
    ixc = np.zeros((num_pages, page_size, 32), np.uint8)
    ixs = np.zeros((num_pages, page_size, 4), np.uint8)
    for b in range(B):
        for s in range(int(n_entries[b])):
            p, sl = block_table[b, s // page_size], s % page_size
            if ix_nib is not None:
                ixc[p, sl] = pack_nibbles(ix_nib[b][s])
            if ix_scales is not None:
                ixs[p, sl] = ix_scales[b][s]
            if kv_nib is not None:
                kvc[p, sl] = pack_nibbles(kv_nib[b][s])
            if kv_scales is not None:
                kvs[p, sl] = kv_scales[b][s]
    return Cache(kv_codes=kvc, kv_scales=kvs, ix_codes=ixc, ix_scales=ixs,
                 block_table=block_table, n_entries=n_entries, page_size=page_size)


def hand_window(rows_bytes, length=None, row_scale=None, pos0=None, window=128):
    """Window from [B][rows][512] E4M3 bytes."""
    codes = np.asarray(rows_bytes, np.uint8)
    B, rows = codes.shape[0], codes.shape[1]
    if length is None:
        length = np.full(B, rows, np.int32)
    return Window(codes=codes, row_scale=None if row_scale is None else np.asarray(row_scale, np.float32),
                  length=np.asarray(length, np.int32),
                  pos0=None if pos0 is None else np.asarray(pos0, np.int32), window=window)


def reorder_pages(cache: Cache, seed: int = 7) -> Cache:
    """Same logical content, pages moved to a shuffled physical order."""
    rng = np.random.default_rng(seed)
    P = cache.kv_codes.shape[0]
    perm = rng.permutation(P)  # new physical page of old page i is perm[i]
    def mv(a):
        out = np.empty_like(a)
        out[perm] = a
        return out
    bt = cache.block_table.copy()
    valid = bt >= 0
    bt[valid] = perm[bt[valid]]
    return Cache(kv_codes=mv(cache.kv_codes), kv_scales=mv(cache.kv_scales),
                 ix_codes=mv(cache.ix_codes), ix_scales=mv(cache.ix_scales), block_table=bt,
                 n_entries=cache.n_entries.copy(), page_size=cache.page_size)


def band_filtered_sets(oracle_scores_row, oracle_idx_row, gpu_idx_row, k, rel=1e-5):
    """Compare two top-K sets outside the near-tie band of the oracle's K-th score.

    Entries whose oracle score lies within ``rel`` (relative) of the oracle's
    K-th selected score are dropped from both sets; the rest must be equal.
    Returns (oracle_set, gpu_set) after dropping.
    """
    o = [int(i) for i in oracle_idx_row if i >= 0]
    g = [int(i) for i in gpu_idx_row if i >= 0]
    if len(o) == 0:
        return set(), set(g)
    sc = oracle_scores_row
    kth = min(sc[i] for i in o)
    band = rel * abs(kth)
    near = lambda i: abs(sc[i] - kth) <= band  # noqa: E731
    return {i for i in o if not near(i)}, {i for i in g if not near(i)}
