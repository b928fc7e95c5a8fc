"""Pins of the CPU oracle against facts it does not compute itself.

Each pin is a plain function that raises AssertionError when the oracle
disagrees with: a format's value table or an independent library decoder, a
hand-derived closed form (fixtures under tests/golden/), an invariant the
method fixes, a textbook routine that a special case reduces to, or a
brute-force property on tiny inputs. ``test_oracle_pins.py`` runs each one,
and ``test_oracle_mutations.py`` re-runs them against oracle builds with a
planted mistake to show that each plausible mistake is caught.
"""

from __future__ import annotations

import itertools
import math

import numpy as np
import torch

import oracle
from helpers import golden, hand_cache, hand_window, pack_nibbles, reorder_pages
from synth import encode_e4m3, encode_fp4_blocks, make_small_decode

TAU = 1.0 / math.sqrt(512.0)


# ---------------------------------------------------------------- formats

def pin_e2m1_table():
    """All 16 E2M1 codes equal the OCP MX E2M1 value table (golden)."""
    g = golden("e2m1_values.json")["values"]
    got = [oracle.e2m1(c) for c in range(16)]
    assert got == g, got
    assert all(math.copysign(1, a) == math.copysign(1, b) for a, b in zip(got, g))


def pin_e4m3_vs_library():
    """All 256 E4M3 bytes decode as torch's float8_e4m3fn does (an independent decoder)."""
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3(b) for b in range(256)])
    nan_r, nan_g = np.isnan(ref), np.isnan(got)
    assert (nan_r == nan_g).all()
    assert (ref[~nan_r] == got[~nan_g]).all()


def pin_e4m3_landmarks():
    g = golden("e4m3_landmarks.json")
    for b, v in zip(g["bytes"], g["values"]):
        got = oracle.e4m3(b)
        assert got == v and math.copysign(1, got) == math.copysign(1, v), (b, got, v)
    for b in g["nan_bytes"]:
        assert math.isnan(oracle.e4m3(b))


def pin_dequant_fp4_exhaustive():
    """Every (code, scale) pair: value = E2M1 table x library E4M3 value; low nibble = even channel."""
    e2 = golden("e2m1_values.json")["values"]
    e4 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    codes = np.arange(16, dtype=np.uint8)
    # one row per scale byte: 16 channels hold codes 0..15 in order
    nib = np.tile(codes, (256, 1))
    packed = pack_nibbles(nib)
    scales = np.arange(256, dtype=np.uint8)[:, None]
    got = oracle.dequant_fp4(packed, scales)
    want = np.array(e2)[None, :] * e4[:, None]
    fin = ~np.isnan(want)
    assert (np.isnan(got) == ~fin).all()
    assert (got[fin] == want[fin]).all()
    # the byte 0x21 holds channel 0 = code 1 (0.5) and channel 1 = code 2 (1.0)
    row = np.zeros(8, np.uint8)
    row[0] = 0x21
    d = oracle.dequant_fp4(row[None, :], np.array([[0x38]], np.uint8))[0]
    assert d[0] == 0.5 and d[1] == 1.0 and (d[2:] == 0).all()


def pin_dequant_scale_groups():
    """Channel c takes scale c // 16 (distinct power-of-two scales per group)."""
    nib = np.full((1, 512), 2, np.uint8)  # 1.0 everywhere
    scale_bytes = (0x20 + 8 * (np.arange(32) % 4)).astype(np.uint8)  # 2^-3..2^0 repeating
    got = oracle.dequant_fp4(pack_nibbles(nib), scale_bytes[None, :])[0]
    e4 = torch.tensor(scale_bytes).view(torch.float8_e4m3fn).double().numpy()
    assert (got == np.repeat(e4, 16)).all()


def pin_dequant_e4m3_rows():
    b = np.arange(256, dtype=np.uint8).reshape(2, 128)
    rs = np.array([1.0, 0.5], np.float32)
    got = oracle.dequant_e4m3(b, rs)
    ref = torch.tensor(b).view(torch.float8_e4m3fn).double().numpy() * rs[:, None]
    fin = ~np.isnan(ref)
    assert (got[fin] == ref[fin]).all() and np.isnan(got[~fin]).all()


def pin_encoder_roundtrip():
    """Values on the E2M1 grid with amax 6 (scale 1.0) survive encode -> oracle decode exactly."""
    grid = np.array(golden("e2m1_values.json")["values"])
    x = np.array([grid[(5 * c + 3) % 16] for c in range(64)], np.float32)
    x[0] = 6.0  # amax 6 in every block -> scale 1
    x[16], x[32], x[48] = -6.0, 6.0, -6.0
    codes, scales = encode_fp4_blocks(x[None, :])
    assert (scales == 0x38).all()
    assert (oracle.dequant_fp4(codes, scales)[0] == x).all()
    # E4M3 window round trip on its own grid
    v = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    assert (oracle.dequant_e4m3(encode_e4m3(v)[None, :])[0] == v).all()


def pin_encode_golden():
    """Hand-derived E2M1 / E4M3 encodings (ties, saturation, signs) and one FP4 block."""
    g = golden("encode_cases.json")
    for y, code in g["e2m1"]["cases"]:
        assert oracle.e2m1_encode(y) == code, (y, oracle.e2m1_encode(y), code)
    xs = np.array([c[0] for c in g["e4m3"]["cases"]], np.float32)
    assert [int(b) for b in oracle.e4m3_encode(xs)] == [c[1] for c in g["e4m3"]["cases"]]
    blk = g["fp4_block"]
    codes, scales = oracle.quantize_fp4(np.array(blk["x"], np.float32)[None, :])
    assert int(scales[0, 0]) == blk["scale"] and [int(c) for c in codes[0]] == blk["codes"]


def pin_e4m3_encode_vs_library():
    """E4M3 encoding equals torch's float8_e4m3fn conversion (a library routine, round to
    nearest even) on random values, every midpoint between neighbouring values, and
    values past 448 (clamped first: the library maps them to NaN)."""
    rng = np.random.default_rng(3)
    v = torch.arange(0, 127, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    mids = (v[1:] + v[:-1]) / 2
    x = np.concatenate([rng.standard_normal(4000) * 30, rng.standard_normal(2000) * 1e-2, mids, -mids,
                        [500.0, -1e5, 449.0]]).astype(np.float32)
    ref = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(x)
    # the library keeps the sign of a negative value that rounds to zero; the reading sets it too
    assert (got == ref).all(), np.nonzero(got != ref)[0][:5]


def pin_fp4_encode_nearest():
    """On random rows (zero groups, huge and tiny values included): the scale byte is the
    library's E4M3 of fp32(amax/6), and every code is an E2M1 value nearest to x/s (fp32),
    a tie going to the even code; dequantisation then errs by at most half a step."""
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((40, 64)) * np.exp(rng.standard_normal((40, 1)) * 3)).astype(np.float32)
    x[3, :16] = 0.0
    x[5, 16:32] = 1e5
    x[7, :] = rng.integers(-12, 13, 64) * 0.25  # many exact midpoints
    codes, scales = oracle.quantize_fp4(x)
    mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    for r in range(x.shape[0]):
        for grp in range(4):
            blk = x[r, 16 * grp:16 * grp + 16]
            amax = np.float32(np.abs(blk).max())
            sref = torch.tensor([min(float(amax / np.float32(6.0)), 448.0)], dtype=torch.float32)
            sref = int(sref.to(torch.float8_e4m3fn).view(torch.uint8).item())
            assert scales[r, grp] == sref, (r, grp)
            s = np.float32(oracle.e4m3(int(scales[r, grp])))
            for i in range(16):
                ch = 16 * grp + i
                nib = (int(codes[r, ch // 2]) >> (4 * (ch & 1))) & 15
                if s == 0:
                    assert nib & 7 == 0
                    continue
                y = np.float32(blk[i]) / s
                d = np.abs(abs(float(y)) - mags)
                best = np.flatnonzero(d == d.min())
                want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
                assert nib & 7 == want, (r, ch, float(y), nib)
                assert (nib >> 3) == (1 if blk[i] < 0 else 0)


def pin_fp4_grid_roundtrip():
    """Rows built on the grid (E2M1 value x E4M3 scale, one channel at 6 s so that amax/6 = s)
    encode back to the same codes and scale."""
    rng = np.random.default_rng(5)
    grid = np.array(golden("e2m1_values.json")["values"])
    for sb in [0x08, 0x30, 0x38, 0x45, 0x6A, 0x7E]:
        s = oracle.e4m3(sb)
        nib = rng.integers(0, 16, 16)
        nib[rng.integers(0, 16)] = 7
        x = (grid[nib] * s).astype(np.float32)
        codes, scales = oracle.quantize_fp4(x[None, :])
        assert scales[0, 0] == sb
        back = oracle.dequant_fp4(codes, scales)[0]
        assert (back == grid[nib] * s).all()  # -0 comes back as +0, equal as a value


def pin_window_append_rows():
    """A window row with a row scale: rs = amax/448, the largest element encodes to +-448,
    and every byte is the E4M3 nearest to x/rs; without a row scale the bytes encode x.
    Rows not named are left alone."""
    rng = np.random.default_rng(6)
    B, rows = 2, 8
    x = (rng.standard_normal((B, 2, 512)) * 3).astype(np.float32)
    codes = np.full((B, rows, 512), 0x11, np.uint8)
    rs = np.full((B, rows), 7.0, np.float32)
    row = np.array([[3, -1], [0, 7]], np.int32)
    oracle.window_append(codes, rs, x, row)
    for b, j, w in [(0, 0, 3), (1, 0, 0), (1, 1, 7)]:
        amax = np.float32(np.abs(x[b, j]).max())
        assert rs[b, w] == amax / np.float32(448.0)
        y = (x[b, j] / rs[b, w]).astype(np.float32)
        ref = torch.from_numpy(np.clip(y, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert (codes[b, w] == ref).all()
        assert (np.abs(oracle.dequant_e4m3(codes[b, w][None, :])[0]).max() == 448.0)
    untouched = [(0, r) for r in range(rows) if r != 3] + [(1, r) for r in range(1, 7)]
    for b, w in untouched:
        assert (codes[b, w] == 0x11).all() and rs[b, w] == 7.0
    c2 = np.zeros((1, 4, 512), np.uint8)
    oracle.window_append(c2, None, x[:1, :1], np.array([[2]], np.int32))
    ref = torch.from_numpy(np.clip(x[0, 0], -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (c2[0, 2] == ref).all() and (c2[0, [0, 1, 3]] == 0).all()


def pin_kv_append_placement():
    """New entries land at page block_table[b][s/page], slot s%page, main KV and indexer
    key both; other rows are untouched; a missing page or a negative entry writes nothing."""
    rng = np.random.default_rng(7)
    B, page, max_pages, num_pages = 2, 4, 3, 6
    bt = np.array([[5, 0, 2], [1, -1, 4]], np.int32)
    kvc = np.full((num_pages * page, 256), 0xAA, np.uint8)
    kvs = np.full((num_pages * page, 32), 0xAB, np.uint8)
    ixc = np.full((num_pages * page, 32), 0xAC, np.uint8)
    ixs = np.full((num_pages * page, 4), 0xAD, np.uint8)
    kv = rng.standard_normal((B, 3, 512)).astype(np.float32)
    ix = rng.standard_normal((B, 3, 64)).astype(np.float32)
    entry = np.array([[9, 2, -1], [5, 0, 11]], np.int32)  # request 1 entry 5: page 1 missing
    oracle.kv_append(kvc, kvs, ixc, ixs, bt, page, kv, ix, entry)
    written = {}
    for b in range(B):
        for j in range(3):
            s = int(entry[b, j])
            if s < 0 or bt[b, s // page] < 0:
                continue
            r = int(bt[b, s // page]) * page + s % page
            written[r] = (b, j)
    assert sorted(written) == sorted([2 * page + 1, 5 * page + 2, 1 * page + 0, 4 * page + 3])
    for r in range(num_pages * page):
        if r in written:
            b, j = written[r]
            c, sc = oracle.quantize_fp4(kv[b, j][None, :])
            assert (kvc[r] == c[0]).all() and (kvs[r] == sc[0]).all()
            c, sc = oracle.quantize_fp4(ix[b, j][None, :])
            assert (ixc[r] == c[0]).all() and (ixs[r] == sc[0]).all()
        else:
            assert (kvc[r] == 0xAA).all() and (kvs[r] == 0xAB).all()
            assert (ixc[r] == 0xAC).all() and (ixs[r] == 0xAD).all()


# ---------------------------------------------------------------- index score

def _ix_query(q_nib, q_scales, w):
    return (pack_nibbles(np.asarray(q_nib))[None, None], np.asarray(q_scales, np.uint8)[None, None],
            np.asarray(w, np.float32)[None, None])


def pin_score_all_ones():
    case = golden("index_score_cases.json")["cases"][0]
    k_nib = np.full((1, 1, 64), case["k_fill_code"])
    cache = hand_cache([1], page_size=4, ix_nib=k_nib, ix_scales=np.full((1, 1, 4), case["k_scale_byte"]))
    qc, qs, w = _ix_query(np.full((4, 64), case["q_fill_code"]), np.full((4, 4), case["q_scale_byte"]), case["w"])
    s = oracle.index_score(cache, qc, qs, w)
    assert s[0, 0, 0] == case["expected"], s[0, 0, 0]
    assert np.isneginf(s[0, 0, 1:]).all()


def pin_score_one_hot_signs():
    case = golden("index_score_cases.json")["cases"][1]
    q_nib = np.zeros((4, 64), np.uint8)
    q_sc = np.full((4, 4), 0x38, np.uint8)
    for h, ch, code, sbyte in case["q"]:
        q_nib[h, ch] = code
        q_sc[h, ch // 16] = sbyte
    k_nib = np.zeros((1, 1, 64), np.uint8)
    for ch, code in case["k"]:
        k_nib[0, 0, ch] = code
    cache = hand_cache([1], page_size=4, ix_nib=k_nib, ix_scales=np.array(case["k_scales"])[None, None])
    qc, qs, w = _ix_query(q_nib, q_sc, case["w"])
    s = oracle.index_score(cache, qc, qs, w)
    assert s[0, 0, 0] == case["expected"], s[0, 0, 0]


def pin_score_all_heads_negative():
    """q = -k on every head: each dot is negative, ReLU gives exactly 0."""
    k_nib = np.full((1, 1, 64), 3)  # 1.5
    q_nib = np.full((4, 64), 3 | 8)  # -1.5
    cache = hand_cache([1], ix_nib=k_nib, ix_scales=np.full((1, 1, 4), 0x38))
    qc, qs, w = _ix_query(q_nib, np.full((4, 4), 0x38), [1, 1, 1, 1])
    assert oracle.index_score(cache, qc, qs, w)[0, 0, 0] == 0.0


def _ramp_cache(N, page_size=4, B=1, block_table=None, num_pages=None):
    """Indexer key of entry s = (s+1)/2 on channel 0 only (codes grow with s up to 12 entries)."""
    vals = [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    k_nib = np.zeros((B, N, 64), np.uint8)
    k_sc = np.full((B, N, 4), 0x38, np.uint8)
    for b in range(B):
        for s in range(N):
            k_nib[b, s, 0] = 1 + (s % 7)          # value vals[s % 7]
            k_sc[b, s, 0] = 0x38 + 8 * (s // 7)   # x 2^(s // 7)
    want = np.array([vals[s % 7] * 2.0 ** (s // 7) for s in range(N)])
    return hand_cache([N] * B, page_size=page_size, ix_nib=k_nib, ix_scales=k_sc,
                      block_table=block_table, num_pages=num_pages), want


def pin_score_entry_placement():
    """Entry s's score comes from page block_table[s // page], slot s % page (shuffled table)."""
    N, P = 13, 4
    bt = np.array([[3, 0, 2, 1]], np.int32)
    cache, want = _ramp_cache(N, page_size=P, block_table=bt, num_pages=4)
    q_nib = np.zeros((4, 64), np.uint8)
    q_nib[0, 0] = 2  # head 0: q[0] = 1
    qc, qs, w = _ix_query(q_nib, np.full((4, 4), 0x38), [1, 1, 1, 1])
    s = oracle.index_score(cache, qc, qs, w)[0, 0]
    assert (s[:N] == want).all(), (s[:N], want)
    assert np.isneginf(s[N:]).all()


def pin_score_block_causal():
    """Entry s (tokens 4s..4s+3) is visible to position p iff 4(s+1) <= p+1."""
    cache, want = _ramp_cache(8)
    q_nib = np.zeros((4, 64), np.uint8)
    q_nib[0, 0] = 2
    qc, qs, w = _ix_query(q_nib, np.full((4, 4), 0x38), [1, 1, 1, 1])
    for p in range(0, 33):
        s = oracle.index_score(cache, qc, qs, w, q_pos=np.array([[p]], np.int32))[0, 0]
        vis = [i for i in range(8) if 4 * (i + 1) <= p + 1]
        assert [i for i in range(8) if np.isfinite(s[i])] == vis, (p, s)


def pin_score_candidates():
    """Reindex scoring of a candidate list equals the Full score of each listed entry; pads -> -inf."""
    wl = make_small_decode([800], layers="F", k=8)  # 200 entries
    L = wl.layers[0]
    full = oracle.index_score(wl.caches[0], L.qix_codes, L.qix_scales, L.w)[0, 0]
    cand = np.array([[[7, 150, -1, 0, 49, 300, 199]]], np.int32)
    sc = oracle.index_score(wl.caches[0], L.qix_codes, L.qix_scales, L.w, cand=cand)[0, 0]
    for j, e in enumerate(cand[0, 0]):
        if 0 <= e < 200:
            assert sc[j] == full[e]
        else:
            assert np.isneginf(sc[j])


def pin_score_exact_product_bound():
    """Per-head dots are exact in fp64: integer-valued inputs give integer scores."""
    rng = np.random.default_rng(3)
    N = 16
    k_nib = rng.integers(0, 16, size=(1, N, 64)).astype(np.uint8)
    m = k_nib & 7
    k_nib[(m == 1) | (m == 3)] = 2  # drop the 0.5 and 1.5 magnitudes: integer values only
    cache = hand_cache([N], ix_nib=k_nib, ix_scales=np.full((1, N, 4), 0x38))
    q_nib = rng.integers(0, 16, size=(4, 64)).astype(np.uint8)
    m = q_nib & 7
    q_nib[(m == 1) | (m == 3)] = 2
    qc, qs, w = _ix_query(q_nib, np.full((4, 4), 0x38), [1, 2, 3, 4])
    s = oracle.index_score(cache, qc, qs, w)[0, 0, :N]
    assert (s == np.round(s)).all()
    # ... and equal to an integer computation of the same definition
    e2 = np.array(golden("e2m1_values.json")["values"])
    kv = e2[k_nib[0]]
    qv = e2[q_nib]
    ref = (np.maximum(qv @ kv.T, 0) * np.array([1, 2, 3, 4])[:, None]).sum(0)
    assert (s == ref).all()


# ---------------------------------------------------------------- selection

def _brute_topk_ok(scores, ids, sel, k):
    """Defining property of the selection, checked pairwise on tiny rows."""
    valid = [(s, i) for s, i in zip(scores, ids) if s > -math.inf]
    chosen = [i for i in sel if i >= 0]
    assert len(chosen) == min(k, len(valid))
    assert chosen == sorted(chosen)
    assert all(i == -1 for i in sel[len(chosen):])
    sc = {i: s for s, i in valid}
    out = [i for _, i in valid if i not in chosen]
    for a in chosen:
        for b in out:
            assert sc[a] > sc[b] or (sc[a] == sc[b] and a < b), (a, b, sc[a], sc[b])


def pin_topk_ties_and_padding():
    s = np.array([1.0, 3.0, 3.0, 2.0, 3.0, -np.inf, 0.0])
    assert oracle.topk(s, 2).tolist() == [1, 2]
    assert oracle.topk(s, 4).tolist() == [1, 2, 3, 4]
    assert oracle.topk(s, 10).tolist() == [0, 1, 2, 3, 4, 6, -1, -1, -1, -1]
    cand = np.array([9, 4, 7], np.int32)
    assert oracle.topk(np.array([1.0, 5.0, 5.0]), 1, cand=cand).tolist() == [4]
    assert oracle.topk(np.array([-np.inf, -np.inf]), 3).tolist() == [-1, -1, -1]


def pin_topk_bruteforce():
    rng = np.random.default_rng(11)
    for n in range(1, 9):
        for trial in range(6):
            s = rng.integers(-2, 3, size=n).astype(np.float64)  # many exact ties
            s[rng.random(n) < 0.2] = -np.inf
            ids = rng.permutation(50)[:n].astype(np.int32)
            for k in range(1, n + 2):
                sel = oracle.topk(s, k, cand=ids).tolist()
                _brute_topk_ok(s, ids, sel, k)
                # exhaustive cross-check: the chosen set maximises the sorted score vector
                valid = [j for j in range(n) if s[j] > -np.inf]
                kk = min(k, len(valid))
                best = max(itertools.combinations(valid, kk),
                           key=lambda c: (sorted((s[j] for j in c), reverse=True),
                                          [-x for x in sorted(ids[j] for j in c)]))
                assert sorted(int(ids[j]) for j in best) == [i for i in sel if i >= 0]


def pin_layer_full_pool_nesting():
    """Full layer: top-K is a subset of the pool; Reindex over an all-entries pool with the
    Full layer's own indexer query reproduces the Full selection."""
    wl = make_small_decode([600, 257], layers="F", k=24, pool=64, page_size=16, shuffle=True)
    L, c = wl.layers[0], wl.caches[0]
    r = oracle.layer_step("F", c, L.win, L.q, L.qix_codes, L.qix_scales, L.w, k=24, pool=64)
    for b in range(2):
        assert set(r["idx"][b, 0][r["idx"][b, 0] >= 0]) <= set(r["pool"][b, 0][r["pool"][b, 0] >= 0])
    allpool = np.full((2, 1, 600), -1, np.int32)
    for b, n in enumerate(c.n_entries):
        allpool[b, 0, :n] = np.arange(n)
    rr = oracle.layer_step("R", c, L.win, L.q, L.qix_codes, L.qix_scales, L.w, k=24, pool=600,
                           idx_in=allpool)
    assert (rr["idx"] == r["idx"]).all()
    assert np.allclose(rr["out"], r["out"], rtol=0, atol=0)
    # Reindex over the Full layer's own pool (ascending ids of a strict subset, then -1
    # pads for the short request) with the same indexer query: the Full top-K lies inside
    # the pool, so the Reindex selection is the Full one
    wl2 = make_small_decode([600, 257], layers="F", k=24, pool=100, page_size=16, shuffle=True)
    L2, c2 = wl2.layers[0], wl2.caches[0]
    r2 = oracle.layer_step("F", c2, L2.win, L2.q, L2.qix_codes, L2.qix_scales, L2.w, k=24, pool=100)
    assert (r2["pool"][1, 0] == -1).sum() == 100 - 64  # the 257-token request has 64 entries
    rr2 = oracle.layer_step("R", c2, L2.win, L2.q, L2.qix_codes, L2.qix_scales, L2.w, k=24, pool=100,
                            idx_in=r2["pool"])
    assert (rr2["idx"] == r2["idx"]).all()
    assert (rr2["out"] == r2["out"]).all()


def _brute_select(scores_row, ids, k):
    """Top-k of (score, id) pairs by (score desc, id asc) with Python's sort; ascending ids, -1 pads."""
    pairs = sorted(((float(scores_row[i]), int(i)) for i in ids), key=lambda t: (-t[0], t[1]))
    sel = sorted(i for _, i in pairs[:k])
    return sel + [-1] * (k - len(sel))


def pin_layer_reindex_pool_mapping():
    """Reindex with a shuffled pool that is not arange(n) -- a random subset in random order
    with -1 pads and ids at or past the request's entry count -- scores exactly the pool's
    ids with the layer's own indexer query and returns entry ids, not pool slots. Expected
    set: the scores of every entry under that query, restricted to the pool's valid ids and
    ranked by a plain sort on (score desc, id asc)."""
    wl = make_small_decode([2400, 1030], layers="FR", k=20, pool=96, page_size=16, shuffle=True)
    c, R = wl.caches[0], wl.layers[1]
    n_ent = [int(x) for x in c.n_entries]  # 600 and 257
    cap = c.block_table.shape[1] * c.page_size
    P, K = 96, 20
    rng = np.random.default_rng(5)
    pool = np.full((2, 1, P), -1, np.int32)
    for b, n in enumerate(n_ent):
        ids = rng.choice(np.arange(1, n), size=70, replace=False)  # never entry 0, never in order
        extra = [n, n + 3, cap - 1, 10 ** 7, -1, -5]                # not entries of this request
        row = np.concatenate([ids, extra]).astype(np.int32)
        rng.shuffle(row)
        pool[b, 0, :row.size] = row
    assert not (np.diff(pool[0, 0, :70]) > 0).all()
    full = oracle.index_score(c, R.qix_codes, R.qix_scales, R.w)  # every entry, this layer's query
    want = np.full((2, 1, K), -1, np.int32)
    for b, n in enumerate(n_ent):
        valid = [int(s) for s in pool[b, 0] if 0 <= s < n]
        want[b, 0] = _brute_select(full[b, 0], valid, K)
    rr = oracle.layer_step("R", c, R.win, R.q, R.qix_codes, R.qix_scales, R.w, k=K, pool=P, idx_in=pool)
    assert (rr["idx"] == want).all(), (rr["idx"], want)
    # the layer attends the entries it selected, with its own query and window
    o, l, _ = oracle.sparse_attend(c, want, R.q, R.win, sm_scale=TAU)
    assert (rr["out"] == o).all() and (rr["lse"] == l).all()
    # the pool's own scores are the full scores at the pool's ids (-inf elsewhere)
    ps = oracle.index_score(c, R.qix_codes, R.qix_scales, R.w, cand=pool)
    for b, n in enumerate(n_ent):
        for j, s in enumerate(pool[b, 0]):
            assert ps[b, 0, j] == (full[b, 0, s] if 0 <= s < n else -np.inf)
    # a pool shorter than K takes all its valid ids, then -1
    short = np.full((2, 1, P), -1, np.int32)
    short[:, 0, :5] = [[7, 3, 599, 600, 11], [200, 256, 257, 1, 0]]
    rs = oracle.layer_step("R", c, R.win, R.q, R.qix_codes, R.qix_scales, R.w, k=K, pool=P, idx_in=short)
    assert rs["idx"][0, 0].tolist() == [3, 7, 11, 599] + [-1] * (K - 4)
    assert rs["idx"][1, 0].tolist() == [0, 1, 200, 256] + [-1] * (K - 4)


def pin_short_rows_pad():
    """N < K: every entry is selected, the rest is -1."""
    wl = make_small_decode([40], layers="F", k=16)
    L = wl.layers[0]
    r = oracle.layer_step("F", wl.caches[0], L.win, L.q, L.qix_codes, L.qix_scales, L.w, k=16)
    assert r["idx"][0, 0].tolist() == list(range(10)) + [-1] * 6


# ---------------------------------------------------------------- attention

def _rows_of(cache, b, ids):
    out = []
    for s in ids:
        p, sl = cache.block_table[b, s // cache.page_size], s % cache.page_size
        out.append(oracle.dequant_fp4(cache.kv_codes[p, sl][None], cache.kv_scales[p, sl][None])[0])
    return np.array(out).reshape(-1, 512)


def pin_attend_golden():
    case = golden("attend_cases.json")["cases"][0]
    kv = np.zeros((1, 1, 512), np.uint8)
    kv[0, 0, 0] = 2
    cache = hand_cache([1], kv_nib=kv, kv_scales=np.full((1, 1, 32), 0x38))
    wrow = np.zeros((1, 1, 512), np.uint8)
    wrow[0, 0, 0] = 0x40
    win = hand_window(wrow)
    q = np.zeros((1, 1, 16, 512), np.float32)
    a = np.float32(math.log(2.0))
    q[0, 0, 0::2, 0] = a
    out, lse, psum = oracle.sparse_attend(cache, np.array([[[0, -1]]], np.int32), q, win,
                                          sm_scale=case["tau"])
    # q carries ln2 rounded to fp32; propagate that rounding exactly into the closed form
    e1, e2 = math.exp(float(a)), math.exp(2 * float(a))
    assert abs(out[0, 0, 0, 0] - (e1 + 2 * e2) / (e1 + e2)) < 1e-15
    assert abs(out[0, 0, 0, 0] - case["even_out0"]) < 1e-7
    assert abs(lse[0, 0, 0] - math.log(e1 + e2)) < 1e-15
    assert abs(lse[0, 0, 0] - case["even_lse"]) < 1e-7
    assert out[0, 0, 1, 0] == case["odd_out0"] and abs(lse[0, 0, 1] - case["odd_lse"]) < 1e-15
    assert (out[0, 0, :, 1:] == 0).all()
    assert np.allclose(psum, 1.0, atol=1e-14)


def pin_attend_dense_equals_sdpa():
    """K >= N: sparse attention equals dense attention (torch SDPA, fp64) over all entries + window."""
    wl = make_small_decode([97 * 4, 33 * 4], layers="F", k=128, page_size=8, shuffle=True,
                           row_scale=True)
    L, c = wl.layers[0], wl.caches[0]
    idx = np.full((2, 1, 128), -1, np.int32)
    for b in range(2):
        n = int(c.n_entries[b])
        idx[b, 0, :n] = np.random.default_rng(b).permutation(n)
    out, lse, psum = oracle.sparse_attend(c, idx, L.q, L.win, sm_scale=TAU)
    for b in range(2):
        n = int(c.n_entries[b])
        rows = _rows_of(c, b, range(n))
        ln = int(L.win.length[b])
        w = oracle.dequant_e4m3(L.win.codes[b, :ln], L.win.row_scale[b, :ln])
        kv = torch.from_numpy(np.concatenate([rows, w], 0))[None, None]
        qq = torch.from_numpy(L.q[b, 0].astype(np.float64))[None, :, None, :]
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kv, kv, scale=TAU)[0, :, 0]
        ref_lse = torch.logsumexp(TAU * (qq[0, :, 0] @ kv[0, 0].T), dim=-1)
        assert np.abs(out[b, 0] - ref.numpy()).max() < 1e-12
        assert np.abs(lse[b, 0] - ref_lse.numpy()).max() < 1e-12
    assert np.abs(psum - 1).max() < 1e-12


def pin_attend_special_cases():
    """Single row -> that row; identical rows -> that row, lse + ln R; q = 0 -> mean of rows."""
    wl = make_small_decode([64], layers="F", k=8)
    c = wl.caches[0]
    empty_win = hand_window(np.zeros((1, 1, 512), np.uint8), length=[0])
    q = wl.layers[0].q
    out, lse, _ = oracle.sparse_attend(c, np.array([[[5] + [-1] * 7]], np.int32), q, empty_win, sm_scale=TAU)
    r5 = _rows_of(c, 0, [5])[0]
    assert np.abs(out[0, 0] - r5[None, :]).max() < 1e-13
    z = TAU * (q[0, 0].astype(np.float64) @ r5)
    assert np.abs(lse[0, 0] - z).max() < 1e-12
    out3, lse3, _ = oracle.sparse_attend(c, np.array([[[5, 5, 5, -1, -1, -1, -1, -1]]], np.int32), q,
                                         empty_win, sm_scale=TAU)
    assert np.abs(out3[0, 0] - r5[None, :]).max() < 1e-13
    assert np.abs(lse3[0, 0] - (z + math.log(3))).max() < 1e-12
    ids = [0, 3, 9, 10]
    outz, lsez, _ = oracle.sparse_attend(c, np.array([[ids + [-1] * 4]], np.int32),
                                         np.zeros_like(q), empty_win, sm_scale=TAU)
    assert np.abs(outz[0, 0] - _rows_of(c, 0, ids).mean(0)[None, :]).max() < 1e-13
    assert np.abs(lsez - math.log(4)).max() < 1e-14
    oute, lsee, _ = oracle.sparse_attend(c, np.full((1, 1, 8), -1, np.int32), q, empty_win, sm_scale=TAU)
    assert (oute == 0).all() and np.isneginf(lsee).all()


def pin_attend_large_logits():
    """Huge logits (scale 448 rows, large q) stay finite: the max is subtracted."""
    kv = np.full((1, 2, 512), 7, np.uint8)  # 6.0
    cache = hand_cache([2], kv_nib=kv, kv_scales=np.full((1, 2, 32), 0x7E))
    q = np.full((1, 1, 16, 512), 50.0, np.float32)
    win = hand_window(np.zeros((1, 1, 512), np.uint8), length=[0])
    out, lse, _ = oracle.sparse_attend(cache, np.array([[[0, 1]]], np.int32), q, win, sm_scale=TAU)
    assert np.isfinite(out).all() and np.isfinite(lse).all()
    assert np.abs(out - 6.0 * 448.0).max() == 0


def pin_attend_permutation_and_window_rows():
    wl = make_small_decode([400], layers="F", k=32, row_scale=True)
    L, c = wl.layers[0], wl.caches[0]
    ids = np.random.default_rng(1).choice(100, 20, replace=False).astype(np.int32)
    a = np.full((1, 1, 32), -1, np.int32)
    a[0, 0, :20] = ids
    b = np.full((1, 1, 32), -1, np.int32)
    b[0, 0, 5:25] = ids[::-1]
    oa, la, _ = oracle.sparse_attend(c, a, L.q, L.win, sm_scale=TAU)
    ob, lb, _ = oracle.sparse_attend(c, b, L.q, L.win, sm_scale=TAU)
    assert np.abs(oa - ob).max() < 1e-12 and np.abs(la - lb).max() < 1e-12
    # window rows: scaling the row scales by 2 equals doubling those rows
    w2 = hand_window(L.win.codes, L.win.length, L.win.row_scale * 2)
    o2, _, _ = oracle.sparse_attend(c, np.full((1, 1, 32), -1, np.int32), L.q, w2, sm_scale=TAU)
    ow = oracle.dequant_e4m3(L.win.codes[0, :L.win.length[0]], L.win.row_scale[0, :L.win.length[0]] * 2)
    kv = torch.from_numpy(ow)[None, None]
    qq = torch.from_numpy(L.q[0, 0].astype(np.float64))[None, :, None, :]
    ref = torch.nn.functional.scaled_dot_product_attention(qq, kv, kv, scale=TAU)[0, :, 0].numpy()
    assert np.abs(o2[0, 0] - ref).max() < 1e-12


def pin_prefill_window_bounds():
    """A query at position p sees window tokens in (p - W, p]."""
    W = 4
    rows = 10
    codes = np.zeros((1, rows, 512), np.uint8)
    for j in range(rows):
        codes[0, j, 0] = encode_e4m3(np.array([float(j + 1)]))[0]  # row j: channel 0 = j+1
    win = hand_window(codes, length=[rows], pos0=[100], window=W)
    cache = hand_cache([0], page_size=4)
    cache.n_entries[:] = 0
    q = np.zeros((1, 3, 16, 512), np.float32)  # q = 0: out = mean of visible rows
    qpos = np.array([[100, 103, 109]], np.int32)
    out, lse, _ = oracle.sparse_attend(cache, np.full((1, 3, 2), -1, np.int32), q, win,
                                       q_pos=qpos, sm_scale=TAU)
    # visible token positions: p=100 -> {100}; 103 -> {100..103}; 109 -> {106..109}
    assert out[0, 0, 0, 0] == 1.0
    assert out[0, 1, 0, 0] == np.mean([1, 2, 3, 4])
    assert out[0, 2, 0, 0] == np.mean([7, 8, 9, 10])
    assert abs(lse[0, 1, 0] - math.log(4)) < 1e-14


def pin_reuse_equals_full_given_indices():
    wl = make_small_decode([800, 300], layers="FU", k=40, page_size=16, shuffle=True)
    F, U = wl.layers
    c = wl.caches[0]
    rf = oracle.layer_step("F", c, F.win, F.q, F.qix_codes, F.qix_scales, F.w, k=40)
    ru = oracle.layer_step("U", c, F.win, F.q, k=40, idx_in=rf["idx"])
    assert (ru["out"] == rf["out"]).all() and (ru["lse"] == rf["lse"]).all()
    # a Reuse layer with its own q and window equals sparse_attend on the inherited indices
    ru2 = oracle.layer_step("U", c, U.win, U.q, k=40, idx_in=rf["idx"])
    o, l, _ = oracle.sparse_attend(c, rf["idx"], U.q, U.win, sm_scale=TAU)
    assert (ru2["out"] == o).all() and (ru2["lse"] == l).all()


def pin_paged_equals_contiguous():
    wl = make_small_decode([300, 130], layers="F", k=20, page_size=8)
    L, c = wl.layers[0], wl.caches[0]
    c2 = reorder_pages(c)
    r1 = oracle.layer_step("F", c, L.win, L.q, L.qix_codes, L.qix_scales, L.w, k=20, want_scores=True)
    r2 = oracle.layer_step("F", c2, L.win, L.q, L.qix_codes, L.qix_scales, L.w, k=20, want_scores=True)
    assert (r1["idx"] == r2["idx"]).all()
    assert (r1["out"] == r2["out"]).all()


ALL_PINS = [
    pin_e2m1_table, pin_e4m3_vs_library, pin_e4m3_landmarks, pin_dequant_fp4_exhaustive,
    pin_dequant_scale_groups, pin_dequant_e4m3_rows, pin_encoder_roundtrip,
    pin_score_all_ones, pin_score_one_hot_signs, pin_score_all_heads_negative,
    pin_score_entry_placement, pin_score_block_causal, pin_score_candidates,
    pin_score_exact_product_bound, pin_topk_ties_and_padding, pin_topk_bruteforce,
    pin_layer_full_pool_nesting, pin_layer_reindex_pool_mapping, pin_short_rows_pad, pin_attend_golden,
    pin_attend_dense_equals_sdpa, pin_attend_special_cases, pin_attend_large_logits,
    pin_attend_permutation_and_window_rows, pin_prefill_window_bounds,
    pin_reuse_equals_full_given_indices, pin_paged_equals_contiguous,
    pin_encode_golden, pin_e4m3_encode_vs_library, pin_fp4_encode_nearest, pin_fp4_grid_roundtrip,
    pin_window_append_rows, pin_kv_append_placement,
]
