"""Helpers for the GPU parity tests: move synthetic inputs to the device, run
the HIP path layer by layer, slice workloads for the oracle, compare."""

from __future__ import annotations

import numpy as np
import torch

import compressed_sparse_attention_06_amd as csa2
from synth.workloads import Cache as HostCache
from synth.workloads import DecodeWorkload, LayerInputs, Window as HostWindow, take_queries, take_requests


def t(a, dtype=None, device="cuda"):
    if a is None:
        return None
    x = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        x = x.to(dtype)
    return x.to(device)


def dev_cache(c: HostCache) -> csa2.Cache:
    return csa2.Cache(kv_codes=t(c.kv_codes), kv_scales=t(c.kv_scales), ix_codes=t(c.ix_codes),
                      ix_scales=t(c.ix_scales), block_table=t(c.block_table), n_entries=t(c.n_entries))


def dev_window(w: HostWindow):
    if w is None:
        return None
    return csa2.Window(codes=t(w.codes), length=t(w.length), row_scale=t(w.row_scale),
                       pos0=t(w.pos0), window=w.window)


class DevWorkload:
    """Device copies of a workload's inputs (caches, per-layer q / window / indexer query)."""

    def __init__(self, wl: DecodeWorkload):
        self.wl = wl
        self.caches = [dev_cache(c) for c in wl.caches]
        self.layers = []
        for L in wl.layers:
            self.layers.append(dict(mode=L.mode, cache_id=L.cache_id, q=t(L.q), win=dev_window(L.win),
                                    qix_codes=t(L.qix_codes), qix_scales=t(L.qix_scales), w=t(L.w)))
        self.q_pos = t(wl.q_pos)

    def calls(self, layers=None):
        """LayerCall objects chained like the model: Reindex reads the latest Full pool,
        Reuse the latest Full/Reindex top-K."""
        wl = self.wl
        out = []
        last_idx = last_pool = None
        sel = range(len(self.layers)) if layers is None else layers
        for li in sel:
            L = self.layers[li]
            cache = self.caches[L["cache_id"]]
            kw = dict(q_pos=self.q_pos)
            if L["mode"] == "F":
                kw.update(qix_codes=L["qix_codes"], qix_scales=L["qix_scales"], w=L["w"])
                pool = wl.pool
            elif L["mode"] == "R":
                kw.update(qix_codes=L["qix_codes"], qix_scales=L["qix_scales"], w=L["w"], idx_in=last_pool)
                pool = wl.pool
            else:
                kw.update(idx_in=last_idx)
                pool = 0
            call = csa2.LayerCall(L["mode"], cache, L["win"], L["q"], wl.k, pool=pool,
                                  sm_scale=wl.sm_scale, **kw)
            if L["mode"] in ("F", "R"):
                last_idx = call.idx_out
            if L["mode"] == "F" and wl.pool > 0:
                last_pool = call.pool_out
            out.append(call)
        return out


def run_gpu(wl: DecodeWorkload, layers=None):
    dw = DevWorkload(wl)
    calls = dw.calls(layers)
    for c in calls:
        c()
    torch.cuda.synchronize()
    res = []
    for c in calls:
        res.append(dict(out=c.out.cpu().numpy(), lse=c.lse.cpu().numpy(),
                        idx=None if c.idx_out is None else c.idx_out.cpu().numpy(),
                        pool=None if c.pool_out is None else c.pool_out.cpu().numpy()))
    return res


slice_requests = take_requests
slice_queries = take_queries


# ---- comparisons -------------------------------------------------------------------

OUT_MAX_ABS = 2e-3
OUT_MEAN_ABS = 1e-3
LSE_ABS = 1e-4
SCORE_RTOL = 1e-6
BAND_REL = 1e-5


def assert_attention_close(g_out, g_lse, o_out, o_lse, what=""):
    o_out = np.asarray(o_out)
    fin = np.isfinite(o_lse)
    assert (np.isfinite(g_lse) == fin).all(), f"{what}: empty-set rows differ"
    assert (g_out[~fin] == 0).all(), f"{what}: empty rows must give 0"
    d = np.abs(g_out - o_out)
    assert d.max() <= OUT_MAX_ABS, f"{what}: out max-abs {d.max():.3e}"
    assert d.mean() <= OUT_MEAN_ABS, f"{what}: out mean-abs {d.mean():.3e}"
    if fin.any():
        dl = np.abs(g_lse[fin] - o_lse[fin])
        assert dl.max() <= LSE_ABS, f"{what}: lse max-abs {dl.max():.3e}"
    return float(d.max()), float(d.mean())


def band_sets(score_of, o_ids, g_ids, rel=BAND_REL):
    """Top-K sets outside the near-tie band around the oracle's K-th score."""
    o = [int(i) for i in o_ids if i >= 0]
    g = [int(i) for i in g_ids if i >= 0]
    if not o:
        return set(), set(g)
    kth = min(score_of(i) for i in o)
    band = rel * abs(kth)
    keep = lambda i: abs(score_of(i) - kth) > band  # noqa: E731
    return {i for i in o if keep(i)}, {i for i in g if keep(i)}


def assert_selection_matches(o_scores_row, o_ids, g_ids, id_to_col=None, what=""):
    """GPU and oracle top-K agree outside the near-tie band; both have the same size."""
    col = (lambda i: id_to_col[i]) if id_to_col is not None else (lambda i: i)
    score_of = lambda i: o_scores_row[col(i)]  # noqa: E731
    o_n = int((np.asarray(o_ids) >= 0).sum())
    g_n = int((np.asarray(g_ids) >= 0).sum())
    assert o_n == g_n, f"{what}: selected {g_n}, oracle {o_n}"
    go = [int(i) for i in g_ids if i >= 0]
    assert len(set(go)) == len(go), f"{what}: duplicate ids"
    a, b = band_sets(score_of, o_ids, g_ids)
    assert a == b, f"{what}: {len(a ^ b)} ids differ outside the tie band"
    return set(int(i) for i in o_ids if i >= 0) == set(go)


def _log(msg):
    print(msg, flush=True)


def compare_workload(wl, res_g, res_o, what):
    """Layer-by-layer comparison of a GPU run with the oracle: selections as sets
    (near-tie band excluded), ascending order, pools; attention on the rows whose
    selection (and inherited selection) agrees exactly."""
    n_exact = n_rows = 0
    for li, (g, o) in enumerate(zip(res_g, res_o)):
        L = wl.layers[li]
        B, nq = L.q.shape[0], L.q.shape[1]
        if L.mode in ("F", "R"):
            for b in range(B):
                for q in range(nq):
                    if L.mode == "F":
                        same = assert_selection_matches(o["scores"][b, q], o["idx"][b, q], g["idx"][b, q],
                                                        what=f"{what} L{li} b{b}")
                    else:
                        pool_ids = res_o[last_full(wl, li)]["pool"][b, q]
                        id_to_col = {int(e): j for j, e in enumerate(pool_ids) if e >= 0}
                        same = assert_selection_matches(o["scores"][b, q], o["idx"][b, q], g["idx"][b, q],
                                                        id_to_col=id_to_col, what=f"{what} L{li} b{b}")
                    assert (np.diff(g["idx"][b, q][g["idx"][b, q] >= 0]) > 0).all(), "idx not ascending"
                    n_rows += 1
                    n_exact += same
        if o.get("pool") is not None and g.get("pool") is not None:
            for b in range(B):
                for q in range(nq):
                    assert_selection_matches(o["scores"][b, q], o["pool"][b, q], g["pool"][b, q],
                                             what=f"{what} L{li} pool b{b}")
                    gp = g["pool"][b, q]
                    nv = int((gp >= 0).sum())
                    assert (gp[nv:] == -1).all() and (np.diff(gp[:nv]) > 0).all(), "pool not ascending, -1 tail"
    # attention: every row. Where the GPU's selection (or the selection it
    # inherits) equals the oracle's, against the oracle's own layer output; where
    # it differs inside the tie band, against the oracle's attention over the
    # GPU's selection (same q, window and positions), so no row goes unchecked.
    _log(f"{what}: {n_exact}/{n_rows} selections identical")
    for li, (g, o) in enumerate(zip(res_g, res_o)):
        L = wl.layers[li]
        src = li
        while wl.layers[src].mode == "U":
            src -= 1
        same = (res_g[src]["idx"] == res_o[src]["idx"]).all(axis=-1)
        o_out, o_lse = o["out"], o["lse"]
        if not same.all():
            r_out, r_lse, _ = oracle_attend(wl.caches[L.cache_id], res_g[src]["idx"], L.q, L.win, wl.q_pos,
                                            wl.sm_scale)
            o_out = np.where(same[..., None, None], o_out, r_out)
            o_lse = np.where(same[..., None], o_lse, r_lse)
        assert_attention_close(g["out"], g["lse"], o_out, o_lse, f"{what} L{li}")


def oracle_attend(cache, idx, q, win, q_pos, sm_scale):
    import oracle  # test infrastructure
    return oracle.sparse_attend(cache, idx, q, win, q_pos=q_pos, sm_scale=sm_scale)


def last_full(wl, li):
    while wl.layers[li].mode != "F":
        li -= 1
    return li
