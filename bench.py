"""Benchmark of the CSA2 decode hot path on one MI355X.

One step = one decode step of the 1M-context workload: batch 8, 1,048,576
tokens of context per request (262,144 compressed entries), layers
[Full, Reindex, Reuse x4] with top-K 2048, a 16,384-entry candidate pool and a
128-token FP8 window per layer. Inputs are seeded and synthetic and resident
in HBM before timing; the step's inputs are rotated over several device
copies so the 256 MB Infinity Cache cannot hold one step's data for the next.
Steps are timed eager and replayed from one HIP graph that holds every timed
step; the better of the two is the value. eager_host_ms_per_step is the
host's time to enqueue one eager step: where it is below the step time, the
host runs ahead of the GPU and both modes wait on the same kernel sequence.

Beside it, under "workloads", the other benchmark workloads are measured the
same way with two input copies and ten steps: the 128K-context batch-32
[Full, Reuse x5] step, the 4096-query prefill chunk, the ragged 64-request
20-layer stack and the speculative step (8 x 6 query rows at 1M). --workload
makes another workload the JSON line's own.

Printed: one JSON line (metric, value = queries/s (tokens/s for the prefill
chunk), CPU-oracle baseline with the host's CPU model and a one-thread timing
of the tiny workload, two measured ceilings beside the 8 TB/s datasheet
figure -- a 1 GiB device copy (read + write) and a 2 GiB read-only stream --,
and rooflines measured live with HIP events around back-to-back calls replayed
from one HIP graph on the stream they run on: `roofline` for the kernel that
takes the most step time, the attention call (k_attend_seg, or k_attend_wave
where every workgroup takes a long range of units, and their merge),
and `roofline_scoring` for the indexer scoring kernel (HBM-bound in decode;
in the prefill chunk the kernel that scores and selects without a score
matrix, against the fp16 matrix-core peak)).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
WORKLOAD = "b8_1m_full_reindex_reuse4"
WORKLOAD_128K = "b32_128k_full_reuse5"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_index_score_b8_1m.json")
SCORE_SRC = os.path.join(ROOT, "compressed_sparse_attention_06_amd", "csrc", "k_score.hip")
ATT_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attend_b8_1m.json")
# the sources an attention traffic record was taken from (kernel + shared helpers)
ATT_SRC = [os.path.join(ROOT, "compressed_sparse_attention_06_amd", "csrc", f)
           for f in ("k_attend.hip", "attend_common.h", "csa2_dev.h")]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--copies", type=int, default=5, help="device copies of the inputs, rotated per step")
    p.add_argument("--kernel-iters", type=int, default=50)
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--skip-cpu", action="store_true")
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--copy-probe-mb", type=int, default=0,
                   help="also run a plain device copy of this size (counter calibration)")
    p.add_argument("--workload", default=WORKLOAD,
                   choices=[WORKLOAD, WORKLOAD_128K, "ragged64_paged_20layer", "prefill_4096q_128k",
                            "b8_1m_spec6"],
                   help="the workload of the JSON line (default: the 1M-context decode step)")
    p.add_argument("--no-topk-compare", action="store_true",
                   help="skip the standalone top-K comparison against torch.topk")
    p.add_argument("--no-secondary", action="store_true",
                   help="skip the other workloads reported beside the main one")
    p.add_argument("--attend-variants", action="store_true",
                   help="after the main workload, 5 attention calls each with (a) its first layer's "
                        "selection, (b) a selection of 512 runs of 4 consecutive entries per row (four "
                        "entries share each 128-byte line of scale bytes), (c) (a) without the window: "
                        "the inputs of the per-array traffic breakdown taken with counters")
    return p.parse_args()


def step_bytes(wl) -> int:
    """Algorithmic HBM bytes of one step (every byte the method must move once).

    Per request with N entries, K = min(k, N), P = min(pool, N):
      Full    = 36N + 160 + 4P + A(K)
      Reindex = 40P + 160 + A(K)
      Reuse   = A(K)
      A(K)    = 292K + window + 32768 + 32832
    (36 B indexer key per scored entry, 160 B indexer query + weights, 4 B per
    pool id written, 40 B per pool entry rescored incl. its id, 288 B main-KV
    row + 4 B id per selected entry, window rows, 32 KB fp32 query, 32 KB
    output + 64 B lse.)
    """
    if wl.q_pos is not None:
        return prefill_bytes(wl)
    total = 0
    for li, L in enumerate(wl.layers):
        c = wl.caches[L.cache_id]
        for b in range(wl.batch):
            N = int(c.n_entries[b])
            K, P = min(wl.k, N), min(wl.pool, N)
            win = int(L.win.length[b]) * (512 + (4 if L.win.row_scale is not None else 0))
            A = 292 * K + win + 32768 + 32832
            if L.mode == "F":
                total += 36 * N + 160 + 4 * P + A
            elif L.mode == "R":
                total += 40 * P + 160 + A
            else:
                total += A
    return total * wl.nq


def prefill_bytes(wl) -> int:
    """Algorithmic bytes when each request has several query rows with their own
    positions (a prefill chunk, or the drafts of a speculative step): each
    request's indexer keys once (36 B per entry, shared by its queries), and per
    query row 160 B of indexer query and weights, 4 B per pool id written (Full)
    or 40 B per pool entry rescored (Reindex), plus A(K), per layer."""
    total = 0
    for L in wl.layers:
        c = wl.caches[L.cache_id]
        for b in range(wl.batch):
            N = int(c.n_entries[b])
            K, P = min(wl.k, N), min(wl.pool, N)
            A = 292 * K + wl.window * (512 + (4 if L.win.row_scale is not None else 0)) + 32768 + 32832
            if L.mode == "F":
                total += 36 * N + wl.nq * (160 + 4 * P + A)
            elif L.mode == "R":
                total += wl.nq * (40 * P + 160 + A)
            else:
                total += wl.nq * A
    return total


def attend_bytes(wl, li) -> int:
    """Algorithmic bytes of one attention call of layer li: A(K) per query row
    (292 B per selected entry incl. its id, the window rows it scans, 32 KB fp32
    query, 32 KB output + 64 B lse)."""
    L = wl.layers[li]
    c = wl.caches[L.cache_id]
    total = 0
    for b in range(wl.batch):
        K = min(wl.k, int(c.n_entries[b]))
        if wl.q_pos is not None:
            win = wl.window * (512 + (4 if L.win.row_scale is not None else 0))
        else:
            win = int(L.win.length[b]) * (512 + (4 if L.win.row_scale is not None else 0))
        total += wl.nq * (292 * K + win + 32768 + 32832)
    return total


def attend_flops(wl, li) -> int:
    """Useful matrix flops of one attention call of layer li: per query row and
    attended row (selected entries, then window rows), 16 heads x 512 channels
    x 2 for QK^T and x 2 for P.V."""
    L = wl.layers[li]
    c = wl.caches[L.cache_id]
    total = 0
    for b in range(wl.batch):
        K = min(wl.k, int(c.n_entries[b]))
        win = wl.window if wl.q_pos is not None else int(L.win.length[b])
        total += wl.nq * (K + win) * 16 * 512 * 4
    return total


def cpu_model() -> str:
    """The host CPU's model name (first "model name" line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def prefill_score_flops(wl) -> int:
    """Useful flops of one prefill scoring launch: 4 heads x 64 channels x 2 per
    visible (query, entry) pair (entry s visible at position p iff 4(s+1) <= p+1)."""
    c = wl.caches[0]
    vis = 0
    for b in range(wl.batch):
        v = np.minimum((wl.q_pos[b].astype(np.int64) + 1) // 4, int(c.n_entries[b]))
        vis += int(np.maximum(v, 0).sum())
    return vis * 4 * 64 * 2


def score_kernel_bytes(wl) -> int:
    """Algorithmic bytes of one launch of the Full-layer scoring kernel: 36 B per
    entry of each request (once, whatever its number of query rows) + 160 B of
    indexer query and weights per query row."""
    c = wl.caches[0]
    return int(sum(36 * int(n) + 160 * wl.nq for n in c.n_entries))


def upload_chains(wl, n_copies, dev):
    """Device copies of a workload's inputs and the chained LayerCalls of each copy."""
    import numpy as np
    import torch

    import compressed_sparse_attention_06_amd as csa2

    def up(a):
        if a is None:
            return None
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    host = dict(caches=[], layers=[])
    for c in wl.caches:
        host["caches"].append(dict(kv_codes=up(c.kv_codes), kv_scales=up(c.kv_scales),
                                   ix_codes=up(c.ix_codes), ix_scales=up(c.ix_scales),
                                   block_table=up(c.block_table), n_entries=up(c.n_entries)))
    for L in wl.layers:
        host["layers"].append(dict(q=up(L.q), win_codes=up(L.win.codes), win_len=up(L.win.length),
                                   win_pos0=up(L.win.pos0), win_rs=up(L.win.row_scale),
                                   qix_codes=up(L.qix_codes), qix_scales=up(L.qix_scales), w=up(L.w)))
    q_pos = up(wl.q_pos)
    copies = []
    for ci in range(n_copies):
        cl = (lambda x: x) if ci == 0 else (lambda x: None if x is None else x.clone())
        caches = [csa2.Cache(**{k: cl(v) for k, v in c.items()}) for c in host["caches"]]
        layers = [{k: cl(v) for k, v in L.items()} for L in host["layers"]]
        copies.append((caches, layers))
    torch.cuda.synchronize()
    k, pool = wl.k, wl.pool

    def build_chain(caches, layers):
        calls, last_idx, last_pool = [], None, None
        for li, Lh in enumerate(wl.layers):
            L = layers[li]
            cache = caches[Lh.cache_id]
            win = csa2.Window(codes=L["win_codes"], length=L["win_len"], pos0=L["win_pos0"],
                              row_scale=L["win_rs"], window=wl.window)
            if Lh.mode == "F":
                c = csa2.LayerCall("F", cache, win, L["q"], k, pool=pool, qix_codes=L["qix_codes"],
                                   qix_scales=L["qix_scales"], w=L["w"], q_pos=q_pos, sm_scale=wl.sm_scale)
                last_idx, last_pool = c.idx_out, c.pool_out
            elif Lh.mode == "R":
                c = csa2.LayerCall("R", cache, win, L["q"], k, pool=pool, qix_codes=L["qix_codes"],
                                   qix_scales=L["qix_scales"], w=L["w"], idx_in=last_pool, q_pos=q_pos,
                                   sm_scale=wl.sm_scale)
                last_idx = c.idx_out
            else:
                c = csa2.LayerCall("U", cache, win, L["q"], k, idx_in=last_idx, q_pos=q_pos,
                                   sm_scale=wl.sm_scale)
            calls.append(c)
        return calls

    return copies, [build_chain(*cp) for cp in copies]


def time_steps(chains, steps, warmup, use_graph):
    """Seconds for `steps` steps, eager and (optionally) replayed from HIP graphs.

    The timed graph holds all `steps` steps (rotating over the input copies) and
    is replayed once, after one replay of a graph of the warm-up steps: every
    graph launch costs a fixed few microseconds on the GPU (measured at 1M with
    two copies: one step per graph 162.6 us/step, five per graph 153.5, eager
    156.3), which a graph per step would charge to every step."""
    import torch

    def run_step(i):
        for c in chains[i % len(chains)]:
            c()

    for i in range(warmup):
        run_step(i)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i in range(steps):
        run_step(i)
    host_s = time.perf_counter() - w0  # every launch enqueued: the host's share
    torch.cuda.synchronize()
    eager_s = time.perf_counter() - w0
    graph_s = None
    if use_graph:
        try:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                for ci in range(len(chains)):
                    run_step(ci)
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()

            def capture(n):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for i in range(n):
                        run_step(i)
                return g

            g_warm = capture(max(1, warmup))
            g_main = capture(steps)
            torch.cuda.synchronize()
            g_warm.replay()
            torch.cuda.synchronize()
            w0 = time.perf_counter()
            g_main.replay()
            torch.cuda.synchronize()
            graph_s = time.perf_counter() - w0
            del g_warm, g_main
        except Exception as e:  # capture unsupported: report eager only
            log(f"graph capture failed: {e!r}")
            graph_s = None
    return eager_s, graph_s, host_s


def src_sha256(src):
    """sha256 of a source file, or of the concatenation of a list of them."""
    h = hashlib.sha256()
    for f in ([src] if isinstance(src, str) else src):
        h.update(open(f, "rb").read())
    return h.hexdigest()


def traffic_of(path, src, name):
    """Calibrated counter bytes per launch from a profiles/ record, while the
    kernel source it was taken from is unchanged and the workload matches."""
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        src_hash = src_sha256(src)
        if rec.get("kernel_source_sha256") == src_hash and rec.get("workload") == name:
            return rec.get("bytes_per_launch")
    except Exception:
        return None
    return None


def measure_workload(wl, name, n_copies, steps, warmup, kernel_iters, use_graph, dev):
    """One workload's step time (eager and graph-replayed), its indexer-scoring
    kernel and its first layer's attention call, each timed live with HIP events
    around back-to-back calls replayed from one HIP graph. Returns (result dict,
    device copies, chains) so that the caller can reuse the uploaded inputs."""
    import torch

    import compressed_sparse_attention_06_amd as csa2

    prefill = wl.q_pos is not None and wl.nq >= 64
    copies, chains = upload_chains(wl, n_copies, dev)
    log(f"{name}: inputs on device, {n_copies} copies, {torch.cuda.memory_allocated() / 2**30:.2f} GiB allocated")
    B, nq, k = wl.batch, wl.nq, wl.k
    eager_s, graph_s, host_s = time_steps(chains, steps, warmup, use_graph)
    log(f"{name}: eager {eager_s / steps * 1e3:.4f} ms/step" +
        ("" if graph_s is None else f"; graph {graph_s / steps * 1e3:.4f} ms/step"))
    best_s = min(x for x in (eager_s, graph_s) if x is not None)
    sbytes = step_bytes(wl)

    qp = None if wl.q_pos is None else torch.from_numpy(wl.q_pos).to(dev)
    if prefill:
        topk_calls = [csa2.IndexTopkCall(caches[0], layers[0]["qix_codes"], layers[0]["qix_scales"],
                                         layers[0]["w"], k, q_pos=qp) for caches, layers in copies]

        def score_once(i):
            topk_calls[i % len(topk_calls)]()
    else:
        scores = torch.empty(B, nq, copies[0][0][0].capacity, dtype=torch.float32, device=dev)
        hist = torch.zeros(B, nq, 4096, dtype=torch.int32, device=dev)

        def score_once(i):
            caches, layers = copies[i % len(copies)]
            csa2.index_score(caches[0], layers[0]["qix_codes"], layers[0]["qix_scales"], layers[0]["w"],
                             q_pos=qp, out=scores, hist=hist)

    k_ms = time_calls(score_once, kernel_iters) * 1e-3
    if prefill:
        kflops = prefill_score_flops(wl)
        k_tflops = kflops / (k_ms * 1e-3) / 1e12
        log(f"{name}: prefill scoring + top-k kernel {k_ms * 1e3:.2f} us/launch, {k_tflops:.1f} TFLOP/s")
        rs = {"kernel": "k_prefill_topk (prefill-chunk indexer scoring fused with the per-query top-K: "
                        "two fp16-MFMA scoring passes and the selection; achieved = one pass's useful "
                        "flops per launch time)", "bound": "mfma",
              "achieved": round(k_tflops, 1), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
              "frac": round(k_tflops / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None,
              "flops_per_launch": kflops, "us_per_launch": round(k_ms * 1e3, 3)}
    else:
        kb = score_kernel_bytes(wl)
        k_gbps = kb / (k_ms * 1e-3) / 1e9
        log(f"{name}: index_score kernel {k_ms * 1e3:.2f} us/launch, {k_gbps:.0f} GB/s algorithmic")
        rs = {"kernel": ("k_index_score_mq (several query rows per request share each key read) + k_hist"
                         if nq > 1 else "k_index_score (Full-layer lightning-indexer scoring)"),
              "bound": "hbm", "achieved": round(k_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
              "frac": round(k_gbps / HBM_PEAK_GBPS, 4),
              "traffic": traffic_of(TRAFFIC_FILE, SCORE_SRC, name),
              "bytes_per_launch": kb, "us_per_launch": round(k_ms * 1e3, 3)}

    # the dominant kernel by step time: attention (k_attend_seg or k_attend_wave + the merge) of the
    # first layer, called with that layer's selection
    li0 = 0
    att_args = []
    for ci, (caches, layers) in enumerate(copies):
        Lh, L = wl.layers[li0], layers[li0]
        win = csa2.Window(codes=L["win_codes"], length=L["win_len"], pos0=L["win_pos0"],
                          row_scale=L["win_rs"], window=wl.window)
        idx = chains[ci][li0].idx_out
        out = torch.empty_like(L["q"])
        lse = torch.empty(L["q"].shape[:3], dtype=torch.float32, device=dev)
        wcap = win.span(qp)
        ws = csa2.alloc_workspace(csa2.workspace_bytes("U", B, nq, 0, k, 0, wcap), dev)
        att_args.append((caches[Lh.cache_id], idx, L["q"], win, out, lse, ws))

    def attend_once(i):
        cache, idx, q, win, out, lse, ws = att_args[i % len(att_args)]
        csa2.sparse_attend(cache, idx, q, win, q_pos=qp, sm_scale=wl.sm_scale, out=out, lse=lse, ws=ws)

    att_ms = time_calls(attend_once, kernel_iters) * 1e-3
    att_b = attend_bytes(wl, li0)
    att_gbps = att_b / (att_ms * 1e-3) / 1e9
    att_f = attend_flops(wl, li0)
    att_tflops = att_f / (att_ms * 1e-3) / 1e12
    log(f"{name}: attention call {att_ms * 1e3:.2f} us/launch, {att_gbps:.0f} GB/s algorithmic, "
        f"{att_tflops:.0f} TFLOP/s useful")
    # decode attention streams its gathered rows from HBM; the prefill chunk's
    # 4096 queries gather from a 9.4 MB cache that stays in the on-chip caches,
    # so there the matrix cores are the roofline
    if prefill:
        ra = {"kernel": "csa2_sparse_attend: k_attend_wave (paired waves; first layer's selection; no merge: "
                        "every row falls whole to one workgroup)",
              "bound": "mfma", "achieved": round(att_tflops, 1), "peak": MFMA_F16_PEAK_TFLOPS,
              "unit": "TFLOP/s", "frac": round(att_tflops / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None,
              "flops_per_launch": att_f, "bytes_per_launch": att_b, "us_per_launch": round(att_ms * 1e3, 3)}
    else:
        ra = {"kernel": "csa2_sparse_attend: k_attend_seg + k_merge_seg (first layer's selection)",
              "bound": "hbm", "achieved": round(att_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
              "frac": round(att_gbps / HBM_PEAK_GBPS, 4),
              "traffic": traffic_of(ATT_TRAFFIC_FILE, ATT_SRC, name),
              "bytes_per_launch": att_b, "flops_per_launch": att_f, "us_per_launch": round(att_ms * 1e3, 3)}

    rows = B * nq
    res = dict(workload=name, batch=B, queries_per_request=nq, context_tokens=int(wl.contexts.max()),
               layers=wl.modes, input_copies=n_copies, steps=steps, warmup=warmup,
               value=round(rows * steps / best_s, 1),
               unit="tokens/s" if prefill else "queries/s",
               ms_per_step=round(best_s / steps * 1e3, 4),
               step_gbps=round(sbytes / (best_s / steps) / 1e9, 1),
               step_pct_of_peak=round(100 * sbytes / (best_s / steps) / 1e9 / HBM_PEAK_GBPS, 2),
               step_algorithmic_bytes=sbytes,
               eager_ms_per_step=round(eager_s / steps * 1e3, 4),
               eager_host_ms_per_step=round(host_s / steps * 1e3, 4),
               graph_ms_per_step=None if graph_s is None else round(graph_s / steps * 1e3, 4),
               timing="graph" if (graph_s is not None and graph_s <= eager_s) else "eager",
               roofline=ra, roofline_scoring=rs)
    return res, copies, chains


_EV = None


def time_calls(fn, iters):
    """us per call: `iters` calls captured in one HIP graph and replayed between two
    HIP events on the stream the graph runs on (torch's current stream), so that
    the binding's per-call host work is not what is timed."""
    import torch

    global _EV
    if _EV is None:
        _EV = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    ev0, ev1 = _EV
    for i in range(3):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_cap):
        with torch.cuda.graph(g, stream=s_cap):
            for i in range(iters):
                fn(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    ev0.record()
    g.replay()
    ev1.record()
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / iters * 1e3


def stream_probes(dev):
    """Practical HBM ceilings measured in the same run: a plain 1 GiB device copy
    (read + write) and a 2 GiB read-only stream (csa2_stream_read, several grid
    sizes, the best kept), both event-timed; neither fits the 256 MB Infinity Cache."""
    import torch

    import compressed_sparse_attention_06_amd as csa2

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nb = 1 << 30
    xs = torch.empty(nb, dtype=torch.uint8, device=dev)
    ys = torch.empty_like(xs)
    for _ in range(2):
        ys.copy_(xs)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        ys.copy_(xs)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * nb * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del xs, ys
    nr = 2 << 30
    xr = torch.ones(nr // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)
    read = {}
    for blocks in (2048, 8192, 16384, 32768):
        for _ in range(2):
            csa2.stream_read(xr, sink, blocks)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(10):
            csa2.stream_read(xr, sink, blocks)
        e1.record()
        torch.cuda.synchronize()
        read[blocks] = nr * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del xr, sink
    best = max(read, key=read.get)
    log(f"stream copy: {copy_gbps:.0f} GB/s (read + write, 1 GiB); stream read: "
        + ", ".join(f"{b} WGs {g:.0f}" for b, g in read.items()) + " GB/s (2 GiB)")
    return copy_gbps, read[best], best


def add_ceilings(res, copy_gbps, read_gbps):
    """The step's and each HBM roofline's rate against the measured ceilings."""
    g = res["step_gbps"]
    res["step_pct_of_stream_copy"] = round(100 * g / copy_gbps, 2)
    res["step_pct_of_stream_read"] = round(100 * g / read_gbps, 2)
    for key in ("roofline", "roofline_scoring"):
        r = res.get(key)
        if r and r["unit"] == "GB/s":
            r["frac_of_stream_copy"] = round(r["achieved"] / copy_gbps, 4)
            r["frac_of_stream_read"] = round(r["achieved"] / read_gbps, 4)


EXTRA_WORKLOADS = [WORKLOAD_128K, "prefill_4096q_128k", "ragged64_paged_20layer", "b8_1m_spec6"]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(decode requests shard by batch with no exchange between GPUs)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import compressed_sparse_attention_06_amd as csa2
    from synth import make_decode_workload, make_prefill_workload, take_queries, take_requests

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    csa2.lib()
    name = args.workload
    prefill = name == "prefill_4096q_128k"
    t0 = time.time()
    wl = make_prefill_workload() if prefill else make_decode_workload(name)
    log(f"workload {name} generated in {time.time() - t0:.1f}s; modes {wl.modes}, "
        f"batch {wl.batch}, queries/request {wl.nq}, N/request {int(wl.caches[0].n_entries[0])}")
    main_res, copies, chains = measure_workload(wl, name, args.copies, args.steps, args.warmup,
                                                args.kernel_iters, not args.no_graph, dev)
    B, nq, k, pool = wl.batch, wl.nq, wl.k, wl.pool
    gen = torch.Generator(device=dev).manual_seed(11)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # ---- the cache's write side: what one decode step appends, and a prefill chunk's worth ----
    gen = torch.Generator(device=dev).manual_seed(11)
    cache0 = copies[0][0][0]
    app = {}
    for label, n_req, n_new in (("decode_step", B, 1), ("prefill_chunk", 1, 1024)):
        kv_new = torch.randn(n_req, n_new, 512, device=dev, generator=gen)
        ix_new = torch.randn(n_req, n_new, 64, device=dev, generator=gen)
        # the last n_new entries of each request are rewritten (distinct slots; entries
        # whose page does not exist are skipped by the kernel)
        base = torch.clamp(cache0.n_entries[:n_req, None] - n_new, min=0)
        ent = (base + torch.arange(n_new, device=dev, dtype=torch.int32)[None, :]).to(torch.int32).contiguous()
        tok = torch.randn(n_req, 4 * n_new, 512, device=dev, generator=gen)
        wcodes = torch.zeros(n_req, max(128, 4 * n_new), 512, dtype=torch.uint8, device=dev)
        wrs = torch.ones(n_req, wcodes.shape[1], dtype=torch.float32, device=dev)
        wrow = (torch.arange(4 * n_new, device=dev, dtype=torch.int32)[None, :] % wcodes.shape[1]).repeat(n_req, 1).contiguous()
        qx = torch.randn(n_req, 1, 4, 64, device=dev, generator=gen)
        qxc = torch.empty(n_req, 1, 4, 32, dtype=torch.uint8, device=dev)
        qxs = torch.empty(n_req, 1, 4, 4, dtype=torch.uint8, device=dev)
        us_kv = time_calls(lambda i: csa2.kv_append(cache0, kv_new, ent, ix=ix_new), 20)
        us_win = time_calls(lambda i: csa2.window_append(wcodes, tok, wrow, row_scale=wrs), 20)
        us_q = time_calls(lambda i: csa2.quantize_fp4(qx, qxc, qxs), 20)
        nbytes = n_req * n_new * (576 * 4 + 324) + n_req * 4 * n_new * (512 * 4 + 516)
        app[label] = dict(requests=n_req, entries_per_request=n_new, tokens_per_request=4 * n_new,
                          kv_append_us=round(us_kv, 2), window_append_us=round(us_win, 2),
                          qix_quantize_us=round(us_q, 2), algorithmic_bytes=nbytes,
                          gbps=round(nbytes / ((us_kv + us_win) * 1e-6) / 1e9, 1))
    log(f"append: {app}")

    # ---- standalone top-K against torch.topk on the same scores (event-timed calls) ----
    topk_cmp = []
    if not args.no_topk_compare:
        for rows, n, kk in ((8, 262144, 2048), (8, 16384, 2048), (32, 32768, 2048),
                            (64, 16384, 2048), (4096, 32768, 2048)):
            sc = torch.randn(rows, 1, n, device=dev, generator=gen)
            out_i = torch.empty(rows, 1, kk, dtype=torch.int32, device=dev)
            wsk = csa2.alloc_workspace(csa2.workspace_bytes("R", rows, 1, n, kk), dev)
            tv = torch.empty(rows, 1, kk, device=dev)
            ti = torch.empty(rows, 1, kk, dtype=torch.int64, device=dev)
            iters = 10 if rows * n > 1e8 else 30

            def ours(i):
                csa2.topk(sc, kk, out=out_i, ws=wsk)

            def theirs(i):
                torch.topk(sc, kk, dim=-1, sorted=False, out=(tv, ti))

            res = {}
            for nm, fn in (("csa2_topk", ours), ("torch_topk", theirs)):
                for i in range(3):
                    fn(i)
                torch.cuda.synchronize()
                ev0.record()
                for i in range(iters):
                    fn(i)
                ev1.record()
                torch.cuda.synchronize()
                res[nm] = ev0.elapsed_time(ev1) / iters * 1e3
            same = bool((torch.sort(ti, dim=-1).values.to(torch.int32) == out_i).all().item())
            topk_cmp.append(dict(rows=rows, n=n, k=kk, csa2_us=round(res["csa2_topk"], 1),
                                 torch_us=round(res["torch_topk"], 1),
                                 speedup=round(res["torch_topk"] / res["csa2_topk"], 2), same_ids=same))
            del sc, out_i, wsk, tv, ti
        log(f"topk vs torch.topk: {topk_cmp}")

    if args.copy_probe_mb:
        n = args.copy_probe_mb * 2**20
        x = torch.empty(n, dtype=torch.uint8, device=dev)
        y = torch.empty_like(x)
        for _ in range(5):
            y.copy_(x)
        # the same copy through an elementwise kernel (16-byte vector loads and
        # stores per lane, like the library's kernels)
        xf, yf = x.view(torch.float32), y.view(torch.float32)
        xf.zero_()
        for _ in range(5):
            torch.mul(xf, 1.0, out=yf)
        torch.cuda.synchronize()
        log(f"copy probe: 5 x {args.copy_probe_mb} MiB device copies (blit) + 5 (elementwise)")

    # ---- attention input variants for the counter breakdown of its traffic ----
    if args.attend_variants and wl.q_pos is None:
        caches, layers = copies[0]
        L = layers[0]
        win = csa2.Window(codes=L["win_codes"], length=L["win_len"], pos0=None, row_scale=L["win_rs"],
                          window=wl.window)
        idx = chains[0][0].idx_out
        n_ent = int(wl.caches[0].n_entries.min())
        rng = np.random.default_rng(0)
        runs = np.stack([np.sort(4 * rng.choice(n_ent // 4, k // 4, replace=False)[:, None] + np.arange(4)[None, :],
                                 axis=None) for _ in range(B * nq)])
        idx_cl = torch.from_numpy(runs.reshape(B, nq, k).astype(np.int32)).to(dev)
        out = torch.empty_like(L["q"])
        lse = torch.empty(L["q"].shape[:3], dtype=torch.float32, device=dev)
        wsv = csa2.alloc_workspace(csa2.workspace_bytes("U", B, nq, 0, k, 0, win.span(None)), dev)
        for vi, (vidx, vwin) in enumerate(((idx, win), (idx_cl, win), (idx, None))):
            for _ in range(5):
                csa2.sparse_attend(caches[0], vidx, L["q"], vwin, sm_scale=wl.sm_scale, out=out, lse=lse, ws=wsv)
        torch.cuda.synchronize()
        log("attention variants: 5 calls each of (a) the selection, (b) runs of 4 consecutive entries, "
            "(c) the selection without the window (the last 15 attention dispatches)")

    # ---- the other workloads beside the main one (two input copies each, fewer steps) ----
    extras = {}
    if not args.no_secondary:
        del chains, copies
        torch.cuda.empty_cache()
        for xname in EXTRA_WORKLOADS:
            if xname == name:
                continue
            t0 = time.time()
            xwl = make_prefill_workload() if xname == "prefill_4096q_128k" else make_decode_workload(xname)
            log(f"workload {xname} generated in {time.time() - t0:.1f}s")
            xs_steps = min(args.steps, 10)
            xres, xc, xch = measure_workload(xwl, xname, min(args.copies, 2), xs_steps, min(args.warmup, 3),
                                             min(args.kernel_iters, 10), not args.no_graph, dev)
            extras[xname] = xres
            log(f"{xname}: {xres['ms_per_step']} ms/step, {xres['value']} {xres['unit']}")
            del xc, xch, xwl
            torch.cuda.empty_cache()

    # ---- measured ceilings: stream copy (read + write) and read-only stream ----
    copy_gbps, read_gbps, read_blocks = stream_probes(dev)
    add_ceilings(main_res, copy_gbps, read_gbps)
    for xres in extras.values():
        add_ceilings(xres, copy_gbps, read_gbps)

    # ---- CPU oracle baseline (bounded sample, host cores) ----
    cpu = None
    if not args.skip_cpu:
        import oracle
        # a bounded sample of the same workload: all requests (decode), a few
        # requests of the ragged stack, or a few query rows of the prefill chunk
        if prefill:
            sample_wl, what = take_queries(wl, range(16)), "16 of the 4096 query rows of the prefill chunk"
        elif wl.batch > 8:
            sample_wl, what = take_requests(wl, range(8)), f"8 of the {wl.batch} requests"
        else:
            sample_wl, what = wl, f"all {wl.batch} requests"
        sq = sample_wl.batch * sample_wl.nq
        reps, t_cpu = 0, 0.0
        w0 = time.perf_counter()
        while reps == 0 or (time.perf_counter() - w0) < args.cpu_seconds:
            oracle.run_workload(sample_wl)
            reps += 1
        t_cpu = time.perf_counter() - w0
        cores = min(oracle.num_threads(), len(os.sched_getaffinity(0)))
        cpu = dict(value=round(sq * reps / t_cpu, 3), unit="queries/s", cores=cores, kind="oracle",
                   sample=f"the whole {len(wl.layers)}-layer step of {what}, repeated {reps}x "
                          f"({t_cpu:.1f}s); fp64 C oracle, OpenMP over query rows",
                   cpu_model=cpu_model())
        # one thread on the tiny workload (1 request, 8192 tokens, one Full layer, top-256)
        tiny = make_decode_workload("tiny_b1_8k_full")
        oracle.set_num_threads(1)
        n1, w1 = 0, time.perf_counter()
        while n1 == 0 or time.perf_counter() - w1 < 1.0:
            oracle.run_workload(tiny)
            n1 += 1
        t1 = time.perf_counter() - w1
        oracle.set_num_threads(cores)
        cpu["single_thread_tiny"] = {"value": round(n1 / t1, 2), "unit": "queries/s",
                                     "workload": "tiny_b1_8k_full", "repeats": n1}
        log(f"cpu oracle: {cpu['value']} queries/s on {cores} threads; "
            f"1 thread on the tiny workload: {cpu['single_thread_tiny']['value']} queries/s")

    line = {
        "metric": "CSA2 decode queries/s + achieved HBM GB/s (% of peak) at 128K and 1M ctx",
        "value": main_res["value"],
        "unit": main_res["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4/fp8 inputs; fp4 and f16 MFMA, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": name, "batch": B, "queries_per_request": nq,
                   "context_tokens": int(wl.contexts[0]),
                   "entries_per_request": int(wl.caches[0].n_entries[0]), "layers": wl.modes,
                   "top_k": k, "pool": pool, "window": 128, "input_copies": args.copies,
                   "timing": main_res["timing"]},
        "step_gbps": main_res["step_gbps"],
        "step_pct_of_peak": main_res["step_pct_of_peak"],
        "stream_copy_gbps": round(copy_gbps, 1),
        "stream_read_gbps": round(read_gbps, 1),
        "stream_read_workgroups": read_blocks,
        "step_pct_of_stream_copy": main_res["step_pct_of_stream_copy"],
        "step_pct_of_stream_read": main_res["step_pct_of_stream_read"],
        "step_algorithmic_bytes": main_res["step_algorithmic_bytes"],
        "eager_ms_per_step": main_res["eager_ms_per_step"],
        "eager_host_ms_per_step": main_res["eager_host_ms_per_step"],
        "graph_ms_per_step": main_res["graph_ms_per_step"],
        "roofline": main_res["roofline"],
        "roofline_scoring": main_res["roofline_scoring"],
        "append": app,
        "topk_vs_torch": topk_cmp,
        "cpu_baseline": cpu,
        "workloads": extras,
        "secondary": extras.get(WORKLOAD_128K),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
