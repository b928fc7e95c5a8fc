// C ABI of the CSA2 decode library: argument checks, workspace layout and the
// launch sequence of each entry point. Every check runs on the host and reads
// no device memory; nothing here allocates or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "../../include/csa2_probe.h"
#include "csa2_dev.h"
#include "kernels.h"

// Library-owned scratch of csa2_sparse_attend_noalloc: the attention's split
// partials for callers that cannot allocate. Host code never uses this name
// as an address (on the host it is only a stand-in for the symbol): the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[CSA2_NOALLOC_SCRATCH_BYTES];
static_assert(CSA2_NOALLOC_SCRATCH_BYTES == csa2::kSegMaxWg * 2 * CSA2_H * csa2::kPartStride * 4,
              "the scratch holds two partials for each of the attention's workgroups");

namespace {

thread_local char g_err[512] = "";

csa2_status fail(csa2_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

csa2_status hip_check(hipError_t e, const char *what) {
  if (e == hipSuccess) return CSA2_OK;
  return fail(CSA2_EHIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kFinItems = 4096;        // rows up to this length select in LDS directly
constexpr int kScoreChunk = 2048;      // scoring columns per workgroup (contiguous entries)
constexpr int kScoreChunkCand = 512;   // ... when gathering a candidate list
constexpr int32_t kPrefillQueries = 64;  // queries per request from which scoring is a matrix-core contraction

// Scoring as a dense queries x entries contraction (many queries of one
// request, every visible entry, pages of at least 16 entries).
bool use_prefill_scoring(int32_t nq, const int32_t *cand, int32_t page_size) {
  return nq >= kPrefillQueries && !cand && page_size >= 16;
}
constexpr int64_t kFusedTopkMinRows = 1024;  // query rows from which a prefill chunk selects without a score matrix

// A Full layer over a prefill chunk of enough query rows (so that 16 rows per
// workgroup fill the GPU), entries up to kPrefillTopkMaxCols and no pool:
// scoring and top-K run as one kernel that keeps no score matrix.
bool use_fused_topk(csa2_mode mode, int64_t batch, int32_t nq, int64_t n_cols, int32_t pool) {
  return mode == CSA2_FULL && pool == 0 && nq >= kPrefillQueries && batch * nq >= kFusedTopkMinRows &&
         n_cols >= 1 && n_cols <= csa2::kPrefillTopkMaxCols;
}
constexpr int64_t kMaxSelectCols = CSA2_MAX_SELECT_COLS;
static_assert(CSA2_MAX_SELECT_COLS <= SEL_MAX_WG * 8192, "the chunked selection takes SEL_MAX_WG chunks of 8192");

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Columns per selection chunk: the smallest of 2048, 4096, 8192 that cuts
// the row into at most SEL_MAX_WG chunks and keeps the final pass (one
// workgroup per chunk, row and target) within two workgroups per compute
// unit; when no size does (many rows), the size with the fewest workgroups.
int32_t select_chunk(int64_t n_cols, int64_t rows, int ntarget) {
  int32_t largest = 0;
  for (int32_t c = 2048; c <= 8192; c <<= 1) {
    const int64_t nwg = (n_cols + c - 1) / c;
    if (nwg > SEL_MAX_WG) continue;
    if (nwg * rows * ntarget <= 512) return c;
    largest = c;
  }
  return largest ? largest : 8192;
}

struct WsLayout {
  size_t scores = 0, hist = 0, zero_end = 0, info = 0, counts = 0, suf = 0, list0 = 0, list1 = 0, eq0 = 0,
         eq1 = 0, part = 0,
         total = 0;
  bool compact = false;   // chunked compaction + final selection (long rows)
  bool row_sel = false;   // one workgroup per row, keys in registers, histogram in LDS (rows up to kSelectRowMax)
  bool fused = false;     // prefill scoring fused with the top-K: no score region
  int max_wg = 0, chunk = 0;
  int64_t seg_stride = 0;
  // attention: units of 128 positions, U per row, T in all, over G workgroups
  int32_t att_U = 0, att_G = 0;
  int64_t att_T = 0;
  int32_t att_slots = 1;  // most workgroups sharing one row (2+: merge pass)
};

// Attention work split: each row's attention set (k entries, then the window
// from k rounded up to 16) in units of 128 positions, shared out evenly over
// at most one workgroup per compute unit. Workgroup w takes units
// [w T / G, (w + 1) T / G) of the T = rows x U in row order. With G a
// multiple of the row count (P workgroups per row), every workgroup's range
// lies inside one row: a workgroup whose range crosses a row boundary pays
// the second row's Q conversion and id -> page -> row chain as well, so such
// a G is taken whenever its largest range is no longer than that of the
// plain split over min(T, 256) workgroups, with the fewest workgroups per row
// that keep that length (fewer partials for the merge).
void attend_geometry(WsLayout &L, int64_t rows, int32_t k, int32_t win_cap) {
  const int64_t span = (((int64_t)k + 15) & ~(int64_t)15) + (win_cap > 0 ? win_cap : 0);
  L.att_U = (int32_t)((span + 127) / 128);
  L.att_T = rows * L.att_U;
  L.att_G = (int32_t)std::min<int64_t>(L.att_T, csa2::kSegMaxWg);
  if (rows >= 1 && rows <= csa2::kSegMaxWg) {
    const int64_t U = L.att_U;
    const int64_t longest = (L.att_T + L.att_G - 1) / L.att_G;  // units of the plain split's largest range
    int64_t P = std::min<int64_t>(U, csa2::kSegMaxWg / rows);
    const int64_t per = (U + P - 1) / P;
    if (per <= longest) {
      while (P > 1 && (U + P - 2) / (P - 1) == per) --P;
      L.att_G = (int32_t)(rows * P);
    }
  }
  const int64_t rows_n = L.att_T / L.att_U;
  auto owner = [&](int64_t u) { return ((u + 1) * L.att_G + L.att_T - 1) / L.att_T - 1; };
  L.att_slots = 1;
  for (int64_t r = 0; r < rows_n; ++r)
    L.att_slots = std::max<int32_t>(L.att_slots,
                                    (int32_t)(owner(r * L.att_U + L.att_U - 1) - owner(r * L.att_U) + 1));
}

WsLayout ws_layout(csa2_mode mode, int64_t rows, int64_t n_cols, int32_t k, int32_t win_cap, int ntarget,
                   bool fused = false) {
  WsLayout L;
  size_t off = 0;
  L.fused = fused;
  if ((mode == CSA2_FULL || mode == CSA2_REINDEX) && !fused) {
    // one workgroup per row pays off once there are enough rows to fill the
    // GPU; few long rows go through the chunked path, which spreads each row
    // over many workgroups
    L.row_sel = n_cols > kFinItems && n_cols <= csa2::kSelectRowMax;
    L.compact = n_cols > csa2::kSelectRowMax;
    L.scores = off;
    off = align256(off + (size_t)rows * n_cols * 4);
    L.hist = off;  // zeroed by a fill before the scoring kernel adds to it
    off += (size_t)rows * HIST_BINS * 4;
    L.zero_end = off;
    off = align256(off);
    if (L.compact) {
      L.chunk = select_chunk(n_cols, rows, ntarget);
      L.max_wg = (int)((n_cols + L.chunk - 1) / L.chunk);
      L.info = off;
      off = align256(off + (size_t)rows * 2 * 4 * 4);
      L.counts = off;
      off = align256(off + (size_t)rows * 2 * L.max_wg * 4);
      L.suf = off;
      off = align256(off + (size_t)rows * 2 * L.max_wg * 256 * 4);
      L.seg_stride = (int64_t)L.max_wg * L.chunk;
      L.list0 = off;
      off = align256(off + (size_t)rows * L.seg_stride * 8);
      L.list1 = off;
      off = align256(off + (size_t)rows * L.seg_stride * 8);
      L.eq0 = off;
      off = align256(off + (size_t)rows * L.seg_stride * 8);
      L.eq1 = off;
      off = align256(off + (size_t)rows * L.seg_stride * 8);
    }
  }
  attend_geometry(L, rows, k, win_cap);
  L.part = off;  // two partials per workgroup
  if (L.att_slots > 1) off = align256(off + (size_t)L.att_G * 2 * CSA2_H * csa2::kPartStride * 4);
  L.total = off;
  return L;
}

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

csa2_status check_cache(const csa2_cache *c, bool need_kv, bool need_ix) {
  if (!c) return fail(CSA2_EINVAL, "cache is NULL");
  if (!c->block_table || !c->n_entries) return fail(CSA2_EINVAL, "cache block_table / n_entries is NULL");
  if (need_kv && (!c->kv_codes || !c->kv_scales)) return fail(CSA2_EINVAL, "cache main-KV arrays are NULL");
  if (need_ix && (!c->ix_codes || !c->ix_scales)) return fail(CSA2_EINVAL, "cache indexer arrays are NULL");
  if (!is_pow2(c->page_size) || c->page_size > 4096)
    return fail(CSA2_EUNSUPPORTED, "page_size %d is not a power of two in [1, 4096]", c->page_size);
  if (c->max_pages <= 0 || c->num_pages <= 0)
    return fail(CSA2_EINVAL, "max_pages (%d) and num_pages (%d) must be positive", c->max_pages, c->num_pages);
  if ((int64_t)c->max_pages * c->page_size >= (1LL << 31) ||
      (int64_t)c->num_pages * c->page_size >= (1LL << 31))
    return fail(CSA2_EUNSUPPORTED, "cache of 2^31 or more entries");
  return CSA2_OK;
}

csa2_status check_window(const csa2_window *w) {
  if (!w) return CSA2_OK;
  if (w->rows < 0 || w->rows > 65536) return fail(CSA2_EINVAL, "window rows %d outside [0, 65536]", w->rows);
  if (!w->pos0 && w->rows > 4096) return fail(CSA2_EINVAL, "a decode window holds at most 4096 rows");
  if (w->window < 1 || w->window > 4096) return fail(CSA2_EINVAL, "window size %d outside [1, 4096]", w->window);
  if (w->rows > 0 && (!w->codes || !w->length)) return fail(CSA2_EINVAL, "window codes / length is NULL");
  return CSA2_OK;
}

int32_t win_cap_of(const csa2_window *w, const int32_t *q_pos) {
  if (!w || w->rows == 0) return 0;
  return (w->pos0 && q_pos) ? w->window : w->rows;
}

DevCache dev_cache(const csa2_cache *c) {
  DevCache d;
  d.kv_codes = c->kv_codes;
  d.kv_scales = c->kv_scales;
  d.ix_codes = c->ix_codes;
  d.ix_scales = c->ix_scales;
  d.block_table = c->block_table;
  d.n_entries = c->n_entries;
  d.page_shift = __builtin_ctz((unsigned)c->page_size);
  d.max_pages = c->max_pages;
  d.num_pages = c->num_pages;
  return d;
}

csa2_status check_ws(void *ws, size_t ws_bytes, size_t need) {
  if (need == 0) return CSA2_OK;
  if (!ws) return fail(CSA2_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (((uintptr_t)ws & 255) != 0) return fail(CSA2_EWORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < need) return fail(CSA2_EWORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  return CSA2_OK;
}

// Selection of the top-T[t] columns of `rows` score rows for one or two
// targets. Scores sit in the workspace's score region (or the caller's); in
// the compact path the coarse histogram was accumulated by the scoring kernel
// (hist_ready, after the zeroing fill) or is built here.
struct SelTarget {
  int32_t T;
  int32_t *out;
  int32_t stride;
};

csa2_status run_select(const WsLayout &L, char *ws, int rows, int32_t n_cols, const int32_t *cand_map,
                       const int32_t *n_entries, const int32_t *q_pos, int32_t nq, const SelTarget *tg,
                       int ntarget, bool hist_ready, const float *scores, hipStream_t st) {
  if (!L.compact) {  // the row fits one workgroup
    csa2::DirectArgs d{};
    d.scores = scores;
    d.n_cols = n_cols;
    d.cand_map = cand_map;
    d.n_entries = n_entries;
    d.q_pos = q_pos;
    d.nq = nq;
    for (int i = 0; i < ntarget; ++i) {
      d.T[i] = tg[i].T;
      d.out[i] = tg[i].out;
      d.out_stride[i] = tg[i].stride;
    }
    return hip_check(L.row_sel ? csa2::launch_sel_rowwise(d, rows, ntarget, st)
                               : csa2::launch_select_direct(d, rows, ntarget, st),
                     "select");
  }
  csa2_status s;
  if (!hist_ready) {
    s = hip_check(csa2::launch_fill_u32((uint32_t *)(ws + L.hist), (int64_t)((L.zero_end - L.hist) / 4), 0u, st),
                  "fill");
    if (s) return s;
    s = hip_check(csa2::launch_hist(scores, n_cols, rows, (uint32_t *)(ws + L.hist), st), "hist");
    if (s) return s;
  }
  csa2::CompactArgs c{};
  c.scores = scores;
  c.n_cols = n_cols;
  c.cand_map = cand_map;
  c.n_entries = n_entries;
  c.q_pos = q_pos;
  c.nq = nq;
  c.hist = (const uint32_t *)(ws + L.hist);
  c.ntarget = ntarget;
  for (int i = 0; i < ntarget; ++i) c.T[i] = tg[i].T;
  c.info = (int32_t *)(ws + L.info);
  c.counts = (uint32_t *)(ws + L.counts);
  c.suf = (uint32_t *)(ws + L.suf);
  c.list[0] = (uint64_t *)(ws + L.list0);
  c.list[1] = (uint64_t *)(ws + L.list1);
  c.eq[0] = (uint64_t *)(ws + L.eq0);
  c.eq[1] = (uint64_t *)(ws + L.eq1);
  c.seg_stride = L.seg_stride;
  c.max_wg = L.max_wg;
  c.chunk = L.chunk;
  if ((s = hip_check(csa2::launch_compact(c, rows, st), "compact"))) return s;
  csa2::FinalArgs f{};
  f.scores = scores;
  f.n_cols = n_cols;
  f.cand_map = cand_map;
  f.n_entries = n_entries;
  f.q_pos = q_pos;
  f.nq = nq;
  f.info = c.info;
  f.counts = c.counts;
  f.suf = c.suf;
  f.list[0] = c.list[0];
  f.list[1] = c.list[1];
  f.eq[0] = c.eq[0];
  f.eq[1] = c.eq[1];
  f.seg_stride = c.seg_stride;
  f.max_wg = c.max_wg;
  f.chunk = c.chunk;
  for (int i = 0; i < ntarget; ++i) {
    f.T[i] = tg[i].T;
    f.out[i] = tg[i].out;
    f.out_stride[i] = tg[i].stride;
  }
  return hip_check(csa2::launch_final(f, rows, ntarget, st), "select");
}

// Attention kernel choice (csa2_set_attend_kernel): auto, the eight-wave
// kernel, or the paired-wave kernel; the initial value from the environment.
int initial_attend_kernel() {
  const char *v = getenv("CSA2_ATTEND_KERNEL");
  if (v && strcmp(v, "seg") == 0) return CSA2_ATTEND_SEG;
  if (v && strcmp(v, "pair") == 0) return CSA2_ATTEND_PAIR;
  return CSA2_ATTEND_AUTO;
}
std::atomic<int> g_attend_kernel{initial_attend_kernel()};

// auto: the paired-wave kernel pays more per row (Q staging, the combine of
// four pairs) and less per unit, so it is taken where a workgroup takes at
// least three units (measured: the prefill chunk, 272 per workgroup; the
// ragged stack and the speculative step, 4-5; even at the 128K decode step's
// 3; the eight-wave kernel is faster with one unit per workgroup, as at 1M)
bool use_pair_kernel(const WsLayout &L) {
  const int k = g_attend_kernel.load(std::memory_order_relaxed);
  if (k != CSA2_ATTEND_AUTO) return k == CSA2_ATTEND_PAIR;
  return (L.att_T + L.att_G - 1) / L.att_G >= 3;
}

csa2_status run_attend(const WsLayout &L, char *ws, const csa2_cache *cache, const int32_t *idx,
                       int32_t k, const float *q, const csa2_window *win, const int32_t *q_pos,
                       float sm_scale, int rows, int32_t nq, float *out, float *lse, hipStream_t st) {
  csa2::AttendArgs a{};
  a.c = dev_cache(cache);
  a.idx = idx;
  a.k = k;
  a.q = q;
  if (win && win->rows > 0) {
    a.win_codes = win->codes;
    a.win_row_scale = win->row_scale;
    a.win_len = win->length;
    a.win_pos0 = q_pos ? win->pos0 : nullptr;
    a.win_rows = win->rows;
    a.win_window = win->window;
  }
  a.win_cap = win_cap_of(win, q_pos);
  a.q_pos = q_pos;
  a.nq = nq;
  a.sm_scale = sm_scale;
  a.part = (float *)(ws + L.part);
  csa2::SegArgs sg{};
  sg.T = L.att_T;
  sg.U = L.att_U;
  sg.G = L.att_G;
  sg.xcd = 1;
  sg.out = out;
  sg.lse = lse;
  if (use_pair_kernel(L)) return hip_check(csa2::launch_attend_wave(a, sg, L.att_slots, st), "attend");
  return hip_check(csa2::launch_attend_seg(a, sg, L.att_slots, st), "attend");
}

}  // namespace

extern "C" {

const char *csa2_status_string(csa2_status s) {
  switch (s) {
    case CSA2_OK: return "ok";
    case CSA2_EINVAL: return "invalid argument";
    case CSA2_EUNSUPPORTED: return "unsupported";
    case CSA2_EWORKSPACE: return "workspace too small";
    case CSA2_EHIP: return "HIP error";
  }
  return "unknown status";
}

const char *csa2_last_error(void) { return g_err; }

const char *csa2_version(void) { return "csa2-mi355x 0.1 (gfx950)"; }

size_t csa2_workspace_bytes(csa2_mode mode, int32_t batch, int32_t nq, int32_t n_cols, int32_t k,
                            int32_t pool, int32_t win_cap) {
  if (batch <= 0 || nq <= 0 || k <= 0) return 0;
  if (mode == CSA2_REUSE) n_cols = 0;
  const int ntarget = (mode == CSA2_FULL && pool > 0) ? 2 : 1;
  return ws_layout(mode, (int64_t)batch * nq, n_cols < 0 ? 0 : n_cols, k, win_cap, ntarget,
                   use_fused_topk(mode, batch, nq, n_cols, pool))
      .total;
}

csa2_status csa2_index_score(const csa2_cache *cache, const uint8_t *qix_codes,
                             const uint8_t *qix_scales, const float *w, const int32_t *q_pos,
                             const int32_t *cand, int32_t n_cand, int32_t batch, int32_t nq,
                             float *scores, uint32_t *hist, void *stream) {
  csa2_status s = check_cache(cache, false, true);
  if (s) return s;
  if (!qix_codes || !qix_scales || !w || !scores) return fail(CSA2_EINVAL, "NULL indexer query, weights or scores");
  if (batch <= 0 || nq <= 0) return fail(CSA2_EINVAL, "batch (%d) and nq (%d) must be positive", batch, nq);
  if (cand && n_cand <= 0) return fail(CSA2_EINVAL, "n_cand must be positive with a candidate list");
  csa2::ScoreArgs a{};
  a.c = dev_cache(cache);
  a.qix_codes = qix_codes;
  a.qix_scales = qix_scales;
  a.w = w;
  a.q_pos = q_pos;
  a.cand = cand;
  a.n_cand = cand ? n_cand : 0;
  a.nq = nq;
  a.n_cols = cand ? n_cand : cache->max_pages * cache->page_size;
  a.scores = scores;
  a.hist = hist;
  a.write_masked = 1;
  a.chunk = kScoreChunk;
  if (use_prefill_scoring(nq, cand, cache->page_size) || (!cand && nq > 1)) {
    // several query rows per request: one read of the keys serves all of them
    a.hist = nullptr;
    s = hip_check(use_prefill_scoring(nq, cand, cache->page_size)
                      ? csa2::launch_prefill_score(a, batch, (hipStream_t)stream)
                      : csa2::launch_index_score_mq(a, batch, (hipStream_t)stream),
                  "index_score");
    if (s || !hist) return s;
    return hip_check(csa2::launch_hist(scores, a.n_cols, batch * nq, hist, (hipStream_t)stream,
                                       cache->n_entries, q_pos, nq), "hist");
  }
  return hip_check(csa2::launch_index_score(a, batch * nq, (hipStream_t)stream), "index_score");
}

csa2_status csa2_topk(const float *scores, const int32_t *cand, int32_t batch, int32_t nq, int32_t n,
                      int32_t k, int32_t *idx_out, void *ws, size_t ws_bytes, void *stream) {
  if (!scores || !idx_out) return fail(CSA2_EINVAL, "NULL scores or idx_out");
  if (batch <= 0 || nq <= 0 || n <= 0) return fail(CSA2_EINVAL, "batch, nq and n must be positive");
  if (k <= 0 || k > CSA2_MAX_K) return fail(CSA2_EINVAL, "k = %d outside [1, %d]", k, CSA2_MAX_K);
  if ((int64_t)n > kMaxSelectCols)
    return fail(CSA2_EUNSUPPORTED, "more than %lld scores per row", (long long)kMaxSelectCols);
  const WsLayout L = ws_layout(CSA2_REINDEX, (int64_t)batch * nq, n, k, 0, 1);
  csa2_status s = check_ws(ws, ws_bytes, L.total);
  if (s) return s;
  const SelTarget tg{k, idx_out, k};
  s = run_select(L, (char *)ws, batch * nq, n, cand, nullptr, nullptr, nq, &tg, 1, false, scores,
                 (hipStream_t)stream);
  if (s || !cand || !(L.compact || L.row_sel)) return s;
  // these paths write ids in column order: sort them when ids are a map
  return hip_check(csa2::launch_sort_rows(idx_out, k, k, batch * nq, (hipStream_t)stream), "sort");
}

}  // extern "C"

namespace {

csa2_status check_attend(const csa2_cache *cache, const int32_t *idx, int32_t k, const float *q,
                         const csa2_window *win, float sm_scale, int32_t batch, int32_t nq, const float *out,
                         const float *lse) {
  csa2_status s = check_cache(cache, true, false);
  if (s) return s;
  if ((s = check_window(win))) return s;
  if (!idx || !q || !out || !lse) return fail(CSA2_EINVAL, "NULL idx, q, out or lse");
  if (batch <= 0 || nq <= 0) return fail(CSA2_EINVAL, "batch (%d) and nq (%d) must be positive", batch, nq);
  if (k <= 0 || k > CSA2_MAX_K) return fail(CSA2_EINVAL, "k = %d outside [1, %d]", k, CSA2_MAX_K);
  if (!isfinite(sm_scale)) return fail(CSA2_EINVAL, "sm_scale is not finite");
  return CSA2_OK;
}

// Device address of `scratch` on the current device, looked up on the first
// call made with that device current and kept per device (each GPU holds its
// own copy of the array at its own address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {};

csa2_status scratch_address(void **out) {
  int dev = -1;
  csa2_status s = hip_check(hipGetDevice(&dev), "hipGetDevice");
  if (s) return s;
  if (dev < 0 || dev >= kMaxDevices) return fail(CSA2_EUNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void *p = nullptr;
    if ((s = hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"))) return s;
    if (!p) return fail(CSA2_EHIP, "hipGetSymbolAddress(scratch) gave NULL");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return CSA2_OK;
}

}  // namespace

extern "C" {

csa2_status csa2_sparse_attend(const csa2_cache *cache, const int32_t *idx, int32_t k, const float *q,
                               const csa2_window *win, const int32_t *q_pos, float sm_scale,
                               int32_t batch, int32_t nq, float *out, float *lse, void *ws,
                               size_t ws_bytes, void *stream) {
  csa2_status s = check_attend(cache, idx, k, q, win, sm_scale, batch, nq, out, lse);
  if (s) return s;
  const WsLayout L = ws_layout(CSA2_REUSE, (int64_t)batch * nq, 0, k, win_cap_of(win, q_pos), 1);
  if ((s = check_ws(ws, ws_bytes, L.total))) return s;
  return run_attend(L, (char *)ws, cache, idx, k, q, win, q_pos, sm_scale, batch * nq, nq, out, lse,
                    (hipStream_t)stream);
}

csa2_status csa2_sparse_attend_noalloc(const csa2_cache *cache, const int32_t *idx, int32_t k,
                                       const float *q, const csa2_window *win, const int32_t *q_pos,
                                       float sm_scale, int32_t batch, int32_t nq, float *out,
                                       float *lse, void *stream) {
  csa2_status s = check_attend(cache, idx, k, q, win, sm_scale, batch, nq, out, lse);
  if (s) return s;
  const WsLayout L = ws_layout(CSA2_REUSE, (int64_t)batch * nq, 0, k, win_cap_of(win, q_pos), 1);
  if (L.total > (size_t)CSA2_NOALLOC_SCRATCH_BYTES)
    return fail(CSA2_EUNSUPPORTED, "the attention split needs %zu bytes of scratch, the library holds %d",
                L.total, CSA2_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  if (L.total > 0 && (s = scratch_address(&ws))) return s;
  return run_attend(L, (char *)ws, cache, idx, k, q, win, q_pos, sm_scale, batch * nq, nq, out, lse,
                    (hipStream_t)stream);
}

// Scoring and selection of a Full or Reindex layer into idx_out (and
// pool_out): everything csa2_layer_step does before it attends.
csa2_status run_layer_select(const csa2_layer_args *p, const WsLayout &L, int32_t n_cols, hipStream_t st) {
  csa2_status s = CSA2_OK;
  char *ws = (char *)p->ws;
  const int rows = p->batch * p->nq;
  if (L.fused) {
    csa2::PrefillTopkArgs a{};
    a.c = dev_cache(p->cache);
    a.qix_codes = p->qix_codes;
    a.qix_scales = p->qix_scales;
    a.w = p->w;
    a.q_pos = p->q_pos;
    a.nq = p->nq;
    a.n_cols = n_cols;
    a.k = p->k;
    a.idx_out = p->idx_out;
    if ((s = hip_check(csa2::launch_prefill_topk(a, p->batch, st), "prefill_topk"))) return s;
  } else {
    float *scores = (float *)(ws + L.scores);
    if (L.compact) {
      s = hip_check(csa2::launch_fill_u32((uint32_t *)(ws + L.hist), (int64_t)((L.zero_end - L.hist) / 4), 0u, st),
                    "fill");
      if (s) return s;
    }
    csa2::ScoreArgs a{};
    a.c = dev_cache(p->cache);
    a.qix_codes = p->qix_codes;
    a.qix_scales = p->qix_scales;
    a.w = p->w;
    a.q_pos = p->q_pos;
    a.cand = p->mode == CSA2_REINDEX ? p->idx_in : nullptr;
    a.n_cand = p->mode == CSA2_REINDEX ? p->pool : 0;
    a.nq = p->nq;
    a.n_cols = n_cols;
    a.scores = scores;
    a.hist = L.compact ? (uint32_t *)(ws + L.hist) : nullptr;
    a.write_masked = 0;
    a.chunk = p->mode == CSA2_REINDEX ? kScoreChunkCand : kScoreChunk;
    // the pool and the top-K of a Full layer are both selected over every visible entry
    const SelTarget tgf[2] = {{p->k, p->idx_out, p->k}, {p->pool, p->pool_out, p->pool}};
    const SelTarget tgr{p->k, p->idx_out, p->k};
    const SelTarget *tg = p->mode == CSA2_FULL ? tgf : &tgr;
    const int ntarget = (p->mode == CSA2_FULL && p->pool > 0) ? 2 : 1;
    if (p->mode == CSA2_FULL && (use_prefill_scoring(p->nq, nullptr, p->cache->page_size) || p->nq > 1)) {
      // several query rows per request share each read of the keys; the
      // histogram (chunked selection only) is a pass of its own
      a.hist = nullptr;
      s = hip_check(use_prefill_scoring(p->nq, nullptr, p->cache->page_size)
                        ? csa2::launch_prefill_score(a, p->batch, st)
                        : csa2::launch_index_score_mq(a, p->batch, st),
                    "index_score");
      if (s) return s;
      if (L.compact &&
          (s = hip_check(csa2::launch_hist(scores, n_cols, rows, (uint32_t *)(ws + L.hist), st,
                                           p->cache->n_entries, p->q_pos, p->nq), "hist")))
        return s;
    } else if ((s = hip_check(csa2::launch_index_score(a, rows, st), "index_score"))) {
      return s;
    }
    if (p->mode == CSA2_FULL)
      s = run_select(L, ws, rows, n_cols, nullptr, p->cache->n_entries, p->q_pos, p->nq, tg, ntarget, true,
                     scores, st);
    else
      s = run_select(L, ws, rows, n_cols, p->idx_in, nullptr, nullptr, p->nq, tg, 1, true, scores, st);
    if (s) return s;
  }
  return s;
}

csa2_status csa2_layer_step(const csa2_layer_args *args, void *stream) {
  if (!args) return fail(CSA2_EINVAL, "args is NULL");
  // the mode's bytes are read as an int first: a C caller may pass any value,
  // and a C++ load of an out-of-range enumerator is undefined
  int32_t mode_raw;
  static_assert(sizeof(csa2_mode) == sizeof(int32_t), "csa2_mode is an int");
  memcpy(&mode_raw, &args->mode, sizeof mode_raw);
  if (mode_raw != CSA2_FULL && mode_raw != CSA2_REINDEX && mode_raw != CSA2_REUSE)
    return fail(CSA2_EINVAL, "unknown mode %d", (int)mode_raw);
  const csa2_layer_args *p = args;
  const bool selecting = p->mode == CSA2_FULL || p->mode == CSA2_REINDEX;
  csa2_status s = check_cache(p->cache, true, selecting);
  if (s) return s;
  if ((s = check_window(p->win))) return s;
  if (!p->q || !p->out || !p->lse) return fail(CSA2_EINVAL, "NULL q, out or lse");
  if (p->batch <= 0 || p->nq <= 0) return fail(CSA2_EINVAL, "batch (%d) and nq (%d) must be positive", p->batch, p->nq);
  if (p->k <= 0 || p->k > CSA2_MAX_K) return fail(CSA2_EINVAL, "k = %d outside [1, %d]", p->k, CSA2_MAX_K);
  if (!isfinite(p->sm_scale)) return fail(CSA2_EINVAL, "sm_scale is not finite");
  if (selecting && (!p->qix_codes || !p->qix_scales || !p->w || !p->idx_out))
    return fail(CSA2_EINVAL, "a selecting layer needs qix_codes, qix_scales, w and idx_out");
  if (p->mode == CSA2_FULL && p->pool != 0) {
    if (p->pool < p->k || p->pool > CSA2_MAX_POOL)
      return fail(CSA2_EINVAL, "pool %d outside [k=%d, %d]", p->pool, p->k, CSA2_MAX_POOL);
    if (!p->pool_out) return fail(CSA2_EINVAL, "pool > 0 needs pool_out");
  }
  if (p->mode == CSA2_FULL && p->pool < 0) return fail(CSA2_EINVAL, "negative pool");
  if (p->mode == CSA2_REINDEX) {
    if (!p->idx_in) return fail(CSA2_EINVAL, "a Reindex layer needs the pool in idx_in");
    if (p->pool < p->k || p->pool > CSA2_MAX_POOL)
      return fail(CSA2_EINVAL, "pool %d outside [k=%d, %d]", p->pool, p->k, CSA2_MAX_POOL);
  }
  if (p->mode == CSA2_REUSE && !p->idx_in) return fail(CSA2_EINVAL, "a Reuse layer needs the inherited top-k in idx_in");

  const int rows = p->batch * p->nq;
  const int32_t capacity = p->cache->max_pages * p->cache->page_size;
  if (selecting && (int64_t)(p->mode == CSA2_FULL ? capacity : p->pool) > kMaxSelectCols)
    return fail(CSA2_EUNSUPPORTED, "more than %lld entries per row to select from", (long long)kMaxSelectCols);
  const int32_t n_cols = p->mode == CSA2_FULL ? capacity : (p->mode == CSA2_REINDEX ? p->pool : 0);
  const int32_t wcap = win_cap_of(p->win, p->q_pos);
  const WsLayout L = ws_layout(p->mode, rows, n_cols, p->k, wcap, (p->mode == CSA2_FULL && p->pool > 0) ? 2 : 1,
                               use_fused_topk(p->mode, p->batch, p->nq, n_cols, p->pool));
  if ((s = check_ws(p->ws, p->ws_bytes, L.total))) return s;
  hipStream_t st = (hipStream_t)stream;
  char *ws = (char *)p->ws;

  const int32_t *att_idx = p->idx_in;
  if (selecting) {
    if ((s = run_layer_select(p, L, n_cols, st))) return s;
    att_idx = p->idx_out;
  }
  return run_attend(L, ws, p->cache, att_idx, p->k, p->q, p->win, p->q_pos, p->sm_scale, rows,
                    p->nq, p->out, p->lse, st);
}

csa2_status csa2_index_topk(const csa2_cache *cache, const uint8_t *qix_codes, const uint8_t *qix_scales,
                            const float *w, const int32_t *q_pos, int32_t batch, int32_t nq, int32_t k,
                            int32_t pool, int32_t *idx_out, int32_t *pool_out, void *ws, size_t ws_bytes,
                            void *stream) {
  csa2_status s = check_cache(cache, false, true);
  if (s) return s;
  if (!qix_codes || !qix_scales || !w || !idx_out)
    return fail(CSA2_EINVAL, "NULL qix_codes, qix_scales, w or idx_out");
  if (batch <= 0 || nq <= 0) return fail(CSA2_EINVAL, "batch (%d) and nq (%d) must be positive", batch, nq);
  if (k <= 0 || k > CSA2_MAX_K) return fail(CSA2_EINVAL, "k = %d outside [1, %d]", k, CSA2_MAX_K);
  if (pool < 0) return fail(CSA2_EINVAL, "negative pool");
  if (pool != 0) {
    if (pool < k || pool > CSA2_MAX_POOL) return fail(CSA2_EINVAL, "pool %d outside [k=%d, %d]", pool, k, CSA2_MAX_POOL);
    if (!pool_out) return fail(CSA2_EINVAL, "pool > 0 needs pool_out");
  }
  const int32_t capacity = cache->max_pages * cache->page_size;
  if ((int64_t)capacity > kMaxSelectCols)
    return fail(CSA2_EUNSUPPORTED, "more than %lld entries per row to select from", (long long)kMaxSelectCols);
  const WsLayout L = ws_layout(CSA2_FULL, (int64_t)batch * nq, capacity, k, 0, pool > 0 ? 2 : 1,
                               use_fused_topk(CSA2_FULL, batch, nq, capacity, pool));
  if ((s = check_ws(ws, ws_bytes, L.total))) return s;
  csa2_layer_args a{};
  a.mode = CSA2_FULL;
  a.cache = cache;
  a.qix_codes = qix_codes;
  a.qix_scales = qix_scales;
  a.w = w;
  a.q_pos = q_pos;
  a.batch = batch;
  a.nq = nq;
  a.k = k;
  a.pool = pool;
  a.idx_out = idx_out;
  a.pool_out = pool_out;
  a.ws = ws;
  a.ws_bytes = ws_bytes;
  return run_layer_select(&a, L, capacity, (hipStream_t)stream);
}

csa2_status csa2_quantize_fp4(const float *x, int64_t n_rows, int32_t channels, uint8_t *codes,
                              uint8_t *scales, void *stream) {
  if (!x || !codes || !scales) return fail(CSA2_EINVAL, "NULL pointer");
  if (n_rows < 0 || channels <= 0 || channels % 16)
    return fail(CSA2_EINVAL, "channels must be a positive multiple of 16 and n_rows >= 0");
  if (((uintptr_t)x & 15) || ((uintptr_t)codes & 7))
    return fail(CSA2_EINVAL, "x must be 16-byte and codes 8-byte aligned");
  return hip_check(csa2::launch_quant_fp4(x, n_rows, channels, codes, scales, (hipStream_t)stream),
                   "quantize_fp4");
}

csa2_status csa2_kv_append(const csa2_cache_w *cache, const float *kv, const float *ix,
                           const int32_t *entry, int32_t batch, int32_t n_new, void *stream) {
  if (!cache || !kv || !entry) return fail(CSA2_EINVAL, "NULL cache, kv or entry");
  if (!cache->kv_codes || !cache->kv_scales || !cache->block_table)
    return fail(CSA2_EINVAL, "cache kv_codes, kv_scales or block_table is NULL");
  if (ix && (!cache->ix_codes || !cache->ix_scales))
    return fail(CSA2_EINVAL, "ix given but the cache has no indexer arrays");
  if (batch <= 0 || n_new < 0) return fail(CSA2_EINVAL, "batch must be positive, n_new >= 0");
  if (!is_pow2(cache->page_size)) return fail(CSA2_EUNSUPPORTED, "page size %d is not a power of two", cache->page_size);
  if (cache->max_pages <= 0 || cache->num_pages <= 0) return fail(CSA2_EINVAL, "empty page table");
  if (((uintptr_t)kv & 15) || ((uintptr_t)ix & 15)) return fail(CSA2_EINVAL, "kv and ix must be 16-byte aligned");
  csa2::AppendArgs a{};
  a.kv_codes = cache->kv_codes;
  a.kv_scales = cache->kv_scales;
  a.ix_codes = cache->ix_codes;
  a.ix_scales = cache->ix_scales;
  a.block_table = cache->block_table;
  a.page_shift = __builtin_ctz((unsigned)cache->page_size);
  a.max_pages = cache->max_pages;
  a.num_pages = cache->num_pages;
  a.kv = kv;
  a.ix = ix;
  a.entry = entry;
  a.batch = batch;
  a.n_new = n_new;
  return hip_check(csa2::launch_kv_append(a, (hipStream_t)stream), "kv_append");
}

csa2_status csa2_window_append(uint8_t *codes, float *row_scale, int32_t rows, const float *x,
                               const int32_t *row, int32_t batch, int32_t n_new, void *stream) {
  if (!codes || !x || !row) return fail(CSA2_EINVAL, "NULL codes, x or row");
  if (rows <= 0 || batch <= 0 || n_new < 0) return fail(CSA2_EINVAL, "rows and batch must be positive, n_new >= 0");
  if (((uintptr_t)x & 15) || ((uintptr_t)codes & 3)) return fail(CSA2_EINVAL, "x must be 16-byte and codes 4-byte aligned");
  return hip_check(csa2::launch_window_append(codes, row_scale, rows, x, row, batch, n_new, (hipStream_t)stream),
                   "window_append");
}

csa2_status csa2_dequant_fp4(const uint8_t *codes, const uint8_t *scales, int64_t n_rows,
                             int32_t channels, uint16_t *out_f16, void *stream) {
  if (!codes || !scales || !out_f16) return fail(CSA2_EINVAL, "NULL pointer");
  if (n_rows < 0 || channels <= 0 || channels % 32) return fail(CSA2_EINVAL, "channels must be a positive multiple of 32");
  return hip_check(csa2::launch_dequant_fp4(codes, scales, n_rows, channels, out_f16, (hipStream_t)stream),
                   "dequant_fp4");
}

csa2_status csa2_stream_read(const void *p, size_t n_bytes, uint32_t *sink, int32_t blocks, void *stream) {
  if (!p || !sink) return fail(CSA2_EINVAL, "NULL pointer");
  if (n_bytes < 16 || n_bytes % 16 || ((uintptr_t)p & 15)) return fail(CSA2_EINVAL, "n_bytes must be a positive multiple of 16, p 16-byte aligned");
  if (blocks < 1) return fail(CSA2_EINVAL, "blocks must be positive");
  return hip_check(csa2::launch_stream_read(p, (int64_t)n_bytes, sink, blocks, (hipStream_t)stream), "stream_read");
}

csa2_status csa2_set_attend_kernel(int32_t kernel) {
  if (kernel != CSA2_ATTEND_AUTO && kernel != CSA2_ATTEND_SEG && kernel != CSA2_ATTEND_PAIR)
    return fail(CSA2_EINVAL, "attend kernel %d is not one of 0 (auto), 1 (seg), 2 (pair)", kernel);
  g_attend_kernel.store(kernel, std::memory_order_relaxed);
  return CSA2_OK;
}

csa2_status csa2_dequant_e4m3(const uint8_t *bytes, int64_t n, float *out, void *stream) {
  if (!bytes || !out) return fail(CSA2_EINVAL, "NULL pointer");
  if (n < 0) return fail(CSA2_EINVAL, "negative n");
  return hip_check(csa2::launch_dequant_e4m3(bytes, n, out, (hipStream_t)stream), "dequant_e4m3");
}

}  // extern "C"
