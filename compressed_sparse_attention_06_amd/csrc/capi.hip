// C ABI of the CSA2 decode library: argument checks, workspace layout and the
// launch sequence of each entry point. Every check runs on the host and reads
// no device memory; nothing here allocates or synchronises.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "csa2_dev.h"
#include "kernels.h"

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

constexpr int kFinItems = 16384;     // rows up to this length select in LDS directly
constexpr int kRowsPerSplit = 256;   // attention rows per workgroup
constexpr int kScoreChunk = 2048;    // scoring columns per workgroup
constexpr int kCompactChunk = 8192;  // compaction columns per workgroup

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t scores = 0, hist = 0, ctr = 0, cand = 0, part = 0, total = 0;
  bool compact = false;
  int n_split = 0;
};

WsLayout ws_layout(csa2_mode mode, int64_t rows, int64_t n_cols, int32_t k, int32_t win_cap) {
  WsLayout L;
  size_t off = 0;
  if (mode == CSA2_FULL || mode == CSA2_REINDEX) {
    L.compact = n_cols > kFinItems;
    L.scores = off;
    off = align256(off + (size_t)rows * n_cols * 4);
    L.hist = off;
    off = align256(off + (size_t)rows * HIST_BINS * 4);
    L.ctr = off;
    off = align256(off + (size_t)rows * 4 * 4);
    L.cand = off;
    if (L.compact) off = align256(off + (size_t)rows * n_cols * 4);
  }
  const int64_t span = (int64_t)k + (win_cap > 0 ? win_cap : 0);
  L.n_split = (int)((span + kRowsPerSplit - 1) / kRowsPerSplit);
  if (L.n_split < 1) L.n_split = 1;
  L.part = off;
  off = align256(off + (size_t)rows * L.n_split * CSA2_H * csa2::kPartStride * 4);
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

// Selection of the top-T columns of `rows` score rows (optionally the top K2
// of that set too). Scores already sit in the workspace's score region, and
// for the compact path the histogram was accumulated by the scoring kernel
// (hist_ready) or is built here.
csa2_status run_select(const WsLayout &L, char *ws, int rows, int32_t n_cols, const int32_t *cand_map,
                       const int32_t *n_entries, const int32_t *q_pos, int32_t nq, int32_t T,
                       int32_t *outT, int32_t outT_stride, int sortT, int32_t K2, int32_t *outK2,
                       int32_t id_limit, bool hist_ready, const float *scores, hipStream_t st) {
  csa2::FinalArgs f{};
  f.scores = scores;
  f.n_cols = n_cols;
  f.cand_map = cand_map;
  f.n_entries = n_entries;
  f.q_pos = q_pos;
  f.nq = nq;
  f.T = T;
  f.outT = outT;
  f.outT_stride = outT_stride;
  f.sortT = sortT;
  f.K2 = K2;
  f.outK2 = outK2;
  f.K2_stride = K2;
  f.id_limit = id_limit;
  if (L.compact) {
    uint32_t *hist = (uint32_t *)(ws + L.hist);
    uint32_t *ctr = (uint32_t *)(ws + L.ctr);
    csa2_status s;
    if (!hist_ready) {
      s = hip_check(csa2::launch_fill_u32(hist, (int64_t)((L.cand - L.hist) / 4), 0u, st), "fill");
      if (s) return s;
      s = hip_check(csa2::launch_hist(scores, n_cols, rows, hist, st), "hist");
      if (s) return s;
    }
    csa2::CompactArgs c{};
    c.scores = scores;
    c.n_cols = n_cols;
    c.cand_map = cand_map;
    c.n_entries = n_entries;
    c.q_pos = q_pos;
    c.nq = nq;
    c.hist = hist;
    c.T = T;
    c.out = outT;
    c.out_stride = outT_stride;
    c.cand_cols = (int32_t *)(ws + L.cand);
    c.ctr = ctr;
    c.chunk = kCompactChunk;
    s = hip_check(csa2::launch_compact(c, rows, st), "compact");
    if (s) return s;
    f.hist = hist;
    f.cand_cols = c.cand_cols;
    f.ctr = ctr;
  }
  return hip_check(csa2::launch_final(f, rows, st), "select");
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
  a.rows_per_split = kRowsPerSplit;
  a.n_split = L.n_split;
  a.part = (float *)(ws + L.part);
  csa2_status s = hip_check(csa2::launch_attend(a, rows, st), "attend");
  if (s) return s;
  csa2::MergeArgs m{};
  m.part = a.part;
  m.n_split = L.n_split;
  m.out = out;
  m.lse = lse;
  return hip_check(csa2::launch_merge(m, rows, st), "merge");
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
  (void)pool;
  if (batch <= 0 || nq <= 0 || k <= 0) return 0;
  if (mode == CSA2_REUSE) n_cols = 0;
  return ws_layout(mode, (int64_t)batch * nq, n_cols < 0 ? 0 : n_cols, k, win_cap).total;
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
  return hip_check(csa2::launch_index_score(a, batch * nq, (hipStream_t)stream), "index_score");
}

csa2_status csa2_topk(const float *scores, const int32_t *cand, int32_t batch, int32_t nq, int32_t n,
                      int32_t k, int32_t *idx_out, void *ws, size_t ws_bytes, void *stream) {
  if (!scores || !idx_out) return fail(CSA2_EINVAL, "NULL scores or idx_out");
  if (batch <= 0 || nq <= 0 || n <= 0) return fail(CSA2_EINVAL, "batch, nq and n must be positive");
  if (k <= 0 || k > CSA2_MAX_K) return fail(CSA2_EINVAL, "k = %d outside [1, %d]", k, CSA2_MAX_K);
  const WsLayout L = ws_layout(CSA2_REINDEX, (int64_t)batch * nq, n, k, 0);
  csa2_status s = check_ws(ws, ws_bytes, L.total);
  if (s) return s;
  // ids of a candidate map are unbounded: sort them over the int32 range only when they are columns
  const int32_t id_limit = cand ? 0x7FFFFFFF : n;
  return run_select(L, (char *)ws, batch * nq, n, cand, nullptr, nullptr, nq, k, idx_out, k, 1, 0,
                    nullptr, id_limit, false, scores, (hipStream_t)stream);
}

csa2_status csa2_sparse_attend(const csa2_cache *cache, const int32_t *idx, int32_t k, const float *q,
                               const csa2_window *win, const int32_t *q_pos, float sm_scale,
                               int32_t batch, int32_t nq, float *out, float *lse, void *ws,
                               size_t ws_bytes, void *stream) {
  csa2_status s = check_cache(cache, true, false);
  if (s) return s;
  if ((s = check_window(win))) return s;
  if (!idx || !q || !out || !lse) return fail(CSA2_EINVAL, "NULL idx, q, out or lse");
  if (batch <= 0 || nq <= 0) return fail(CSA2_EINVAL, "batch (%d) and nq (%d) must be positive", batch, nq);
  if (k <= 0 || k > CSA2_MAX_K) return fail(CSA2_EINVAL, "k = %d outside [1, %d]", k, CSA2_MAX_K);
  if (!isfinite(sm_scale)) return fail(CSA2_EINVAL, "sm_scale is not finite");
  const WsLayout L = ws_layout(CSA2_REUSE, (int64_t)batch * nq, 0, k, win_cap_of(win, q_pos));
  if ((s = check_ws(ws, ws_bytes, L.total))) return s;
  return run_attend(L, (char *)ws, cache, idx, k, q, win, q_pos, sm_scale, batch * nq, nq, out, lse,
                    (hipStream_t)stream);
}

csa2_status csa2_layer_step(const csa2_layer_args *p, void *stream) {
  if (!p) return fail(CSA2_EINVAL, "args is NULL");
  const bool selecting = p->mode == CSA2_FULL || p->mode == CSA2_REINDEX;
  if (p->mode != CSA2_FULL && p->mode != CSA2_REINDEX && p->mode != CSA2_REUSE)
    return fail(CSA2_EINVAL, "unknown mode %d", (int)p->mode);
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
  const int32_t n_cols = p->mode == CSA2_FULL ? capacity : (p->mode == CSA2_REINDEX ? p->pool : 0);
  const int32_t wcap = win_cap_of(p->win, p->q_pos);
  const WsLayout L = ws_layout(p->mode, rows, n_cols, p->k, wcap);
  if ((s = check_ws(p->ws, p->ws_bytes, L.total))) return s;
  hipStream_t st = (hipStream_t)stream;
  char *ws = (char *)p->ws;

  const int32_t *att_idx = p->idx_in;
  if (selecting) {
    float *scores = (float *)(ws + L.scores);
    if (L.compact) {
      s = hip_check(csa2::launch_fill_u32((uint32_t *)(ws + L.hist), (int64_t)((L.cand - L.hist) / 4), 0u, st), "fill");
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
    a.chunk = kScoreChunk;
    if ((s = hip_check(csa2::launch_index_score(a, rows, st), "index_score"))) return s;
    if (p->mode == CSA2_FULL) {
      const bool with_pool = p->pool > 0;
      s = run_select(L, ws, rows, n_cols, nullptr, p->cache->n_entries, p->q_pos, p->nq,
                     with_pool ? p->pool : p->k, with_pool ? p->pool_out : p->idx_out,
                     with_pool ? p->pool : p->k, with_pool ? 0 : 1, with_pool ? p->k : 0,
                     with_pool ? p->idx_out : nullptr, capacity, true, scores, st);
    } else {
      s = run_select(L, ws, rows, n_cols, p->idx_in, nullptr, nullptr, p->nq, p->k, p->idx_out,
                     p->k, 1, 0, nullptr, capacity, true, scores, st);
    }
    if (s) return s;
    att_idx = p->idx_out;
  }
  return run_attend(L, ws, p->cache, att_idx, p->k, p->q, p->win, p->q_pos, p->sm_scale, rows,
                    p->nq, p->out, p->lse, st);
}

csa2_status csa2_dequant_fp4(const uint8_t *codes, const uint8_t *scales, int64_t n_rows,
                             int32_t channels, uint16_t *out_f16, void *stream) {
  if (!codes || !scales || !out_f16) return fail(CSA2_EINVAL, "NULL pointer");
  if (n_rows < 0 || channels <= 0 || channels % 32) return fail(CSA2_EINVAL, "channels must be a positive multiple of 32");
  return hip_check(csa2::launch_dequant_fp4(codes, scales, n_rows, channels, out_f16, (hipStream_t)stream),
                   "dequant_fp4");
}

csa2_status csa2_dequant_e4m3(const uint8_t *bytes, int64_t n, float *out, void *stream) {
  if (!bytes || !out) return fail(CSA2_EINVAL, "NULL pointer");
  if (n < 0) return fail(CSA2_EINVAL, "negative n");
  return hip_check(csa2::launch_dequant_e4m3(bytes, n, out, (hipStream_t)stream), "dequant_e4m3");
}

}  // extern "C"
