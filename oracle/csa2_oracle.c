/*
 * CSA2 decode oracle -- TEST INFRASTRUCTURE ONLY (see csa2_oracle.h).
 *
 * Plain fp64 loops in the order the method is described, one function per
 * step. OpenMP only splits independent (request, query) rows across threads;
 * there is no blocking, fusion or reordering of any sum beyond the
 * definitions below.
 */
#include "csa2_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_D 512      /* main-KV latent channels, shared by all query heads */
#define ORC_H 16       /* query heads */
#define ORC_HI 4       /* indexer heads */
#define ORC_DI 64      /* indexer channels */
#define ORC_G 16       /* channels per E4M3 scale ([P2-FP4]) */
#define ORC_TPE 4      /* tokens per compressed entry (reading: m = 4) */

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Threads for the following calls (timing only; results do not depend on it). */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}

/* ---- Step 1: the two number formats ([P2-FP4]) --------------------------
 * E2M1: sign | 2 exponent bits | 1 mantissa bit, bias 1, subnormal at e=0:
 *   e == 0: 0.5*m; else 2^(e-1) * (1 + m/2).
 * E4M3 (OCP "fn" variant, the one whose maximum is 448): sign | 4 exp | 3 man,
 *   bias 7; e == 0: 2^-6 * m/8; else 2^(e-7) * (1 + m/8); exponent 15 with
 *   mantissa 7 is NaN (no infinities).
 * Reading: the pages name "E4M3" and compare with NVFP4, whose scale is this
 * OCP variant; the sign bit is decoded honestly even for scales. */
double orc_e2m1(int code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

double orc_e4m3(int byte) {
  int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
  if (e == 15 && m == 7) return NAN;
  double v = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

static double T_E2M1[16];
static double T_E4M3[256];
static int tables_ready = 0;

static void build_tables(void) {
  if (tables_ready) return;
  for (int i = 0; i < 16; ++i) T_E2M1[i] = orc_e2m1(i);
  for (int i = 0; i < 256; ++i) T_E4M3[i] = orc_e4m3(i);
  tables_ready = 1;
}

/* ---- Step 2: dequantisation ----------------------------------------------
 * Channel c of an FP4 row: nibble c of the code bytes (reading: the even
 * channel in the low nibble) times the E4M3 scale of its 16-channel group. */
static double fp4_value(const uint8_t *codes, const uint8_t *scales, int c) {
  int nib = (codes[c >> 1] >> ((c & 1) * 4)) & 15;
  return T_E2M1[nib] * T_E4M3[scales[c / ORC_G]];
}

void orc_dequant_fp4(const uint8_t *codes, const uint8_t *scales, int64_t n_rows,
                     int32_t channels, double *out) {
  build_tables();
  for (int64_t r = 0; r < n_rows; ++r)
    for (int c = 0; c < channels; ++c)
      out[r * channels + c] = fp4_value(codes + r * (channels / 2),
                                        scales + r * (channels / ORC_G), c);
}

void orc_dequant_e4m3(const uint8_t *bytes, const float *row_scale, int64_t n_rows,
                      int32_t channels, double *out) {
  build_tables();
  for (int64_t r = 0; r < n_rows; ++r) {
    double rs = row_scale ? (double)row_scale[r] : 1.0;
    for (int c = 0; c < channels; ++c) out[r * channels + c] = T_E4M3[bytes[r * channels + c]] * rs;
  }
}

/* ---- Encoding (the write side of the cache) -------------------------------
 * Nearest representable value by exhaustive search over the format's
 * magnitudes in increasing order; a tie goes to the even mantissa (the even
 * code, since consecutive codes differ in the mantissa's last bit).
 * Readings are listed in csa2_oracle.h. */
static int nearest_even(const double *mag, int n, double a) {
  int best = 0;
  double bd = fabs(a - mag[0]);
  for (int i = 1; i < n; ++i) {
    double d = fabs(a - mag[i]);
    if (d < bd || (d == bd && (i & 1) == 0 && (best & 1) == 1)) {
      best = i;
      bd = d;
    }
  }
  return best;
}

int orc_e4m3_encode(float x) {
  build_tables();
  /* finite magnitudes: bytes 0x00..0x7E (0x7F is NaN) */
  int b = nearest_even(T_E4M3, 0x7F, fabs((double)x));
  return b | (x < 0.0f ? 0x80 : 0);
}

void orc_e4m3_encode_n(const float *x, int64_t n, uint8_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_e4m3_encode(x[i]);
}

int orc_e2m1_encode(float y) {
  build_tables();
  int c = nearest_even(T_E2M1, 8, fabs((double)y));
  return c | (y < 0.0f ? 8 : 0);
}

void orc_quantize_fp4(const float *x, int64_t n_rows, int32_t channels, uint8_t *codes,
                      uint8_t *scales) {
  build_tables();
  for (int64_t r = 0; r < n_rows; ++r) {
    const float *xr = x + r * channels;
    uint8_t *cr = codes + r * (channels / 2);
    for (int c = 0; c < channels / 2; ++c) cr[c] = 0;
    for (int g = 0; g < channels / ORC_G; ++g) {
      float amax = 0.0f;
      for (int i = 0; i < ORC_G; ++i) {
        float a = fabsf(xr[g * ORC_G + i]);
        if (a > amax) amax = a;
      }
      int sb = orc_e4m3_encode(amax / 6.0f);
      scales[r * (channels / ORC_G) + g] = (uint8_t)sb;
      float s = (float)T_E4M3[sb];
      for (int i = 0; i < ORC_G; ++i) {
        int ch = g * ORC_G + i;
        float v = xr[ch];
        int code = (s == 0.0f) ? (v < 0.0f ? 8 : 0) : orc_e2m1_encode(v / s);
        cr[ch >> 1] |= (uint8_t)(code << ((ch & 1) * 4));
      }
    }
  }
}

void orc_kv_append(const orc_cache_w *c, const float *kv, const float *ix, const int32_t *entry,
                   int32_t B, int32_t n_new) {
  for (int b = 0; b < B; ++b)
    for (int j = 0; j < n_new; ++j) {
      int32_t s = entry[(int64_t)b * n_new + j];
      if (s < 0 || s / c->page_size >= c->max_pages) continue;
      int32_t page = c->block_table[(int64_t)b * c->max_pages + s / c->page_size];
      if (page < 0 || page >= c->num_pages) continue;
      int64_t row = (int64_t)page * c->page_size + s % c->page_size;
      orc_quantize_fp4(kv + ((int64_t)b * n_new + j) * ORC_D, 1, ORC_D, c->kv_codes + row * (ORC_D / 2),
                       c->kv_scales + row * (ORC_D / ORC_G));
      if (ix)
        orc_quantize_fp4(ix + ((int64_t)b * n_new + j) * ORC_DI, 1, ORC_DI,
                         c->ix_codes + row * (ORC_DI / 2), c->ix_scales + row * (ORC_DI / ORC_G));
    }
}

void orc_window_append(uint8_t *codes, float *row_scale, int32_t rows, const float *x,
                       const int32_t *row, int32_t B, int32_t n_new) {
  for (int b = 0; b < B; ++b)
    for (int j = 0; j < n_new; ++j) {
      int32_t w = row[(int64_t)b * n_new + j];
      if (w < 0 || w >= rows) continue;
      const float *xr = x + ((int64_t)b * n_new + j) * ORC_D;
      uint8_t *dst = codes + ((int64_t)b * rows + w) * ORC_D;
      float rs = 1.0f;
      if (row_scale) {
        float amax = 0.0f;
        for (int c = 0; c < ORC_D; ++c)
          if (fabsf(xr[c]) > amax) amax = fabsf(xr[c]);
        rs = amax > 0.0f ? amax / 448.0f : 1.0f;
        row_scale[(int64_t)b * rows + w] = rs;
      }
      for (int c = 0; c < ORC_D; ++c)
        dst[c] = (uint8_t)orc_e4m3_encode(row_scale ? xr[c] / rs : xr[c]);
    }
}

/* Physical row of entry s of request b, or -1 if the page table has no page. */
static int64_t entry_row(const orc_cache *c, int b, int64_t s) {
  int32_t page = c->block_table[(int64_t)b * c->max_pages + s / c->page_size];
  if (page < 0 || page >= c->num_pages) return -1;
  return (int64_t)page * c->page_size + s % c->page_size;
}

/* ---- Step 3: visibility --------------------------------------------------
 * Decode: every written entry. With a query position p (prefill), entry s
 * covers tokens 4s..4s+3 and is visible once complete: 4(s+1) <= p+1
 * (reading of "block-causal"; an entry is never partly visible). */
static int64_t visible_entries(const orc_cache *c, const int32_t *q_pos, int b, int nq, int t) {
  int64_t V = c->n_entries[b];
  if (q_pos) {
    int64_t vp = ((int64_t)q_pos[(int64_t)b * nq + t] + 1) / ORC_TPE;
    if (vp < V) V = vp;
    if (V < 0) V = 0;
  }
  return V;
}

/* ---- Step 4: lightning-indexer score ([P2-CSA2], [P2-FP4]) ---------------
 * Reading (pages give no formula; the indexer descends from V3.2's DSA
 * lightning indexer): I_s = sum_h w_h * max(0, q_h . k_s), four indexer heads
 * sharing one 64-channel key per entry, q_h and k_s dequantised FP4. */
static double index_score_one(const double qd[ORC_HI][ORC_DI], const double *wq,
                              const uint8_t *kcodes, const uint8_t *kscales) {
  double kd[ORC_DI];
  for (int c = 0; c < ORC_DI; ++c) kd[c] = fp4_value(kcodes, kscales, c);
  double I = 0.0;
  for (int h = 0; h < ORC_HI; ++h) {
    double dot = 0.0;
    for (int c = 0; c < ORC_DI; ++c) dot += qd[h][c] * kd[c];
    I += wq[h] * (dot > 0.0 ? dot : 0.0);
  }
  return I;
}

int orc_index_score(const orc_cache *c, const uint8_t *qix_codes, const uint8_t *qix_scales,
                    const float *w, const int32_t *q_pos, const int32_t *cand, int32_t n_cand,
                    int32_t B, int32_t nq, int32_t n_cols, double *scores) {
  build_tables();
  if (cand) n_cols = n_cand;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bt = 0; bt < (int64_t)B * nq; ++bt) {
    int b = (int)(bt / nq), t = (int)(bt % nq);
    double qd[ORC_HI][ORC_DI], wq[ORC_HI];
    for (int h = 0; h < ORC_HI; ++h) {
      const uint8_t *qc = qix_codes + (bt * ORC_HI + h) * (ORC_DI / 2);
      const uint8_t *qs = qix_scales + (bt * ORC_HI + h) * (ORC_DI / ORC_G);
      for (int ch = 0; ch < ORC_DI; ++ch) qd[h][ch] = fp4_value(qc, qs, ch);
      wq[h] = (double)w[bt * ORC_HI + h];
    }
    int64_t V = visible_entries(c, q_pos, b, nq, t);
    double *row = scores + bt * (int64_t)n_cols;
    for (int64_t j = 0; j < n_cols; ++j) {
      int64_t s = cand ? (int64_t)cand[bt * (int64_t)n_cand + j] : j;
      int64_t r = (s >= 0 && s < V) ? entry_row(c, b, s) : -1;
      row[j] = (r < 0) ? -INFINITY
                       : index_score_one((const double(*)[ORC_DI])qd, wq,
                                         c->ix_codes + r * (ORC_DI / 2),
                                         c->ix_scales + r * (ORC_DI / ORC_G));
    }
  }
  return 0;
}

/* ---- Step 5: Top-K selection ([P2-CSA2]: "re-score with its own Q and pick
 * Top-K") --------------------------------------------------------------------
 * Order key: score descending, entry id ascending (reading: ties go to the
 * lower id). Masked candidates (-inf) are never selected; short rows are
 * padded with -1. The selected set is returned sorted by id. */
typedef struct { double score; int32_t id; } orc_pair;

static int by_score_then_id(const void *pa, const void *pb) {
  const orc_pair *a = (const orc_pair *)pa, *b = (const orc_pair *)pb;
  if (a->score > b->score) return -1;
  if (a->score < b->score) return 1;
  return (a->id > b->id) - (a->id < b->id);
}

static int by_id(const void *pa, const void *pb) {
  int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
  return (a > b) - (a < b);
}

int orc_topk(const double *scores, const int32_t *cand, int32_t B, int32_t nq, int32_t n,
             int32_t k, int32_t *idx_out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bt = 0; bt < (int64_t)B * nq; ++bt) {
    orc_pair *p = (orc_pair *)malloc(sizeof(orc_pair) * (size_t)(n > 0 ? n : 1));
    int64_t m = 0;
    for (int64_t j = 0; j < n; ++j) {
      double s = scores[bt * (int64_t)n + j];
      if (!(s > -INFINITY)) continue;
      p[m].score = s;
      p[m].id = cand ? cand[bt * (int64_t)n + j] : (int32_t)j;
      ++m;
    }
    qsort(p, (size_t)m, sizeof(orc_pair), by_score_then_id);
    int32_t *o = idx_out + bt * (int64_t)k;
    int64_t take = m < k ? m : k;
    for (int64_t j = 0; j < take; ++j) o[j] = p[j].id;
    qsort(o, (size_t)take, sizeof(int32_t), by_id);
    for (int64_t j = take; j < k; ++j) o[j] = -1;
    free(p);
  }
  return 0;
}

/* ---- Steps 6-7: the attention set and its softmax ([P1-CSA2], [P2-CSA2],
 * [P2-FP4]) -------------------------------------------------------------------
 * Rows = the selected compressed entries (FP4 latent, used as both key and
 * value: all 16 heads share one 512-channel latent) together with the
 * layer's own window rows (E4M3 x row scale). Reading: one joint softmax over
 * both sets; an entry that overlaps the window is not removed.
 *   z_hr = tau * (q_h . row_r),  M_h = max_r z_hr,  L_h = sum_r exp(z_hr - M_h)
 *   out_h = sum_r exp(z_hr - M_h) row_r / L_h,   lse_h = M_h + ln L_h
 * An empty set gives out = 0, lse = -inf. Padding (-1) and ids outside
 * [0, n_entries) are not rows. */
int orc_sparse_attend(const orc_cache *c, const int32_t *idx, int32_t k, const float *q,
                      const orc_window *win, const int32_t *q_pos, double sm_scale,
                      int32_t B, int32_t nq, double *out, double *lse, double *psum) {
  build_tables();
  int64_t max_rows = (int64_t)k + (win ? win->rows : 0);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bt = 0; bt < (int64_t)B * nq; ++bt) {
    int b = (int)(bt / nq);
    double *rows = (double *)malloc(sizeof(double) * (size_t)(max_rows > 0 ? max_rows : 1) * ORC_D);
    double *z = (double *)malloc(sizeof(double) * (size_t)(max_rows > 0 ? max_rows : 1));
    int64_t R = 0;
    for (int64_t j = 0; j < k; ++j) {
      int32_t s = idx[bt * (int64_t)k + j];
      if (s < 0 || s >= c->n_entries[b]) continue;
      int64_t r = entry_row(c, b, s);
      if (r < 0) continue;
      for (int ch = 0; ch < ORC_D; ++ch)
        rows[R * ORC_D + ch] = fp4_value(c->kv_codes + r * (ORC_D / 2),
                                         c->kv_scales + r * (ORC_D / ORC_G), ch);
      ++R;
    }
    if (win) {
      int64_t len = win->length[b];
      for (int64_t j = 0; j < len; ++j) {
        if (win->pos0 && q_pos) {
          int64_t tok = (int64_t)win->pos0[b] + j, p = q_pos[bt];
          if (!(tok <= p && tok > p - win->window)) continue;
        }
        const uint8_t *src = win->codes + ((int64_t)b * win->rows + j) * ORC_D;
        double rs = win->row_scale ? (double)win->row_scale[(int64_t)b * win->rows + j] : 1.0;
        for (int ch = 0; ch < ORC_D; ++ch) rows[R * ORC_D + ch] = T_E4M3[src[ch]] * rs;
        ++R;
      }
    }
    for (int h = 0; h < ORC_H; ++h) {
      const float *qh = q + (bt * ORC_H + h) * ORC_D;
      double *oh = out + (bt * ORC_H + h) * ORC_D;
      for (int ch = 0; ch < ORC_D; ++ch) oh[ch] = 0.0;
      if (R == 0) {
        lse[bt * ORC_H + h] = -INFINITY;
        if (psum) psum[bt * ORC_H + h] = 0.0;
        continue;
      }
      double M = -INFINITY;
      for (int64_t r = 0; r < R; ++r) {
        double dot = 0.0;
        for (int ch = 0; ch < ORC_D; ++ch) dot += (double)qh[ch] * rows[r * ORC_D + ch];
        z[r] = sm_scale * dot;
        if (z[r] > M) M = z[r];
      }
      double L = 0.0;
      for (int64_t r = 0; r < R; ++r) L += exp(z[r] - M);
      double ps = 0.0;
      for (int64_t r = 0; r < R; ++r) {
        double p = exp(z[r] - M) / L;
        ps += p;
        for (int ch = 0; ch < ORC_D; ++ch) oh[ch] += p * rows[r * ORC_D + ch];
      }
      lse[bt * ORC_H + h] = M + log(L);
      if (psum) psum[bt * ORC_H + h] = ps;
    }
    free(rows);
    free(z);
  }
  return 0;
}

/* ---- Step 8: the three layer modes ([P1-CSA2], [P2-CSA2]) -----------------
 * Full computes its own index scores over every visible entry and selects;
 * it also emits the candidate pool for later Reindex layers (reading of the
 * garbled pool sentence: the pool is the Full layer's own top-`pool` by the
 * same score, so its top-K is a subset of the pool). Reindex keeps the Full
 * layer's KV and indexer keys, re-scores only the pool with its own indexer
 * query and weights, and selects its own top-K. Reuse inherits the top-K
 * and computes no index score. Every mode attends with its own query and its
 * own window. */
int orc_layer_step(int mode, const orc_cache *c, const orc_window *win, const float *q,
                   const uint8_t *qix_codes, const uint8_t *qix_scales, const float *w,
                   const int32_t *q_pos, int32_t B, int32_t nq, int32_t k, int32_t pool,
                   const int32_t *idx_in, int32_t *idx_out, int32_t *pool_out,
                   double sm_scale, double *out, double *lse, double *scores_out) {
  const int32_t *use_idx = idx_in;
  if (mode == 0 || mode == 1) {
    int32_t n = (mode == 0) ? c->max_pages * c->page_size : pool;
    const int32_t *cand = (mode == 0) ? NULL : idx_in;
    double *sc = scores_out ? scores_out
                            : (double *)malloc(sizeof(double) * (size_t)B * nq * (size_t)(n > 0 ? n : 1));
    orc_index_score(c, qix_codes, qix_scales, w, q_pos, cand, n, B, nq, n, sc);
    if (mode == 0 && pool > 0 && pool_out) orc_topk(sc, NULL, B, nq, n, pool, pool_out);
    orc_topk(sc, cand, B, nq, n, k, idx_out);
    if (!scores_out) free(sc);
    use_idx = idx_out;
  }
  return orc_sparse_attend(c, use_idx, k, q, win, q_pos, sm_scale, B, nq, out, lse, NULL);
}
