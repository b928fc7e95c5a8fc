/*
 * CSA2 decode oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, fp64 CPU reference for the decode-time hot path of CSA2
 * (compressed sparse attention, second generation) as summarised on the pages
 * about DeepSeek V4.1 Flash. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it. It shares no code, header, table
 * or constant with the HIP library under compressed_sparse_attention_06_amd/.
 *
 * Sources (page title, section):
 *  [P1-CSA2]  "DeepSeek V4.1 Flash深度解析：KV缓存压缩437倍的技术路径", section on
 *             compressed attention gen. 2: per-layer Full / Reindex / Reuse modes,
 *             6-layer groups, the candidate pool, 4-bit main KV and 8-bit window.
 *  [P2-CSA2]  "DeepSeek V4.1 Flash 如何靠压缩 KV 缓存实现小模型干翻大模型", section
 *             "CSA2": what each mode computes and reuses; every mode keeps its own
 *             global Q and its own SWA KV.
 *  [P2-FP4]   same page, section "FP4 量化 + Bounded Replay": E2M1 with one E4M3
 *             scale per 16 channels, no second-level scale; FP4 indexer Q/K;
 *             window of the last 128 tokens.
 *
 * Readings where the pages are silent are listed beside each function.
 * Floating point results are fp64. Nothing here allocates device memory.
 */
#ifndef CSA2_ORACLE_H
#define CSA2_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One Full layer's cache, paged: entry s of request b is at page
 * block_table[b*max_pages + s/page_size], slot s%page_size. */
typedef struct {
  const uint8_t *kv_codes;   /* [num_pages][page][256] two E2M1 codes per byte */
  const uint8_t *kv_scales;  /* [num_pages][page][32]  E4M3, one per 16 channels */
  const uint8_t *ix_codes;   /* [num_pages][page][32]  indexer key, 64 channels */
  const uint8_t *ix_scales;  /* [num_pages][page][4] */
  const int32_t *block_table;/* [B][max_pages] */
  const int32_t *n_entries;  /* [B] */
  int32_t page_size, max_pages, num_pages;
} orc_cache;

/* Sliding-window rows of one layer. pos0 == NULL: every one of the length[b]
 * rows is visible (decode). Otherwise row j holds token pos0[b]+j and a query
 * at position p sees rows with token position in (p - window, p]. */
typedef struct {
  const uint8_t *codes;      /* [B][rows][512] E4M3 */
  const float *row_scale;    /* [B][rows] or NULL (= 1) */
  const int32_t *length;     /* [B] */
  const int32_t *pos0;       /* [B] or NULL */
  int32_t rows, window;
} orc_window;

double orc_e2m1(int code);   /* code 0..15 */
double orc_e4m3(int byte);   /* byte 0..255; NaN for 0x7F / 0xFF */

/* Dequantise FP4 rows: out[r][c] = E2M1(code) * E4M3(scale[r][c/16]). */
void orc_dequant_fp4(const uint8_t *codes, const uint8_t *scales, int64_t n_rows,
                     int32_t channels, double *out);
/* Dequantise E4M3 rows: out[r][c] = E4M3(byte) * row_scale[r] (NULL -> 1). */
void orc_dequant_e4m3(const uint8_t *bytes, const float *row_scale, int64_t n_rows,
                      int32_t channels, double *out);

/* Index scores (fp64) [B][nq][n_cols]; -inf where masked / padding. */
int orc_index_score(const orc_cache *c, const uint8_t *qix_codes, const uint8_t *qix_scales,
                    const float *w, const int32_t *q_pos, const int32_t *cand, int32_t n_cand,
                    int32_t B, int32_t nq, int32_t n_cols, double *scores);

/* Selection: idx_out [B][nq][k], sorted ascending, -1 padded. */
int orc_topk(const double *scores, const int32_t *cand, int32_t B, int32_t nq, int32_t n,
             int32_t k, int32_t *idx_out);

/* Attention over the selected entries and the window: out [B][nq][16][512],
 * lse [B][nq][16], psum [B][nq][16] (sum of softmax weights; may be NULL). */
int orc_sparse_attend(const orc_cache *c, const int32_t *idx, int32_t k, const float *q,
                      const orc_window *win, const int32_t *q_pos, double sm_scale,
                      int32_t B, int32_t nq, double *out, double *lse, double *psum);

/* One CSA2 layer. mode 0 Full, 1 Reindex, 2 Reuse.
 * Full:    scores all visible entries; pool_out [B][nq][pool] if pool > 0;
 *          idx_out [B][nq][k]; attends idx_out.
 * Reindex: idx_in is the pool [B][nq][pool]; idx_out [B][nq][k]; attends.
 * Reuse:   idx_in [B][nq][k] inherited; attends.
 * scores_out (nullable) receives the layer's index scores. */
int orc_layer_step(int mode, const orc_cache *c, const orc_window *win, const float *q,
                   const uint8_t *qix_codes, const uint8_t *qix_scales, const float *w,
                   const int32_t *q_pos, int32_t B, int32_t nq, int32_t k, int32_t pool,
                   const int32_t *idx_in, int32_t *idx_out, int32_t *pool_out,
                   double sm_scale, double *out, double *lse, double *scores_out);

/* ---- Encoding: the write side of the cache ([P2-FP4]; [P2-FP4] also keeps
 * the last 128 tokens of the window). The pages give the formats only; the
 * rounding is a reading:
 *  - E4M3 encode: the finite E4M3 value nearest to x, ties to the even
 *    mantissa, saturating at +-448; the sign bit is x < 0.
 *  - FP4 block of 16 channels: scale byte = E4M3 encode of amax/6 (amax the
 *    group's largest |x|, 6 the largest E2M1 magnitude, the division in
 *    fp32); s = its value; each channel's code is the E2M1 magnitude nearest
 *    to |y|, y = x / s in fp32, ties to the even mantissa, saturating at 6,
 *    with the sign bit for x < 0 (s = 0 gives magnitude 0).
 *  - Window row: with a row scale, rs = amax/448 in fp32 (1 when amax is 0)
 *    and each byte encodes x / rs in fp32; without, each byte encodes x. */
int orc_e4m3_encode(float x);
void orc_e4m3_encode_n(const float *x, int64_t n, uint8_t *out);
int orc_e2m1_encode(float y);  /* y already divided by the block scale */

/* Quantise rows [n_rows][channels] (channels a multiple of 16) to codes
 * [n_rows][channels/2] (channel 2j in the low nibble of byte j) and scales
 * [n_rows][channels/16]. */
void orc_quantize_fp4(const float *x, int64_t n_rows, int32_t channels, uint8_t *codes,
                      uint8_t *scales);

/* Append new compressed entries: for request b and new entry j, when
 * entry[b*n_new + j] >= 0 it is the entry index s written: main KV row
 * kv[b][j][512] and (when ix != NULL) indexer key ix[b][j][64], quantised,
 * at page block_table[b*max_pages + s/page_size], slot s%page_size. Entries
 * whose page is missing are skipped. n_entries is left to the caller. */
typedef struct {
  uint8_t *kv_codes, *kv_scales, *ix_codes, *ix_scales;
  const int32_t *block_table;
  int32_t page_size, max_pages, num_pages;
} orc_cache_w;
void orc_kv_append(const orc_cache_w *c, const float *kv, const float *ix, const int32_t *entry,
                   int32_t B, int32_t n_new);

/* Window ring append: token j of request b, when row[b*n_new + j] >= 0, is
 * written at codes[b][row][512] (and row_scale[b][row] when row_scale !=
 * NULL). */
void orc_window_append(uint8_t *codes, float *row_scale, int32_t rows, const float *x,
                       const int32_t *row, int32_t B, int32_t n_new);

int orc_num_threads(void);
void orc_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
