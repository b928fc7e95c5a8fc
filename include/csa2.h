/*
 * csa2.h -- C ABI of the CSA2 decode hot path on AMD Instinct MI355X (gfx950).
 *
 * CSA2 ("compressed sparse attention", second generation) as described in the
 * public summaries of DeepSeek V4.1 Flash:
 *
 *   [P1]  "DeepSeek V4.1 Flash深度解析：KV缓存压缩437倍的技术路径", section on the
 *         second-generation compressed attention (layer modes, 6-layer groups,
 *         the candidate pool, 4-bit main KV, 8-bit sliding window).
 *   [P2]  "DeepSeek V4.1 Flash 如何靠压缩 KV 缓存实现小模型干翻大模型", section
 *         "CSA2" (Full / Reindex / Reuse; each mode keeps its own global Q and
 *         SWA KV) and section "FP4 量化 + Bounded Replay" (FP4 E2M1 with one E4M3
 *         scale per 16 channels and no second-level scale; FP4 indexer Q/K;
 *         window of the last 128 tokens).
 *
 * Data formats (all buffers are caller-owned device memory unless noted):
 *  - FP4 row: two E2M1 codes per byte, channel 2j in the low nibble of byte
 *    j; one OCP E4M3 scale byte per 16 consecutive channels, stored in a
 *    separate array. Main KV rows have 512 channels (256 code bytes + 32
 *    scale bytes); indexer keys and indexer queries have 64 channels per head
 *    (32 + 4 bytes).
 *  - Window rows: 512 OCP E4M3 bytes, optionally times a per-row fp32 scale.
 *  - Caches are paged: entry s of request b sits in page
 *    block_table[b*max_pages + s/page_size], slot s % page_size.
 *
 * Conventions for every entry point:
 *  - Asynchronous on `stream` (a hipStream_t, NULL = legacy default stream).
 *    No call allocates device memory, synchronises, or throws.
 *  - Argument checks happen on the host before any launch and return
 *    CSA2_EINVAL / CSA2_EUNSUPPORTED / CSA2_EWORKSPACE with nothing launched;
 *    they read no device memory, so they can be exercised without a GPU.
 *  - Pointers are borrowed until the stream reaches the call.
 *  - Device-resident values are not validated: an index outside
 *    [0, n_entries[b]), a page id outside [0, num_pages) or a -1 pad is
 *    treated as "no entry" (never dereferenced), so bad data cannot fault.
 *  - Workspace: caller-provided device memory of at least
 *    csa2_workspace_bytes(...) bytes, 256-byte aligned. Its contents need not
 *    be initialised; calls sharing one workspace must not overlap in time.
 *  - The error text of the last failing call on the calling thread is
 *    available from csa2_last_error().
 */
#ifndef CSA2_API_H
#define CSA2_API_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_LATENT 512     /* main-KV latent channels, shared by all query heads */
#define CSA2_HEADS 16       /* query heads */
#define CSA2_IX_HEADS 4     /* indexer query heads */
#define CSA2_IX_DIM 64      /* indexer channels */
#define CSA2_TOKENS_PER_ENTRY 4
#define CSA2_MAX_K 4096
#define CSA2_MAX_POOL 65536
#define CSA2_MAX_SELECT_COLS 524288  /* longest score row a selection takes (2M tokens) */

typedef enum {
  CSA2_OK = 0,
  CSA2_EINVAL = 1,       /* null required pointer, non-positive size, inconsistent sizes */
  CSA2_EUNSUPPORTED = 2, /* valid request this library does not implement */
  CSA2_EWORKSPACE = 3,   /* workspace missing, too small or misaligned */
  CSA2_EHIP = 4          /* a HIP launch failed; see csa2_last_error() */
} csa2_status;

typedef enum { CSA2_FULL = 0, CSA2_REINDEX = 1, CSA2_REUSE = 2 } csa2_mode;

/* One Full layer's compressed cache (read as well by the Reindex and Reuse
 * layers that follow it, [P2] "CSA2"). */
typedef struct {
  const uint8_t *kv_codes;     /* [num_pages][page_size][256] main-KV E2M1 pairs */
  const uint8_t *kv_scales;    /* [num_pages][page_size][32]  E4M3 per 16 channels */
  const uint8_t *ix_codes;     /* [num_pages][page_size][32]  indexer key (64 ch) */
  const uint8_t *ix_scales;    /* [num_pages][page_size][4] */
  const int32_t *block_table;  /* [batch][max_pages] page ids; unused slots may hold -1 */
  const int32_t *n_entries;    /* [batch] compressed entries written per request */
  int32_t page_size;           /* power of two, 1..4096 */
  int32_t max_pages;           /* columns of block_table */
  int32_t num_pages;           /* pages in the arrays above */
} csa2_cache;

/* One layer's sliding-window rows ([P1] keeps the window at 8 bit; [P2]
 * truncates it to the last 128 tokens).
 * pos0 == NULL (decode): the length[b] valid rows are all visible.
 * pos0 != NULL (a chunk of queries with positions q_pos): row j holds token
 * pos0[b] + j and a query at position p sees rows with token position in
 * (p - window, p]. */
typedef struct {
  const uint8_t *codes;     /* [batch][rows][512] E4M3 */
  const float *row_scale;   /* [batch][rows] or NULL (= 1.0) */
  const int32_t *length;    /* [batch] valid rows, <= rows */
  const int32_t *pos0;      /* [batch] or NULL */
  int32_t rows;             /* row capacity per request, 0..65536 */
  int32_t window;           /* window size in tokens (128), 1..4096 */
} csa2_window;

/* Index scores of the lightning indexer ([P2] "CSA2", "FP4 ..."):
 *   I_s = sum_{h<4} w_h * max(0, q_h . k_s)
 * with q_h the FP4 indexer query of head h and k_s the FP4 indexer key of
 * entry s. Visible entries: s < n_entries[b] and, when q_pos != NULL,
 * 4(s+1) <= q_pos + 1 (an entry covers 4 tokens and is visible once whole).
 *  qix_codes  [batch][nq][4][32], qix_scales [batch][nq][4][4], w [batch][nq][4] fp32
 *  q_pos      [batch][nq] absolute token positions, or NULL (decode)
 *  cand       NULL: column j is entry j, n_cols = max_pages*page_size.
 *             else [batch][nq][n_cand] entry ids (a Reindex pool), n_cols = n_cand.
 *  scores     [batch][nq][n_cols] fp32 out; -inf for masked entries and pads.
 *  hist       NULL, or [batch][nq][4096] uint32 to which the count of each
 *             finite score's top 12 order-key bits is added (the histogram
 *             the selection starts from; the key of a score is its IEEE bits
 *             with the sign bit flipped for non-negative values and all bits
 *             flipped for negative ones, -0 counted as +0). */
csa2_status csa2_index_score(const csa2_cache *cache, const uint8_t *qix_codes,
                             const uint8_t *qix_scales, const float *w, const int32_t *q_pos,
                             const int32_t *cand, int32_t n_cand, int32_t batch, int32_t nq,
                             float *scores, uint32_t *hist, void *stream);

/* Top-K selection ([P2] "CSA2": each selecting layer picks its own Top-K).
 * For each of the rows = batch*nq score rows of length n, selects the k
 * largest finite scores, ties broken towards the lower entry id; entry id of
 * column j is j, or cand[row][j] when cand != NULL. -inf columns are never
 * selected. idx_out [rows][k]: the selected ids in ascending order, then -1.
 * n <= CSA2_MAX_SELECT_COLS, else CSA2_EUNSUPPORTED.
 * Workspace: csa2_workspace_bytes(CSA2_REINDEX, batch, nq, n, k, 0, 0). */
csa2_status csa2_topk(const float *scores, const int32_t *cand, int32_t batch, int32_t nq,
                      int32_t n, int32_t k, int32_t *idx_out, void *ws, size_t ws_bytes,
                      void *stream);

/* Sparse attention over the selected entries and the window ([P2] "CSA2":
 * every mode attends with its own global Q and its own window).
 * Rows of the attention set: the FP4 main-KV latent of each listed entry
 * (used as both key and value by all 16 heads) and the visible window rows
 * (E4M3 x row scale). One softmax over both sets:
 *   z = sm_scale * q_h . row,  out_h = sum softmax(z) * row,  lse_h = logsumexp(z)
 * An empty set gives out = 0 and lse = -inf.
 *  idx  [batch][nq][k] entry ids (-1 = padding), q [batch][nq][16][512] fp32,
 *  out  [batch][nq][16][512] fp32, lse [batch][nq][16] fp32 (natural log).
 * Workspace: csa2_workspace_bytes(CSA2_REUSE, batch, nq, 0, k, 0, win_cap). */
csa2_status csa2_sparse_attend(const csa2_cache *cache, const int32_t *idx, int32_t k,
                               const float *q, const csa2_window *win, const int32_t *q_pos,
                               float sm_scale, int32_t batch, int32_t nq, float *out,
                               float *lse, void *ws, size_t ws_bytes, void *stream);

/* csa2_sparse_attend for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. The same computation and kernels as csa2_sparse_attend, but the
 * split partials (the only scratch the attention uses) live in a
 * library-owned device array of CSA2_NOALLOC_SCRATCH_BYTES (one copy per GPU
 * the library runs on, held until the process ends) instead of a caller
 * workspace; the caller still passes every input and output. The array's
 * device address is looked up once per device, on the first call made with
 * that device current. Nothing is allocated or freed, and nothing in the
 * array needs to start at any value. Every call on one GPU shares that GPU's
 * array: calls that overlap in time on the same GPU (other streams, other
 * threads) race and must be serialised by the caller. A call whose attention
 * split would need more scratch than the array holds returns
 * CSA2_EUNSUPPORTED (the split uses at most 256 workgroups, so no valid
 * call does). */
#define CSA2_NOALLOC_SCRATCH_BYTES (256 * 2 * 16 * 516 * 4) /* 16,908,288 */
csa2_status csa2_sparse_attend_noalloc(const csa2_cache *cache, const int32_t *idx, int32_t k,
                                       const float *q, const csa2_window *win, const int32_t *q_pos,
                                       float sm_scale, int32_t batch, int32_t nq, float *out,
                                       float *lse, void *stream);

/* One CSA2 layer ([P1], [P2] "CSA2").
 *  FULL:    score every visible entry with this layer's indexer query; select
 *           the top `pool` entries into pool_out [batch][nq][pool] (when
 *           pool > 0) and the top k into idx_out [batch][nq][k]; both hold
 *           ascending ids followed by -1 pads; attend. The cache capacity
 *           max_pages*page_size is at most CSA2_MAX_SELECT_COLS.
 *  REINDEX: idx_in is the pool of the preceding Full layer [batch][nq][pool]
 *           as pool_out wrote it (ascending ids, then -1); rescore only those
 *           entries with this layer's own indexer query, select the top k
 *           into idx_out; attend. With a pool that is not ascending, idx_out
 *           holds the same selected set, in pool order rather than ascending
 *           once pool > 4096.
 *  REUSE:   idx_in [batch][nq][k] inherited; no indexer work; attend.
 * All modes use this layer's own q and window.
 * A FULL call over a prefill chunk (nq >= 64, batch*nq >= 1024, pool = 0,
 * capacity <= 32768 entries) scores and selects in one pass per query group
 * and keeps no score matrix; csa2_workspace_bytes sizes its workspace
 * accordingly. The selected sets are the same as those of csa2_index_score
 * followed by csa2_topk on the same inputs. */
typedef struct {
  csa2_mode mode;
  const csa2_cache *cache;
  const csa2_window *win;     /* may be NULL: no window rows */
  const float *q;             /* [batch][nq][16][512] */
  const uint8_t *qix_codes;   /* FULL/REINDEX: [batch][nq][4][32] */
  const uint8_t *qix_scales;  /* FULL/REINDEX: [batch][nq][4][4] */
  const float *w;             /* FULL/REINDEX: [batch][nq][4] */
  const int32_t *q_pos;       /* [batch][nq] or NULL (decode) */
  int32_t batch, nq, k, pool;
  const int32_t *idx_in;      /* REINDEX: pool; REUSE: inherited top-k */
  int32_t *idx_out;           /* FULL/REINDEX */
  int32_t *pool_out;          /* FULL with pool > 0 */
  float sm_scale;
  float *out, *lse;
  void *ws;
  size_t ws_bytes;
} csa2_layer_args;

csa2_status csa2_layer_step(const csa2_layer_args *args, void *stream);

/* Scoring and selection of a Full layer without attention ([P2] "CSA2": a
 * Full layer scores every visible entry and keeps its own top-K, and the
 * pool Reindex layers rescore): idx_out [batch][nq][k] and, when pool > 0,
 * pool_out [batch][nq][pool], exactly as csa2_layer_step(FULL) writes them
 * before it attends (ascending ids, then -1). Arguments as for
 * csa2_layer_step; the prefill-chunk shapes it names run the fused kernel.
 * Workspace: csa2_workspace_bytes(CSA2_FULL, batch, nq, n_cols, k, pool, 0). */
csa2_status csa2_index_topk(const csa2_cache *cache, const uint8_t *qix_codes,
                            const uint8_t *qix_scales, const float *w, const int32_t *q_pos,
                            int32_t batch, int32_t nq, int32_t k, int32_t pool, int32_t *idx_out,
                            int32_t *pool_out, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes for one call.
 *  FULL:    n_cols = max_pages*page_size of the cache; pool may be 0.
 *  REINDEX: n_cols = pool (also the size to use for csa2_topk with n = n_cols).
 *  REUSE:   n_cols and pool ignored.
 * win_cap is the window's attention span: rows when pos0 == NULL, else
 * window (0 when there is no window). */
size_t csa2_workspace_bytes(csa2_mode mode, int32_t batch, int32_t nq, int32_t n_cols, int32_t k,
                            int32_t pool, int32_t win_cap);

/* Bit-exact dequantisation probes (same device code as the attention path).
 * fp4: codes [n_rows][channels/2], scales [n_rows][channels/16] -> out fp16
 *      [n_rows][channels] (raw IEEE half bits), channels a multiple of 32.
 * e4m3: bytes [n] -> out fp32 [n]. */
csa2_status csa2_dequant_fp4(const uint8_t *codes, const uint8_t *scales, int64_t n_rows,
                             int32_t channels, uint16_t *out_f16, void *stream);
csa2_status csa2_dequant_e4m3(const uint8_t *bytes, int64_t n, float *out, void *stream);

/* ---- The write side of the cache ([P2] "FP4 量化 + Bounded Replay": main KV
 * and indexer Q/K in E2M1 with one E4M3 scale per 16 channels, no
 * second-level scale; the window holds the last 128 tokens in 8 bits).
 * The pages give the formats, not the rounding. Rounding used: nearest
 * representable value, ties to the even mantissa, saturating (6 for E2M1,
 * 448 for E4M3); the block scale byte encodes amax/6 of its 16 channels
 * (division in fp32) and each channel encodes x / scale (fp32); the sign bit
 * is x < 0. Bit-exact against the oracle. The learned compressor that makes
 * the fp32 entries is not part of this library. */

/* Quantise rows: x [n_rows][channels] fp32 (16-byte aligned; channels a
 * positive multiple of 16) -> codes [n_rows][channels/2] (channel 2j in the
 * low nibble of byte j; 8-byte aligned) and scales [n_rows][channels/16].
 * Used for new entries and for the decode indexer query ([batch][nq][4][64]
 * is 4*batch*nq rows of 64). */
csa2_status csa2_quantize_fp4(const float *x, int64_t n_rows, int32_t channels, uint8_t *codes,
                              uint8_t *scales, void *stream);

/* Writable view of a paged cache (same layout as csa2_cache). */
typedef struct {
  uint8_t *kv_codes;        /* [num_pages][page][256] */
  uint8_t *kv_scales;       /* [num_pages][page][32] */
  uint8_t *ix_codes;        /* [num_pages][page][32]; may be NULL when ix is NULL */
  uint8_t *ix_scales;       /* [num_pages][page][4] */
  const int32_t *block_table; /* [batch][max_pages] */
  int32_t page_size, max_pages, num_pages;
} csa2_cache_w;

/* Append new compressed entries (one every 4 tokens): for request b and new
 * entry j, when entry[b][j] >= 0 it is the entry index s written; the main-KV
 * row kv[b][j][512] (and, when ix != NULL, the indexer key ix[b][j][64]) is
 * quantised into page block_table[b][s / page_size], slot s % page_size.
 * Entries whose page is missing (out of the table or negative) are skipped.
 * n_entries is the caller's to advance. kv, ix: fp32, 16-byte aligned. Two
 * entries of one call must not name the same slot. */
csa2_status csa2_kv_append(const csa2_cache_w *cache, const float *kv, const float *ix,
                           const int32_t *entry, int32_t batch, int32_t n_new, void *stream);

/* Append window tokens to each request's ring of `rows` rows: for token j of
 * request b, when row[b][j] is in [0, rows), x[b][j][512] (fp32, 16-byte
 * aligned) is encoded into codes[b][row][512]. With row_scale != NULL the row
 * is scaled first: rs = amax/448 (1 when amax is 0), stored in
 * row_scale[b][row], and each byte encodes x / rs. The caller keeps the
 * ring's position and length (csa2_window.length / pos0). */
csa2_status csa2_window_append(uint8_t *codes, float *row_scale, int32_t rows, const float *x,
                               const int32_t *row, int32_t batch, int32_t n_new, void *stream);

const char *csa2_status_string(csa2_status s);
const char *csa2_last_error(void);
const char *csa2_version(void);

#ifdef __cplusplus
}
#endif
#endif
