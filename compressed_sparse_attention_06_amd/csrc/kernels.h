// Kernel argument blocks and host-side launchers of the CSA2 HIP library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa2_dev.h"

namespace csa2 {

struct ScoreArgs {
  DevCache c;
  const uint8_t *qix_codes, *qix_scales;  // [rows][4][32], [rows][4][4]
  const float *w;                         // [rows][4]
  const int32_t *q_pos;                   // [rows] or null
  const int32_t *cand;                    // [rows][n_cand] or null
  int32_t n_cand;
  int32_t nq;
  int32_t n_cols;        // columns per score row
  float *scores;         // [rows][n_cols]
  uint32_t *hist;        // [rows][HIST_BINS] or null
  int32_t write_masked;  // Full rows: also write -inf past the visible entries
  int32_t chunk;         // columns per workgroup (multiple of 128)
};

// Selection of one or two targets (T[t] largest keys of each score row) over
// rows cut into chunks of `chunk` columns (2048, 4096 or 8192), at most
// SEL_MAX_WG chunks per row.
#define SEL_MAX_WG 64

// k_compact, workgroup w of row r, for each target t:
//  info[(r*2+t)*4 + 0..2]  (workgroup 0 only) threshold bin, keys above it,
//                          keys in the row (histogram total)
//  counts[(r*2+t)*max_wg + w] = keys above the bin | keys in the bin << 16
//  suf[((r*2+t)*max_wg + w)*256 + d] = keys in the bin with digit >= d
//  list[t][r*seg_stride + w*chunk + ...] (key << 32 | id) of the keys at or
//                          above the bin, in column order
//  eq[t][r*seg_stride + w*chunk + ...] (key << 32 | id) of the keys in the
//                          bin, grouped by digit from 255 down
struct CompactArgs {
  const float *scores;
  int32_t n_cols;
  const int32_t *cand_map;   // [rows][n_cols] ids or null (id = column)
  const int32_t *n_entries;  // [batch] or null: limit columns to the visible entries
  const int32_t *q_pos;      // [rows] or null
  int32_t nq;
  const uint32_t *hist;      // coarse [rows][HIST_BINS]
  int32_t ntarget;
  int32_t T[2];
  int32_t *info;
  uint32_t *counts;
  uint32_t *suf;
  uint64_t *list[2];
  uint64_t *eq[2];
  int64_t seg_stride;        // per row, >= max_wg * chunk
  int32_t max_wg;
  int32_t chunk;
};

struct FinalArgs {
  const float *scores;
  int32_t n_cols;
  const int32_t *cand_map;
  const int32_t *n_entries;
  const int32_t *q_pos;
  int32_t nq;
  const int32_t *info;
  const uint32_t *counts;
  const uint32_t *suf;
  const uint64_t *list[2];
  const uint64_t *eq[2];
  int64_t seg_stride;
  int32_t max_wg;
  int32_t chunk;
  int32_t T[2];
  int32_t *out[2];
  int32_t out_stride[2];
};

// Rows of at most 8192 columns: one workgroup per row and target.
struct DirectArgs {
  const float *scores;
  int32_t n_cols;
  const int32_t *cand_map;
  const int32_t *n_entries;
  const int32_t *q_pos;
  int32_t nq;
  int32_t T[2];
  int32_t *out[2];
  int32_t out_stride[2];
};

struct AttendArgs {
  DevCache c;
  const int32_t *idx;  // [rows][k]
  int32_t k;
  const float *q;      // [rows][16][512]
  // window
  const uint8_t *win_codes;
  const float *win_row_scale;
  const int32_t *win_len, *win_pos0;
  int32_t win_rows, win_window, win_cap;  // win_cap = rows scanned per query
  const int32_t *q_pos;
  int32_t nq;
  float sm_scale;
  float *part;   // [G][2][16][kPartStride]: partials of rows cut between workgroups
};

// Attention work split: units of 128 positions (U per row, T = rows * U in
// all) shared out over G workgroups; out/lse receive the rows.
constexpr int kSegMaxWg = 256;
struct SegArgs {
  int64_t T;
  int32_t U, G;
  int32_t xcd;  // 1: workgroups renumbered so that each XCD runs a contiguous block of rows
  float *out, *lse;
};

struct MergeArgs {
  const float *part;
};

// New compressed entries written into a paged cache (one FP4 row each).
struct AppendArgs {
  uint8_t *kv_codes, *kv_scales, *ix_codes, *ix_scales;
  const int32_t *block_table;
  int32_t page_shift, max_pages, num_pages;
  const float *kv;       // [batch][n_new][512]
  const float *ix;       // [batch][n_new][64] or null
  const int32_t *entry;  // [batch][n_new] entry index, < 0: none
  int32_t batch, n_new;
};

hipError_t launch_quant_fp4(const float *x, int64_t n_rows, int32_t channels, uint8_t *codes,
                            uint8_t *scales, hipStream_t st);
hipError_t launch_kv_append(const AppendArgs &a, hipStream_t st);
hipError_t launch_window_append(uint8_t *codes, float *row_scale, int32_t rows, const float *x,
                                const int32_t *row, int32_t batch, int32_t n_new, hipStream_t st);
hipError_t launch_fill_u32(uint32_t *p, int64_t n, uint32_t v, hipStream_t st);
hipError_t launch_index_score(const ScoreArgs &a, int rows, hipStream_t st);
hipError_t launch_hist(const float *scores, int32_t n_cols, int rows, uint32_t *hist,
                       hipStream_t st, const int32_t *n_entries = nullptr,
                       const int32_t *q_pos = nullptr, int32_t nq = 1);
hipError_t launch_prefill_score(const ScoreArgs &a, int batch, hipStream_t st);

// Prefill chunk, scoring fused with the per-query top-K (no score matrix):
// rows of at most kPrefillTopkMaxCols entries, 16 query rows per workgroup.
constexpr int32_t kPrefillTopkMaxCols = 32768;
struct PrefillTopkArgs {
  DevCache c;
  const uint8_t *qix_codes, *qix_scales;  // [rows][4][32], [rows][4][4]
  const float *w;                         // [rows][4]
  const int32_t *q_pos;                   // [rows] or null
  int32_t nq;
  int32_t n_cols;                         // cache capacity (bounds the visible entries)
  int32_t k;
  int32_t *idx_out;                       // [rows][k] ascending ids, then -1
};
hipError_t launch_prefill_topk(const PrefillTopkArgs &a, int batch, hipStream_t st);
// several query rows per request (2..63): key loads shared by the rows; no histogram
hipError_t launch_index_score_mq(const ScoreArgs &a, int batch, hipStream_t st);
hipError_t launch_compact(const CompactArgs &a, int rows, hipStream_t st);
hipError_t launch_final(const FinalArgs &a, int rows, int ntarget, hipStream_t st);
hipError_t launch_select_direct(const DirectArgs &a, int rows, int ntarget, hipStream_t st);
// one workgroup per row of up to kSelectRowMax columns, histogram in LDS; ids in column order
constexpr int kSelectRowMax = 16384;
hipError_t launch_sel_rowwise(const DirectArgs &a, int rows, int ntarget, hipStream_t st);
hipError_t launch_sort_rows(int32_t *ids, int32_t stride, int32_t T, int rows, hipStream_t st);
// max_slots: most workgroups sharing one row (2 or more: rows cut between
// workgroups are combined by a merge pass)
hipError_t launch_attend_seg(const AttendArgs &a, const SegArgs &s, int max_slots, hipStream_t st);
// the same work split with each of four waves taking 32 positions of every unit on its own
hipError_t launch_attend_wave(const AttendArgs &a, const SegArgs &s, int max_slots, hipStream_t st);
// the pass that combines the partials of rows cut between workgroups (max_slots >= 2)
hipError_t launch_merge_seg(const AttendArgs &a, const SegArgs &s, int max_slots, hipStream_t st);
hipError_t launch_dequant_fp4(const uint8_t *codes, const uint8_t *scales, int64_t n_rows,
                              int32_t channels, uint16_t *out, hipStream_t st);
hipError_t launch_dequant_e4m3(const uint8_t *bytes, int64_t n, float *out, hipStream_t st);
hipError_t launch_stream_read(const void *p, int64_t n_bytes, uint32_t *sink, int blocks, hipStream_t st);

constexpr int kPartStride = CSA2_D + 4;  // per head: 512 unnormalised outputs, max, sum, 2 pad

}  // namespace csa2
