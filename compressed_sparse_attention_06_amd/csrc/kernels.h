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

// Candidate compaction against the coarse threshold bin.
struct CompactArgs {
  const float *scores;
  int32_t n_cols;
  const int32_t *cand_map;   // [rows][n_cols] ids or null (id = column)
  const int32_t *n_entries;  // [batch] or null: limit columns to the visible entries
  const int32_t *q_pos;      // [rows] or null
  int32_t nq;
  const uint32_t *hist;      // [rows][HIST_BINS]
  int32_t T;                 // target count
  int32_t *out;              // [rows][out_stride]
  int32_t out_stride;
  int32_t *cand_cols;        // [rows][n_cols]
  uint32_t *ctr;             // [rows][4]: 0 = emitted, 1 = candidates
  int32_t chunk;
};

struct FinalArgs {
  const float *scores;
  int32_t n_cols;
  const int32_t *cand_map;
  const int32_t *n_entries;
  const int32_t *q_pos;
  int32_t nq;
  const uint32_t *hist;       // null: direct mode (every column is an item)
  const int32_t *cand_cols;   // compact mode lists
  const uint32_t *ctr;
  int32_t T;
  int32_t *outT;              // [rows][outT_stride]
  int32_t outT_stride;
  int32_t sortT;              // sort outT ascending (T <= CSA2_MAX_K)
  int32_t K2;                 // > 0: also select top K2 of the T-set (keys scores[row][id])
  int32_t *outK2;
  int32_t K2_stride;
  int32_t id_limit;           // every id is < id_limit
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
  int32_t rows_per_split;
  int32_t n_split;
  float *part;   // [rows][n_split][16][512 + 2]
};

struct MergeArgs {
  const float *part;
  int32_t n_split;
  float *out, *lse;
};

hipError_t launch_fill_u32(uint32_t *p, int64_t n, uint32_t v, hipStream_t st);
hipError_t launch_index_score(const ScoreArgs &a, int rows, hipStream_t st);
hipError_t launch_hist(const float *scores, int32_t n_cols, int rows, uint32_t *hist,
                       hipStream_t st);
hipError_t launch_compact(const CompactArgs &a, int rows, hipStream_t st);
hipError_t launch_final(const FinalArgs &a, int rows, hipStream_t st);
hipError_t launch_attend(const AttendArgs &a, int rows, hipStream_t st);
hipError_t launch_merge(const MergeArgs &a, int rows, hipStream_t st);
hipError_t launch_dequant_fp4(const uint8_t *codes, const uint8_t *scales, int64_t n_rows,
                              int32_t channels, uint16_t *out, hipStream_t st);
hipError_t launch_dequant_e4m3(const uint8_t *bytes, int64_t n, float *out, hipStream_t st);

constexpr int kPartStride = CSA2_D + 2;  // per head: 512 unnormalised outputs, max, sum

}  // namespace csa2
