// Lightning-indexer scoring for decode, gfx950.
//
// Score of entry s for one query: I_s = sum_{h<4} w_h * max(0, q_h . k_s),
// q_h and k_s 64-channel FP4 rows with one E4M3 scale per 16 channels
// (DeepSeek V4.1 Flash summaries: "DeepSeek V4.1 Flash 如何靠压缩 KV 缓存实现小模型
// 干翻大模型", sections "CSA2" and "FP4 量化 + Bounded Replay").
//
// Design. Decode scoring streams 36 bytes per entry (32 code bytes + 4 scale
// bytes) and does 256 multiply-adds on them. At HBM rate that is ~177 VALU
// lane-ops per entry on MI355X, about what a nibble-decode + FMA loop needs,
// so a VALU version would be ALU-bound. The FP4 matrix core consumes the raw
// E2M1 codes directly: one v_mfma_scale_f32_16x16x128_f8f6f4 (both operands
// FP4, unit block scales) gives the 16 products D[h][g][s] = sum over the 16
// channels of group g of E2M1(q_h) * E2M1(k_s), exact in fp32, for 16 entries.
// The A operand is block-diagonal: row (h, g) holds q_h's codes in group g
// and zeros elsewhere, so all 16 rows of the tile do useful work. The K
// dimension is 128 codes, two entries' worth of 64: the same B registers feed
// a second MFMA whose A operand sits in the upper half, so one 16-byte load
// per lane covers 32 entries (1 KB, contiguous within a page). The epilogue
// applies the two E4M3 scales per group in fp32, the ReLU, the head weight,
// and sums the 4 heads across lanes.
//
// Lane layouts (checked on gfx950): for 16x16x128 FP4 lane l holds row/col
// l%16 and K = 32*(l/16)+j in nibble j%8 of dword j/8; C lane l holds rows
// 4*(l/16)+i of column l%16.
#include "csa2_dev.h"
#include "kernels.h"

namespace csa2 {

#define SC_UNROLL 4          // 32-entry groups per wave batch (all loads issued first)
#define SC_MAX_PAGES 80      // page ids cached per workgroup (chunk / 32 + 2)

// CAND: columns are a candidate list of entry ids; PCACHE: contiguous columns
// whose page ids are cached in LDS (pages of at least 32 entries). Both are
// template parameters so no branch sits between a load and its use.
// One chunk of columns [col0, col0 + chunk) of score row r. Candidate
// columns are all scored (pads and ids past the visible entries give -inf);
// entry columns are scored up to the row's visible entries, and past them
// either left alone or, with write_masked, set to -inf by plain stores.
template <bool CAND, bool PCACHE>
__device__ __forceinline__ void score_chunk(const ScoreArgs &a, int r, int64_t col0, uint32_t *lhist,
                                            int32_t *spage) {
  const int b = r / a.nq, t = r % a.nq;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t nent = a.c.n_entries[b];
  const int32_t V = visible_entries(a.c, a.q_pos, b, a.nq, t);
  const int64_t col_end = min(col0 + (int64_t)a.chunk, (int64_t)a.n_cols);
  const int64_t work_end = CAND ? col_end : min(col_end, (int64_t)V);
  const bool do_hist = a.hist != nullptr;
  if (!CAND && a.write_masked) {  // masked tail: -inf, no key loads
    float *sr = a.scores + (int64_t)r * a.n_cols;
    for (int64_t c = max(col0, work_end) + threadIdx.x; c < col_end; c += 256) sr[c] = -INFINITY;
  }
  if (col0 < work_end) {  // uniform across the block
  for (int i = threadIdx.x; i < HIST_BINS; i += 256) lhist[i] = 0;
  // Full rows with pages of >= 32 entries: cache this chunk's page ids in LDS
  const int shift = a.c.page_shift;
  const int64_t pg0 = col0 >> shift;
  if (PCACHE) {
    const int64_t npg = ((col_end - 1) >> shift) - pg0 + 1;
    for (int i = threadIdx.x; i < npg; i += 256) {
      const int64_t pg = pg0 + i;
      spage[i] = (pg < a.c.max_pages) ? a.c.block_table[(int64_t)b * a.c.max_pages + pg] : -1;
    }
  }
  __syncthreads();

  // A operands (block-diagonal indexer query), rows m = 4h + g.
  const int m = lane & 15, h = m >> 2, g = m & 3, kg = lane >> 4;
  const uint32_t *qc = (const uint32_t *)(a.qix_codes + ((int64_t)r * CSA2_HI + h) * 32);
  v8i A1 = {0, 0, 0, 0, 0, 0, 0, 0}, A2 = {0, 0, 0, 0, 0, 0, 0, 0};
  {
    const uint32_t d0 = qc[2 * g], d1 = qc[2 * g + 1];
    if (kg == (g >> 1)) { A1[2 * (g & 1)] = (int)d0; A1[2 * (g & 1) + 1] = (int)d1; }
    if (kg == 2 + (g >> 1)) { A2[2 * (g & 1)] = (int)d0; A2[2 * (g & 1) + 1] = (int)d1; }
  }
  // Epilogue constants: C rows of this lane are (head hc, group i), i = 0..3.
  const int hc = lane >> 4;
  float sq[4];
  {
    const uint32_t sw = *(const uint32_t *)(a.qix_scales + ((int64_t)r * CSA2_HI + hc) * 4);
    v2f lo = e4m3x2_lo_to_f32(sw), hi = e4m3x2_hi_to_f32(sw);
    sq[0] = lo[0]; sq[1] = lo[1]; sq[2] = hi[0]; sq[3] = hi[1];
  }
  const float wh = a.w[(int64_t)r * CSA2_HI + hc];
  const int64_t out_base = (int64_t)r * a.n_cols;
  const int32_t *cand_row = a.cand ? a.cand + (int64_t)r * a.n_cand : nullptr;
  const int half = (lane >> 4) & 1;
  const int lcol = ((lane >> 5) << 4) + (lane & 15);  // column this lane loads within a group

  for (int64_t e_base = col0 + wave * 32; e_base < work_end; e_base += 4 * 32 * SC_UNROLL) {
    // Loads are issued unconditionally from clamped, in-range addresses and
    // batched per dependency level (candidate id -> page id -> codes), so a
    // level's loads are all in flight together; validity is applied after.
    int32_t row_l[SC_UNROLL];
    int32_t sid_l[SC_UNROLL];
#pragma unroll
    for (int u = 0; u < SC_UNROLL; ++u) {
      const int64_t jl = e_base + (int64_t)u * 128 + lcol;
      const int64_t jc = min(jl, col_end - 1);
      if constexpr (CAND) sid_l[u] = cand_row[jc];
      else sid_l[u] = (int32_t)jl;
    }
    int32_t page_l[SC_UNROLL];
#pragma unroll
    for (int u = 0; u < SC_UNROLL; ++u) {
      const int32_t sc = min(max(sid_l[u], 0), max(nent - 1, 0));
      if constexpr (PCACHE) {
        page_l[u] = spage[min(max((int64_t)(sc >> shift) - pg0, (int64_t)0), (int64_t)SC_MAX_PAGES - 1)];
      } else {
        const int32_t pg = min(sc >> shift, a.c.max_pages - 1);
        page_l[u] = a.c.block_table[(int64_t)b * a.c.max_pages + pg];
      }
    }
#pragma unroll
    for (int u = 0; u < SC_UNROLL; ++u) {
      const int64_t e0 = e_base + (int64_t)u * 128;
      const int64_t jl = e0 + lcol;
      const int32_t sidx = sid_l[u];
      const int32_t page = page_l[u];
      const bool ok = e0 < work_end && jl < col_end && sidx >= 0 && sidx < V && sidx < nent &&
                      page >= 0 && page < a.c.num_pages;
      row_l[u] = ok ? (page << shift) + (sidx & ((1 << shift) - 1)) : -1;
    }
    // 2. issue every data load of the batch (row 0 stands in for missing rows)
    v4i code[SC_UNROLL];
    uint32_t ks1[SC_UNROLL], ks2[SC_UNROLL];
    int32_t row1[SC_UNROLL], row2[SC_UNROLL];
#pragma unroll
    for (int u = 0; u < SC_UNROLL; ++u) {
      row1[u] = __shfl(row_l[u], lane & 15);
      row2[u] = __shfl(row_l[u], 32 + (lane & 15));
      code[u] = *(const v4i *)(a.c.ix_codes + (int64_t)max(row_l[u], 0) * 32 + half * 16);
      ks1[u] = *(const uint32_t *)(a.c.ix_scales + (int64_t)max(row1[u], 0) * 4);
      ks2[u] = *(const uint32_t *)(a.c.ix_scales + (int64_t)max(row2[u], 0) * 4);
    }
#pragma unroll
    for (int u = 0; u < SC_UNROLL; ++u)
      if (row_l[u] < 0) code[u] = (v4i){0, 0, 0, 0};
    // 3. compute
#pragma unroll
    for (int u = 0; u < SC_UNROLL; ++u) {
      const int64_t e0 = e_base + (int64_t)u * 128;
      if (e0 >= work_end) break;  // uniform within the wave
      const v8i B = {code[u][0], code[u][1], code[u][2], code[u][3], 0, 0, 0, 0};
      const v4f z = {0.f, 0.f, 0.f, 0.f};
      const v4f C1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A1, B, z, 4, 4, 0, 127, 0, 127);
      const v4f C2 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A2, B, z, 4, 4, 0, 127, 0, 127);
      float t1, t2;
      {
        const v2f lo = e4m3x2_lo_to_f32(ks1[u]), hi = e4m3x2_hi_to_f32(ks1[u]);
        float p = C1[0] * (sq[0] * lo[0]);
        p = fmaf(C1[1], sq[1] * lo[1], p);
        p = fmaf(C1[2], sq[2] * hi[0], p);
        p = fmaf(C1[3], sq[3] * hi[1], p);
        t1 = wh * fmaxf(p, 0.f);
      }
      {
        const v2f lo = e4m3x2_lo_to_f32(ks2[u]), hi = e4m3x2_hi_to_f32(ks2[u]);
        float p = C2[0] * (sq[0] * lo[0]);
        p = fmaf(C2[1], sq[1] * lo[1], p);
        p = fmaf(C2[2], sq[2] * hi[0], p);
        p = fmaf(C2[3], sq[3] * hi[1], p);
        t2 = wh * fmaxf(p, 0.f);
      }
      // sum the four heads (lanes n, n+16, n+32, n+48 hold heads 0..3 of column n)
      t1 = sum_rows4(t1);
      t2 = sum_rows4(t2);
      if (lane < 32) {
        const int64_t col = e0 + lane;  // lanes 0..15: first tile; 16..31: second tile
        const float sc = (lane < 16) ? t1 : t2;
        const int32_t rv = (lane < 16) ? row1[u] : row2[u];
        if (col < col_end) {
          const float o = (rv >= 0) ? sc : -INFINITY;
          a.scores[out_base + col] = o;
          if (do_hist && rv >= 0) atomicAdd(&lhist[score_key(o) >> HIST_SHIFT], 1u);
        }
      }
    }
  }
  if (do_hist) {
    __syncthreads();
    uint32_t *gh = a.hist + (int64_t)r * HIST_BINS;
    for (int i = threadIdx.x; i < HIST_BINS; i += 256) {
      const uint32_t v = lhist[i];
      if (v) atomicAdd(&gh[i], v);
    }
  }
  }  // active workgroup
}

template <bool CAND, bool PCACHE>
__global__ __launch_bounds__(256) void k_index_score(ScoreArgs a) {
  __shared__ uint32_t lhist[HIST_BINS];
  __shared__ int32_t spage[SC_MAX_PAGES];
  score_chunk<CAND, PCACHE>(a, blockIdx.y, (int64_t)blockIdx.x * a.chunk, lhist, spage);
}

hipError_t launch_index_score(const ScoreArgs &a, int rows, hipStream_t st) {
  const int64_t chunks = (a.n_cols + a.chunk - 1) / a.chunk;
  dim3 grid((unsigned)chunks, (unsigned)rows);
  // a chunk spans at most chunk / page + 1 pages
  const bool pcache = a.c.page_shift >= 5 && (a.chunk >> a.c.page_shift) + 2 <= SC_MAX_PAGES;
  if (a.cand)
    hipLaunchKernelGGL((k_index_score<true, false>), grid, dim3(256), 0, st, a);
  else if (pcache)
    hipLaunchKernelGGL((k_index_score<false, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((k_index_score<false, false>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---- several query rows of one request per workgroup --------------------------------
// Speculative verification (a few draft tokens per request) scores every entry
// for each query row. The entries' codes are loaded once per workgroup and
// feed two MFMAs per query row (QB rows per workgroup), so the key bytes
// cross HBM once per request instead of once per row. Each row keeps its own
// visibility limit (block-causal among the newest entries): columns past it
// are written as -inf. No histogram here: the host adds one pass when the
// chunked selection needs it.
template <int QB, bool PCACHE>
__global__ __launch_bounds__(256) void k_index_score_mq(ScoreArgs a, int32_t qblocks) {
  __shared__ int32_t spage[SC_MAX_PAGES];
  const int b = blockIdx.y / qblocks, t0 = (blockIdx.y % qblocks) * QB;
  const int nqb = min(QB, a.nq - t0);  // query rows in this workgroup (uniform)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int32_t nent = a.c.n_entries[b];
  int32_t V[QB];
  int32_t vmax = 0;
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    V[q] = q < nqb ? visible_entries(a.c, a.q_pos, b, a.nq, t0 + q) : 0;
    vmax = max(vmax, V[q]);
  }
  const int64_t col0 = (int64_t)blockIdx.x * a.chunk;
  const int64_t col_end = min(col0 + (int64_t)a.chunk, (int64_t)a.n_cols);
  const int64_t work_end = a.write_masked ? col_end : min(col_end, (int64_t)vmax);
  if (col0 >= work_end) return;  // uniform across the block
  const int shift = a.c.page_shift;
  const int64_t pg0 = col0 >> shift;
  if (PCACHE) {
    const int64_t npg = ((col_end - 1) >> shift) - pg0 + 1;
    for (int i = threadIdx.x; i < npg; i += 256) {
      const int64_t pg = pg0 + i;
      spage[i] = (pg < a.c.max_pages) ? a.c.block_table[(int64_t)b * a.c.max_pages + pg] : -1;
    }
  }
  __syncthreads();

  // per query row: block-diagonal A operands (rows m = 4h + g), epilogue constants
  const int m = lane & 15, h = m >> 2, g = m & 3, kg = lane >> 4;
  const int hc = lane >> 4;
  v8i A1[QB], A2[QB];
  float sq[QB][4], wh[QB];
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    const int64_t r = (int64_t)b * a.nq + t0 + min(q, nqb - 1);
    const uint32_t *qc = (const uint32_t *)(a.qix_codes + (r * CSA2_HI + h) * 32);
    A1[q] = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
    A2[q] = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
    const uint32_t d0 = qc[2 * g], d1 = qc[2 * g + 1];
    if (kg == (g >> 1)) { A1[q][2 * (g & 1)] = (int)d0; A1[q][2 * (g & 1) + 1] = (int)d1; }
    if (kg == 2 + (g >> 1)) { A2[q][2 * (g & 1)] = (int)d0; A2[q][2 * (g & 1) + 1] = (int)d1; }
    const uint32_t sw = *(const uint32_t *)(a.qix_scales + (r * CSA2_HI + hc) * 4);
    const v2f lo = e4m3x2_lo_to_f32(sw), hi = e4m3x2_hi_to_f32(sw);
    sq[q][0] = lo[0];
    sq[q][1] = lo[1];
    sq[q][2] = hi[0];
    sq[q][3] = hi[1];
    wh[q] = a.w[r * CSA2_HI + hc];
  }
  const int half = (lane >> 4) & 1;
  const int lcol = ((lane >> 5) << 4) + (lane & 15);

  for (int64_t e_base = col0 + wave * 32; e_base < work_end; e_base += 4 * 32 * SC_UNROLL) {
    int32_t row_l[SC_UNROLL], page_l[SC_UNROLL];
#pragma unroll
    for (int u = 0; u < SC_UNROLL; ++u) {
      const int64_t jl = e_base + (int64_t)u * 128 + lcol;
      const int32_t sc = (int32_t)min(jl, (int64_t)max(nent - 1, 0));
      if constexpr (PCACHE) {
        page_l[u] = spage[min(max((int64_t)(sc >> shift) - pg0, (int64_t)0), (int64_t)SC_MAX_PAGES - 1)];
      } else {
        const int32_t pg = min(sc >> shift, a.c.max_pages - 1);
        page_l[u] = a.c.block_table[(int64_t)b * a.c.max_pages + pg];
      }
    }
#pragma unroll
    for (int u = 0; u < SC_UNROLL; ++u) {
      const int64_t e0 = e_base + (int64_t)u * 128;
      const int64_t jl = e0 + lcol;
      const int32_t page = page_l[u];
      const bool ok = e0 < work_end && jl < col_end && jl < nent && page >= 0 && page < a.c.num_pages;
      row_l[u] = ok ? (page << shift) + (int32_t)(jl & ((1 << shift) - 1)) : -1;
    }
    v4i code[SC_UNROLL];
    uint32_t ks1[SC_UNROLL], ks2[SC_UNROLL];
    int32_t row1[SC_UNROLL], row2[SC_UNROLL];
#pragma unroll
    for (int u = 0; u < SC_UNROLL; ++u) {
      row1[u] = __shfl(row_l[u], lane & 15);
      row2[u] = __shfl(row_l[u], 32 + (lane & 15));
      code[u] = *(const v4i *)(a.c.ix_codes + (int64_t)max(row_l[u], 0) * 32 + half * 16);
      ks1[u] = *(const uint32_t *)(a.c.ix_scales + (int64_t)max(row1[u], 0) * 4);
      ks2[u] = *(const uint32_t *)(a.c.ix_scales + (int64_t)max(row2[u], 0) * 4);
    }
#pragma unroll
    for (int u = 0; u < SC_UNROLL; ++u)
      if (row_l[u] < 0) code[u] = (v4i){0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < SC_UNROLL; ++u) {
      const int64_t e0 = e_base + (int64_t)u * 128;
      if (e0 >= work_end) break;  // uniform within the wave
      const v8i B = {code[u][0], code[u][1], code[u][2], code[u][3], 0, 0, 0, 0};
      const v4f z = {0.f, 0.f, 0.f, 0.f};
      const v2f l1 = e4m3x2_lo_to_f32(ks1[u]), h1 = e4m3x2_hi_to_f32(ks1[u]);
      const v2f l2 = e4m3x2_lo_to_f32(ks2[u]), h2 = e4m3x2_hi_to_f32(ks2[u]);
      const int64_t col = e0 + lane;  // lanes 0..15: first tile; 16..31: second tile
      const int32_t rv = (lane < 16) ? row1[u] : row2[u];
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        if (q >= nqb) break;  // uniform
        const v4f C1 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A1[q], B, z, 4, 4, 0, 127, 0, 127);
        const v4f C2 = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A2[q], B, z, 4, 4, 0, 127, 0, 127);
        float p1 = C1[0] * (sq[q][0] * l1[0]);
        p1 = fmaf(C1[1], sq[q][1] * l1[1], p1);
        p1 = fmaf(C1[2], sq[q][2] * h1[0], p1);
        p1 = fmaf(C1[3], sq[q][3] * h1[1], p1);
        float p2 = C2[0] * (sq[q][0] * l2[0]);
        p2 = fmaf(C2[1], sq[q][1] * l2[1], p2);
        p2 = fmaf(C2[2], sq[q][2] * h2[0], p2);
        p2 = fmaf(C2[3], sq[q][3] * h2[1], p2);
        const float t1 = sum_rows4(wh[q] * fmaxf(p1, 0.f)), t2 = sum_rows4(wh[q] * fmaxf(p2, 0.f));
        if (lane < 32 && col < col_end) {
          const float sc = (lane < 16) ? t1 : t2;
          const int64_t r = (int64_t)b * a.nq + t0 + q;
          a.scores[r * a.n_cols + col] = (rv >= 0 && col < V[q]) ? sc : -INFINITY;
        }
      }
    }
  }
}

hipError_t launch_index_score_mq(const ScoreArgs &a, int batch, hipStream_t st) {
  if (a.cand || a.nq < 2) return hipErrorInvalidValue;
  const int qb = a.nq <= 2 ? 2 : (a.nq <= 4 ? 4 : 8);
  const int32_t qblocks = (a.nq + qb - 1) / qb;
  const int64_t chunks = (a.n_cols + a.chunk - 1) / a.chunk;
  const dim3 grid((unsigned)chunks, (unsigned)(batch * qblocks));
  const bool pcache = a.c.page_shift >= 5 && (a.chunk >> a.c.page_shift) + 2 <= SC_MAX_PAGES;
#define CSA2_MQ_LAUNCH(Q)                                                                    \
  if (pcache)                                                                                \
    hipLaunchKernelGGL((k_index_score_mq<Q, true>), grid, dim3(256), 0, st, a, qblocks);     \
  else                                                                                       \
    hipLaunchKernelGGL((k_index_score_mq<Q, false>), grid, dim3(256), 0, st, a, qblocks);
  if (qb == 2) {
    CSA2_MQ_LAUNCH(2)
  } else if (qb == 4) {
    CSA2_MQ_LAUNCH(4)
  } else {
    CSA2_MQ_LAUNCH(8)
  }
#undef CSA2_MQ_LAUNCH
  return hipGetLastError();
}

}  // namespace csa2
