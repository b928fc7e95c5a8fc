// Lightning-indexer scoring of a prefill chunk, gfx950: many queries of one
// request against the same entries (DeepSeek V4.1 Flash summaries: "DeepSeek
// V4.1 Flash 如何靠压缩 KV 缓存实现小模型干翻大模型", sections "CSA2" and
// "FP4 量化 + Bounded Replay"; block-causal visibility as for the decode
// scoring).
//
// Scoring a chunk of queries is a dense contraction (queries x entries x 64
// channels, per indexer head), so here M = 16 queries, N = 16 entries and
// K = the 64 channels of one head in two steps of v_mfma_f32_16x16x32_f16.
// Both operands are dequantised exactly to fp16 in registers (E2M1 x E4M3
// needs at most 6 significant bits), so every product is exact in fp32; each
// head's dot is accumulated in fp32 by the matrix core. K order: step ks,
// lane quarter g', element j stand for channel 16 g' + 8 ks + j, so a lane's
// two steps cover one 16-channel scale group (8 code bytes + 1 scale byte).
// The epilogue applies ReLU, the per-query head weights and the head sum.
// A workgroup (4 waves) takes 64 consecutive queries and PF_E consecutive
// entries; it stops early when the whole chunk lies past every query's
// visible limit (block-causal prefill), and writes only visible columns
// (or -inf past the limit when write_masked is set).
#include "csa2_dev.h"
#include "kernels.h"
#include "prefill_ops.h"

namespace csa2 {

#define PF_Q 64
#define PF_E 512
#define PF_BATCH 8   // 16-entry tiles whose loads are issued together
#define PF_PAGES (PF_E / 16 + 2)

__global__ __launch_bounds__(256) void k_prefill_score(ScoreArgs a, int32_t qblocks) {
  __shared__ int32_t spage[PF_PAGES];
  __shared__ int32_t smax[4];
  const int b = blockIdx.y / qblocks, qb = blockIdx.y % qblocks;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int m = lane & 15, gq = lane >> 4;  // operand row (query / entry) and channel quarter
  const int64_t e0 = (int64_t)blockIdx.x * PF_E;
  const int32_t nent = a.c.n_entries[b];
  // visible limit of each of the lane's 4 result rows (queries 16 wave + 4 gq + i)
  int32_t lim_r[4];
  bool qok_r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = qb * PF_Q + wave * 16 + 4 * gq + i;
    qok_r[i] = t < a.nq;
    lim_r[i] = qok_r[i] ? visible_entries(a.c, a.q_pos, b, a.nq, t) : 0;
  }
  // the block's largest limit decides whether any of its columns are visible
  {
    int32_t mx = max(max(lim_r[0], lim_r[1]), max(lim_r[2], lim_r[3]));
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) mx = max(mx, __shfl_xor(mx, off));
    if (lane == 0) smax[wave] = mx;
  }
  const int shift = a.c.page_shift;
  const int64_t pg0 = e0 >> shift;
  const int64_t e_end = min(e0 + (int64_t)PF_E, (int64_t)a.n_cols);
  const int64_t npg = ((e_end - 1) >> shift) - pg0 + 1;
  for (int i = tid; i < npg && i < PF_PAGES; i += 256) {
    const int64_t pg = pg0 + i;
    spage[i] = (pg < a.c.max_pages) ? a.c.block_table[(int64_t)b * a.c.max_pages + pg] : -1;
  }
  __syncthreads();
  const int32_t blk_lim = max(max(smax[0], smax[1]), max(smax[2], smax[3]));
  const int64_t work_end = a.write_masked ? e_end : min(e_end, (int64_t)blk_lim);
  if (e0 >= work_end) return;  // uniform: nothing visible, nothing to write

  // A operands: query m of the wave, every head, both steps
  const int t_a = qb * PF_Q + wave * 16 + m;
  const bool qok_a = t_a < a.nq;
  const int64_t row_a = (int64_t)b * a.nq + min(t_a, a.nq - 1);
  v8h qa[CSA2_HI][2];
#pragma unroll
  for (int h = 0; h < CSA2_HI; ++h) {
    const v2f c = *(const v2f *)(a.qix_codes + (row_a * CSA2_HI + h) * 32 + 8 * gq);
    const uint32_t sb = a.qix_scales[(row_a * CSA2_HI + h) * 4 + gq];
    const _Float16 s = qok_a ? e4m3_to_f16(sb) : (_Float16)0.f;
    qa[h][0] = fp4x8_dequant((uint32_t)__float_as_int(c[0]), s);
    qa[h][1] = fp4x8_dequant((uint32_t)__float_as_int(c[1]), s);
  }
  // head weights of the lane's 4 result rows
  float wr[4][CSA2_HI];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = min(qb * PF_Q + wave * 16 + 4 * gq + i, a.nq - 1);
#pragma unroll
    for (int h = 0; h < CSA2_HI; ++h) wr[i][h] = a.w[((int64_t)b * a.nq + t) * CSA2_HI + h];
  }
  const int64_t out_row0 = (int64_t)b * a.nq + qb * PF_Q + wave * 16 + 4 * gq;

  for (int64_t tb = e0; tb < work_end; tb += 16 * PF_BATCH) {
    // every load of the batch first (row 0 stands in for a missing entry)
    v2f code[PF_BATCH];
    uint32_t scb[PF_BATCH];
    bool eok[PF_BATCH];
#pragma unroll
    for (int u = 0; u < PF_BATCH; ++u) {
      const int64_t e = tb + 16 * u + m;
      const int32_t page = spage[min(max((e >> shift) - pg0, (int64_t)0), (int64_t)PF_PAGES - 1)];
      eok[u] = e < e_end && e < nent && page >= 0 && page < a.c.num_pages;
      const int64_t crow = eok[u] ? ((int64_t)page << shift) + (e & ((1 << shift) - 1)) : 0;
      code[u] = *(const v2f *)(a.c.ix_codes + crow * 32 + 8 * gq);
      scb[u] = a.c.ix_scales[crow * 4 + gq];
    }
#pragma unroll
    for (int u = 0; u < PF_BATCH; ++u) {
      const int64_t et = tb + 16 * u;  // first entry of the tile
      if (et >= work_end) break;       // uniform
      const _Float16 s = e4m3_to_f16(scb[u]);
      const v8h b0 = fp4x8_dequant((uint32_t)__float_as_int(code[u][0]), s);
      const v8h b1 = fp4x8_dequant((uint32_t)__float_as_int(code[u][1]), s);
      v4f acc[CSA2_HI];
#pragma unroll
      for (int h = 0; h < CSA2_HI; ++h) {
        acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[h][0], b0, (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[h][1], b1, acc[h], 0, 0, 0);
      }
      // lane holds dots of queries 4 gq + i with entry et + m, the entry this
      // lane loaded a quarter of (so eok[u] is its validity)
      const int64_t e = et + m;
      const bool ev = eok[u];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float sc = 0.f;
#pragma unroll
        for (int h = 0; h < CSA2_HI; ++h) sc = fmaf(wr[i][h], fmaxf(acc[h][i], 0.f), sc);
        const bool vis = qok_r[i] && ev && e < lim_r[i];
        if (qok_r[i] && e < e_end && (vis || a.write_masked))
          a.scores[(out_row0 + i) * a.n_cols + e] = vis ? sc : -INFINITY;
      }
    }
  }
}

// Pages of at least 16 entries (the page ids of a chunk are cached in LDS).
hipError_t launch_prefill_score(const ScoreArgs &a, int batch, hipStream_t st) {
  if ((PF_E >> a.c.page_shift) + 2 > PF_PAGES || a.cand) return hipErrorInvalidValue;
  const int32_t qblocks = (a.nq + PF_Q - 1) / PF_Q;
  dim3 grid((unsigned)((a.n_cols + PF_E - 1) / PF_E), (unsigned)(batch * qblocks));
  hipLaunchKernelGGL(k_prefill_score, grid, dim3(256), 0, st, a, qblocks);
  return hipGetLastError();
}

}  // namespace csa2
