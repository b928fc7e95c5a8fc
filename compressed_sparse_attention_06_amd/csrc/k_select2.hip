// Top-K selection of rows of up to 16384 columns, gfx950 (each selecting
// layer picks its own Top-K; a Reindex layer rescores the Full layer's
// candidate pool and selects from it: DeepSeek V4.1 Flash summaries,
// "DeepSeek V4.1 Flash深度解析" section on compressed attention gen. 2 and
// "DeepSeek V4.1 Flash 如何靠压缩 KV 缓存实现小模型干翻大模型" section "CSA2").
//
// Order: score descending, entry id ascending on exact ties (order-preserving
// 32-bit keys; the id is the column, or the candidate map's entry at it).
// k_sel_rowwise: one 1024-thread workgroup per row and target holds the row's
// keys (and ids) in registers, bins them over the row's own key range (4096
// bins from its smallest to its largest key), and takes every key above the
// bin that holds the T-th largest; the keys of that bin go to LDS, where the
// `need` best are settled exactly (binned again over their own range, then
// ranked pairwise; radix levels when many keys are equal). The taken columns'
// ids are written in column order, then -1. No global histogram and no fill:
// the scoring kernel before it adds nothing, and this is the only launch.
#include "csa2_dev.h"
#include "kernels.h"
#include "block_ops.h"

namespace csa2 {

#define SR_NT 1024
#define SR_PER 16        // columns per thread in k_sel_rowwise (16 x 1024 = 16384)
#define SR_CAP 8192      // keys of the threshold bin ranked from LDS (row kernel)

// The row read again from global memory when its threshold bin overflows LDS
// (many equal keys): keys outside the bin read as absent.
struct RowBinKeys {
  const float *row;
  const int32_t *map;
  int32_t lim;
  uint32_t kmin;
  int shift, thr;
  __device__ void get(int i, uint32_t &k, int32_t &d) const {
    const uint32_t kk = score_key(row[i]);
    const bool in = i < lim && kk > KEY_NEG_INF && (int)((kk - kmin) >> shift) == thr;
    k = in ? kk : 0u;
    d = map ? map[i] : i;
  }
};

template <bool VEC>
__global__ __launch_bounds__(SR_NT) void k_sel_rowwise(DirectArgs a) {
  __shared__ uint32_t hist[HIST_BINS];
  __shared__ uint32_t ekey[SR_CAP];
  __shared__ int32_t eid[SR_CAP];
  __shared__ uint32_t sk[64];
  __shared__ int32_t sd[64];
  __shared__ uint32_t scan[SR_NT / 64 * 3];
  __shared__ int hout[4];
  __shared__ SelShared<8> sh;
  const int r = blockIdx.x, tg = blockIdx.y, t = threadIdx.x;
  const float *row = a.scores + (int64_t)r * a.n_cols;
  const int32_t *map = a.cand_map ? a.cand_map + (int64_t)r * a.n_cols : nullptr;
  const int32_t lim = row_limit(a.n_entries, a.q_pos, a.nq, r, a.n_cols);
  const int T = a.T[tg];
  int32_t *gout = a.out[tg] + (int64_t)r * a.out_stride[tg];
  const int32_t c0 = t * SR_PER;

  // keys and ids, every load issued unconditionally from an in-range address
  uint32_t key[SR_PER];
  int32_t id[SR_PER];
  if constexpr (VEC) {
#pragma unroll
    for (int j = 0; j < SR_PER / 4; ++j) {
      const int32_t c = min(c0 + 4 * j, a.n_cols - 4);  // in the row even past its end
      const v4f v = *(const v4f *)(row + c);
#pragma unroll
      for (int e = 0; e < 4; ++e) key[4 * j + e] = score_key(v[e]);
      if (map) {
        const v4i m = *(const v4i *)(map + c);
#pragma unroll
        for (int e = 0; e < 4; ++e) id[4 * j + e] = m[e];
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < SR_PER; ++j) key[j] = score_key(row[min(c0 + j, a.n_cols - 1)]);
    if (map) {
#pragma unroll
      for (int j = 0; j < SR_PER; ++j) id[j] = map[min(c0 + j, a.n_cols - 1)];
    }
  }
  if (!map) {
#pragma unroll
    for (int j = 0; j < SR_PER; ++j) id[j] = c0 + j;
  }
  for (int i = t; i < HIST_BINS; i += SR_NT) hist[i] = 0;
  uint32_t valid_m = 0, nv = 0, lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int j = 0; j < SR_PER; ++j) {
    const bool ok = c0 + j < lim && key[j] > KEY_NEG_INF;
    valid_m |= (ok ? 1u : 0u) << j;
    nv += ok ? 1u : 0u;
    lo = ok ? min(lo, key[j]) : lo;
    hi = ok ? max(hi, key[j]) : hi;
  }
  uint32_t n_valid, kmin, kmax;
  block_sum_minmax(nv, lo, hi, scan, n_valid, kmin, kmax);
  uint32_t take_m = valid_m;  // every key when the row holds at most T
  if (n_valid > (uint32_t)T) {  // uniform
    const uint32_t range = kmax - kmin;
    const int bits = range ? 32 - __builtin_clz(range) : 0;
    const int shift = bits > HIST_BITS ? bits - HIST_BITS : 0;
#pragma unroll
    for (int j = 0; j < SR_PER; ++j)
      if ((valid_m >> j) & 1u) atomicAdd(&hist[(key[j] - kmin) >> shift], 1u);
    __syncthreads();
    hist_threshold_n<HIST_BINS, SR_NT, true>(hist, (uint32_t)T, scan, hout);
    const int thr = hout[0], before = hout[1];  // thr >= 0: more than T keys
    uint32_t eq_m = 0;
    take_m = 0;
#pragma unroll
    for (int j = 0; j < SR_PER; ++j) {
      const int bin = (int)((key[j] - kmin) >> shift);
      const uint32_t v = (valid_m >> j) & 1u;
      take_m |= (v && bin > thr ? 1u : 0u) << j;
      eq_m |= (v && bin == thr ? 1u : 0u) << j;
    }
    const int need = T - before;  // >= 1: keys still to take from the bin
    uint32_t F;
    const uint32_t pos = block_exclusive_scan((uint32_t)__popc(eq_m), scan, &F);
    SelRule rule{0u, 0u, 0xFFFFFFFFu};  // everything in the bin
    if ((uint32_t)need < F) {
      if (F <= SR_CAP) {
        uint32_t p = pos;
#pragma unroll
        for (int j = 0; j < SR_PER; ++j) {
          if ((eq_m >> j) & 1u) {
            ekey[p] = key[j];
            eid[p] = id[j];
            ++p;
          }
        }
        __syncthreads();
        rule = list_rule<SR_NT>(ekey, eid, (int)F, need, hist, sk, sd, scan, hout, sh);
      } else {
        rule = block_rule<8, SR_NT>(RowBinKeys{row, map, lim, kmin, shift, thr}, lim, need, sh);
      }
    }
#pragma unroll
    for (int j = 0; j < SR_PER; ++j)
      if (((eq_m >> j) & 1u) && rule_pass(rule, key[j], id[j])) take_m |= 1u << j;
  }
  uint32_t n_taken;
  uint32_t o = block_exclusive_scan((uint32_t)__popc(take_m), scan, &n_taken);
#pragma unroll
  for (int j = 0; j < SR_PER; ++j) {
    if ((take_m >> j) & 1u) {
      if (o < (uint32_t)T) gout[o] = id[j];
      ++o;
    }
  }
  for (int i = (int)min(n_taken, (uint32_t)T) + t; i < T; i += SR_NT) gout[i] = -1;
}

hipError_t launch_sel_rowwise(const DirectArgs &a, int rows, int ntarget, hipStream_t st) {
  if (a.n_cols > kSelectRowMax || a.n_cols < 4) return hipErrorInvalidValue;
  const bool vec = (a.n_cols & 3) == 0 && (((uintptr_t)a.scores) & 15) == 0 &&
                   (!a.cand_map || (((uintptr_t)a.cand_map) & 15) == 0);
  const dim3 grid((unsigned)rows, (unsigned)ntarget);
  if (vec)
    hipLaunchKernelGGL(k_sel_rowwise<true>, grid, dim3(SR_NT), 0, st, a);
  else
    hipLaunchKernelGGL(k_sel_rowwise<false>, grid, dim3(SR_NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa2
