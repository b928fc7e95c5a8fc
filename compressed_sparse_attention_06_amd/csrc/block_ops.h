// Workgroup-level helpers shared by the scoring and selection kernels.
// Every thread of the workgroup must call each of them (blockDim.x a multiple
// of 64, at most 1024).
#pragma once

#include "csa2_dev.h"

namespace csa2 {

#define DIG_BINS 4096

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts
// within each row of 16 lanes (out-of-row sources read as 0), then the last
// lane of row 0 added to row 1 and row 3 (row_bcast:15) and the last lane of
// row 1 to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false); // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false); // row_bcast:31
  return v;
}

// Reductions over the 64 lanes of a wave, the result in every lane: DPP moves
// within each row of 16 lanes (swap neighbours, swap pairs, mirror within 8,
// mirror within 16), then gfx950's 16- and 32-lane row swaps of the register
// with itself, whose two results together hold both rows of each pair. All
// VALU: no LDS permutes.
template <class OP>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, OP op) {
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op((uint32_t)a[0], (uint32_t)a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op((uint32_t)b[0], (uint32_t)b[1]);
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  return wave_reduce(v, [](uint32_t x, uint32_t y) { return x + y; });
}
__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
  return wave_reduce(v, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
}
__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  return wave_reduce(v, [](uint32_t x, uint32_t y) { return x > y ? x : y; });
}

// Exclusive prefix sum of one value per thread in thread order; returns this
// thread's offset, *total gets the block total. s: blockDim.x / 64 words.
// Wave scans in registers, one LDS exchange of the wave totals.
__device__ inline uint32_t block_exclusive_scan(uint32_t v, uint32_t *s, uint32_t *total) {
  const int t = threadIdx.x, w = t >> 6, nw = blockDim.x >> 6;
  const uint32_t inc = wave_inclusive_scan(v);
  if ((t & 63) == 63) s[w] = inc;
  __syncthreads();
  uint32_t before = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    const uint32_t x = s[i];
    before += (i < w) ? x : 0u;
    tot += x;
  }
  *total = tot;
  __syncthreads();
  return before + inc - v;
}

// Sum of one value per thread, returned to every thread. s: blockDim.x / 64 words.
__device__ inline uint32_t block_sum(uint32_t v, uint32_t *s) {
  const int t = threadIdx.x, nw = blockDim.x >> 6;
  v = wave_sum(v);
  if ((t & 63) == 0) s[t >> 6] = v;
  __syncthreads();
  uint32_t tot = 0;
  for (int i = 0; i < nw; ++i) tot += s[i];
  __syncthreads();
  return tot;
}

// From an NBINS histogram in LDS: the bin holding the `need`-th largest key
// (descending) or smallest (ascending). out[0] = bin, or -1 when the
// histogram holds at most `need` keys; out[1] = keys strictly before that bin
// in the scan direction (all keys when out[0] = -1); out[2] = total.
// NT = blockDim.x; NBINS and NT powers of two. Each thread keeps its
// segment's counts in registers, so the bin is found without a second pass
// over LDS.
template <int NBINS, int NT, bool DESC>
__device__ inline void hist_threshold_n(const uint32_t *h, uint32_t need, uint32_t *scan, int *out) {
  constexpr bool descending = DESC;
  constexpr int PER = NBINS >= NT ? NBINS / NT : 1;
  constexpr int NSEG = NBINS / PER;
  const int t = threadIdx.x;
  // segments in thread order run from the scan's far end; threads past the
  // last segment hold nothing
  const int seg = descending ? t : (NSEG - 1 - t);
  const bool has = t < NSEG;
  uint32_t v[PER];
  const int base = has ? seg * PER : 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) v[i] = h[base + i];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) sum += has ? v[i] : 0u;
  uint32_t total;
  const uint32_t pre = block_exclusive_scan(sum, scan, &total);
  // every thread has passed the scan's barriers: earlier readers of `out` are done
  if (t == 0) out[2] = (int)total;
  if (total <= need) {
    if (t == 0) {
      out[0] = -1;
      out[1] = (int)total;
    }
  } else {
    const uint32_t before = total - pre - sum;  // keys in segments the scan meets first
    if (has && before < need && before + sum >= need) {
      uint32_t cum = before;
      int bin = -1, cb = 0;
#pragma unroll
      for (int k = 0; k < PER; ++k) {
        const int i = descending ? (PER - 1 - k) : k;
        if (bin < 0 && cum + v[i] >= need) {
          bin = seg * PER + i;
          cb = (int)cum;
        }
        cum += v[i];
      }
      out[0] = bin;
      out[1] = cb;
    }
  }
  __syncthreads();
}

}  // namespace csa2
