// Workgroup-level helpers shared by the scoring and selection kernels.
// Every thread of the workgroup must call each of them (blockDim.x a multiple
// of 64, at most 1024).
#pragma once

#include "csa2_dev.h"

namespace csa2 {

#define DIG_BINS 4096

// Columns of selection row r that may hold a score: the visible entries of
// its request (when n_entries is given; with q_pos, only those whole at the
// query's position), at most n_cols.
__device__ __forceinline__ int32_t row_limit(const int32_t *n_entries, const int32_t *q_pos,
                                             int nq, int r, int32_t n_cols) {
  int32_t lim = n_cols;
  if (n_entries) {
    int32_t V = n_entries[r / nq];
    if (q_pos) {
      const int64_t vp = ((int64_t)q_pos[r] + 1) / CSA2_TOKENS_PER_ENTRY;
      if (vp < V) V = (int32_t)(vp < 0 ? 0 : vp);
    }
    if (V < lim) lim = V;
  }
  return lim < 0 ? 0 : lim;
}

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

// ---- exact selection at the boundary ------------------------------------------------
template <int BITS>
struct SelShared {
  uint32_t hist[1 << BITS];
  uint32_t scan[16];
  int out[4];
  uint32_t kmin, kmax, mcount, cnt;
};

// An item with key k and id d is selected iff (k & kmask) > kpref, or
// (k & kmask) == kpref and d <= idthr.
struct SelRule {
  uint32_t kmask, kpref, idthr;
};

__device__ __forceinline__ bool rule_pass(const SelRule &R, uint32_t k, int32_t d) {
  const uint32_t km = k & R.kmask;
  return km > R.kpref || (km == R.kpref && (uint32_t)d <= R.idthr);
}

// The rule that keeps the `need` best (key desc, id asc) of the items whose
// key is above KEY_NEG_INF (need >= 1). Keys are settled BITS bits at a time
// after the leading bits every item shares; exact key ties are settled on the
// id the same way.
template <int BITS, int NT, class Acc>
__device__ inline SelRule block_rule(const Acc &acc, int count, int need, SelShared<BITS> &sh) {
  constexpr int NB = 1 << BITS;
  const int t = threadIdx.x, nt = NT;
  if (t == 0) {
    sh.kmin = 0xFFFFFFFFu;
    sh.kmax = 0u;
    sh.mcount = 0;
  }
  __syncthreads();
  {
    uint32_t lo = 0xFFFFFFFFu, hi = 0u, c = 0;
    for (int i = t; i < count; i += nt) {
      uint32_t k;
      int32_t d;
      acc.get(i, k, d);
      if (k > KEY_NEG_INF) {
        lo = min(lo, k);
        hi = max(hi, k);
        ++c;
      }
    }
    if (c) {
      atomicMin(&sh.kmin, lo);
      atomicMax(&sh.kmax, hi);
      atomicAdd(&sh.mcount, c);
    }
  }
  __syncthreads();
  const uint32_t diff = sh.kmin ^ sh.kmax;
  int known = (sh.mcount == 0) ? 32 : (diff ? __clz(diff) : 32);
  uint32_t kmask = known ? (0xFFFFFFFFu << (32 - known)) : 0u;
  uint32_t kpref = sh.kmin & kmask;
  int left = need;
  int eqcnt = (int)sh.mcount;
  bool take_all_eq = (left >= eqcnt);
  __syncthreads();
  while (!take_all_eq && known < 32) {
    const int width = (32 - known) < BITS ? (32 - known) : BITS;
    const int shift = 32 - known - width;
    const uint32_t dmask = (1u << width) - 1u;
    for (int i = t; i < NB; i += nt) sh.hist[i] = 0;
    __syncthreads();
    for (int i = t; i < count; i += nt) {
      uint32_t k;
      int32_t d;
      acc.get(i, k, d);
      if (k > KEY_NEG_INF && (k & kmask) == kpref) atomicAdd(&sh.hist[(k >> shift) & dmask], 1u);
    }
    __syncthreads();
    hist_threshold_n<NB, NT, true>(sh.hist, (uint32_t)left, sh.scan, sh.out);
    const int dsel = sh.out[0];
    if (dsel < 0) {  // every item with this prefix is needed
      take_all_eq = true;
    } else {
      left -= sh.out[1];
      eqcnt = (int)sh.hist[dsel];
      kpref |= (uint32_t)dsel << shift;
      kmask |= dmask << shift;
      known += width;
      take_all_eq = (left >= eqcnt);
    }
    __syncthreads();
  }
  uint32_t idthr = 0xFFFFFFFFu;
  if (!take_all_eq) {  // exact key ties at the boundary: keep the lowest ids
    uint32_t ipref = 0, imask = 0;
    int ib = 32;
    while (ib > 0) {
      const int width = ib < BITS ? ib : BITS;
      const int shift = ib - width;
      const uint32_t dmask = (1u << width) - 1u;
      for (int i = t; i < NB; i += nt) sh.hist[i] = 0;
      __syncthreads();
      for (int i = t; i < count; i += nt) {
        uint32_t k;
        int32_t d;
        acc.get(i, k, d);
        if (k == kpref && ((uint32_t)d & imask) == ipref)
          atomicAdd(&sh.hist[((uint32_t)d >> shift) & dmask], 1u);
      }
      __syncthreads();
      hist_threshold_n<NB, NT, false>(sh.hist, (uint32_t)left, sh.scan, sh.out);
      const int dsel = sh.out[0] < 0 ? (int)dmask : sh.out[0];
      if (sh.out[0] >= 0) left -= sh.out[1];
      ipref |= (uint32_t)dsel << shift;
      imask |= dmask << shift;
      ib -= width;
      __syncthreads();
    }
    idthr = ipref;
  }
  return SelRule{kmask, kpref, idthr};
}

// Items held in LDS as (key[i], id[i]).
struct LdsKeyId {
  const uint32_t *key;
  const int32_t *id;
  __device__ void get(int i, uint32_t &k, int32_t &d) const {
    k = key[i];
    d = id[i];
  }
};

// Sum and min / max over the workgroup in one exchange (s: blockDim.x / 64 x 3 words).
__device__ __forceinline__ void block_sum_minmax(uint32_t v, uint32_t lo, uint32_t hi, uint32_t *s,
                                                 uint32_t &sum, uint32_t &mn, uint32_t &mx) {
  v = wave_sum(v);
  lo = wave_min(lo);
  hi = wave_max(hi);
  const int t = threadIdx.x, nw = blockDim.x >> 6;
  if ((t & 63) == 0) {
    s[3 * (t >> 6)] = v;
    s[3 * (t >> 6) + 1] = lo;
    s[3 * (t >> 6) + 2] = hi;
  }
  __syncthreads();
  sum = 0;
  mn = 0xFFFFFFFFu;
  mx = 0u;
  for (int i = 0; i < nw; ++i) {
    sum += s[3 * i];
    mn = min(mn, s[3 * i + 1]);
    mx = max(mx, s[3 * i + 2]);
  }
  __syncthreads();
}

// The item of rank need - 1 among n <= 64 items in LDS (key[i], id[i]) by
// (key desc, id asc), found by wave 0 comparing every pair, as a rule: an
// item passes iff its key is larger, or equal with an id not above. Every
// thread of the workgroup must call it; sh.kmin / sh.kmax carry the result.
template <int BITS>
__device__ inline SelRule pairwise_rule(const uint32_t *key, const int32_t *id, int n, int need,
                                        SelShared<BITS> &sh) {
  const int t = threadIdx.x;
  if (t < 64) {
    const bool has = t < n;
    const uint32_t kl = has ? key[t] : 0u;
    const uint32_t dl = has ? (uint32_t)id[t] : 0u;
    uint32_t rank = 0;
    for (int j = 0; j < n; ++j) {
      const uint32_t kj = key[j], dj = (uint32_t)id[j];
      rank += (kj > kl || (kj == kl && dj < dl)) ? 1u : 0u;
    }
    // the last item taken: the largest rank below need (equal items share it)
    const uint32_t r1 = (has && rank < (uint32_t)need) ? rank + 1u : 0u;
    const uint32_t rmax = wave_max(r1);
    if (has && r1 == rmax) {
      sh.kmin = kl;
      sh.kmax = dl;
    }
  }
  __syncthreads();
  const SelRule rule{0xFFFFFFFFu, sh.kmin, sh.kmax};
  __syncthreads();
  return rule;
}

// The rule that keeps the `need` best (key desc, id asc) of `count` items in
// LDS (key[i], id[i], every key above KEY_NEG_INF; 1 <= need < count). Up to
// 64 items are ranked pairwise by one wave. More are binned over their own
// key range (4096 bins in `hist`), and only the threshold bin's items are
// ranked pairwise (gathered into sk / sd, 64 entries each); a threshold bin
// of more than 64 items (exact ties) falls back to radix levels over the
// whole list. NT = blockDim.x.
template <int NT>
__device__ inline SelRule list_rule(const uint32_t *key, const int32_t *id, int count, int need,
                                    uint32_t *hist, uint32_t *sk, int32_t *sd, uint32_t *scan, int *hout,
                                    SelShared<8> &sh) {
  if (count <= 64) return pairwise_rule<8>(key, id, count, need, sh);
  const int t = threadIdx.x;
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for (int i = t; i < count; i += NT) {
    lo = min(lo, key[i]);
    hi = max(hi, key[i]);
  }
  uint32_t dummy, kmin, kmax;
  for (int i = t; i < HIST_BINS; i += NT) hist[i] = 0;
  if (t == 0) sh.cnt = 0;
  block_sum_minmax(0u, lo, hi, scan, dummy, kmin, kmax);
  const uint32_t range = kmax - kmin;
  const int bits = range ? 32 - __builtin_clz(range) : 0;
  const int shift = bits > HIST_BITS ? bits - HIST_BITS : 0;
  for (int i = t; i < count; i += NT) atomicAdd(&hist[(key[i] - kmin) >> shift], 1u);
  __syncthreads();
  hist_threshold_n<HIST_BINS, NT, true>(hist, (uint32_t)need, scan, hout);
  const int thr = hout[0];
  const int need2 = need - hout[1];
  const uint32_t f2 = hist[thr];
  __syncthreads();
  if (f2 > 64) return block_rule<8, NT>(LdsKeyId{key, id}, count, need, sh);
  for (int i = t; i < count; i += NT) {
    if ((int)((key[i] - kmin) >> shift) == thr) {
      const uint32_t p = atomicAdd(&sh.cnt, 1u);
      sk[p] = key[i];
      sd[p] = id[i];
    }
  }
  __syncthreads();
  // items of higher bins have larger keys than every item of the threshold bin
  return pairwise_rule<8>(sk, sd, (int)f2, need2, sh);
}
}  // namespace csa2
