// Top-K selection for CSA2 on gfx950 (each selecting layer picks its own
// Top-K; a Full layer also keeps a candidate pool for the Reindex layers that
// follow: DeepSeek V4.1 Flash summaries, "DeepSeek V4.1 Flash深度解析" section on
// compressed attention gen. 2 and "DeepSeek V4.1 Flash 如何靠压缩 KV 缓存实现小模型
// 干翻大模型" section "CSA2").
//
// Order: score descending, entry id ascending on exact ties. Scores map to
// order-preserving 32-bit keys. Pipeline for a row of n scores and target T:
//  1. a 4096-bin histogram of the top 12 key bits (fused into the scoring
//     kernel, or k_hist for standalone scores);
//  2. k_compact (many workgroups per row): every workgroup finds the bin
//     that holds the T-th key, appends the ids of keys in higher bins to the
//     output and the columns of keys in that bin to a candidate list;
//  3. k_final (one workgroup per row): radix select, 8 bits per pass in LDS,
//     of the missing count among the candidates, then exact ties by id;
//     optionally the top K2 of the selected set (the Full layer's top-K out
//     of its pool); ids of a top-K are emitted in ascending order through a
//     bitmap, pads are -1.
// Rows short enough to sit in LDS skip steps 1-2 (direct mode).
#include "csa2_dev.h"
#include "kernels.h"

namespace csa2 {

#define FIN_NT 512
#define FIN_ITEMS 16384
#define BM_WORDS 4096
#define BM_BITS (BM_WORDS * 32)

__global__ void k_fill_u32(uint32_t *p, int64_t n, uint32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_u32(uint32_t *p, int64_t n, uint32_t v, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

// ---- block helpers (every thread of the block must call them) ----------------

// s[0..255] <- suffix sums of in[0..255]; s[256] = 0.  Uses threads < 256.
__device__ void suffix_scan256(const uint32_t *in, uint32_t *s) {
  const int t = threadIdx.x;
  if (t < 256) s[t] = in[t];
  if (t == 0) s[256] = 0;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    uint32_t add = 0;
    if (t < 256 && t + off < 256) add = s[t + off];
    __syncthreads();
    if (t < 256) s[t] += add;
    __syncthreads();
  }
}

// Exclusive prefix sum of one value per thread (blockDim.x <= 1024); returns
// this thread's offset, *total gets the block total.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t *s, uint32_t *total) {
  const int t = threadIdx.x, n = blockDim.x;
  s[t] = v;
  __syncthreads();
  for (int off = 1; off < n; off <<= 1) {
    uint32_t add = (t >= off) ? s[t - off] : 0;
    __syncthreads();
    s[t] += add;
    __syncthreads();
  }
  const uint32_t incl = s[t];
  *total = s[n - 1];
  __syncthreads();
  return incl - v;
}

// Threshold bin of the T-th largest key from a HIST_BINS histogram held in
// LDS (256 threads or more). Returns bin (-1 when at most T valid keys) and
// the number of keys in higher bins.
__device__ void find_threshold_bin(const uint32_t *h, int T, uint32_t *s_tmp, uint32_t *s_suf,
                                   int *s_out) {
  const int t = threadIdx.x;
  constexpr int PER = HIST_BINS / 256;
  if (t < 256) {
    uint32_t sum = 0;
    for (int i = 0; i < PER; ++i) sum += h[t * PER + i];
    s_tmp[t] = sum;
  }
  __syncthreads();
  suffix_scan256(s_tmp, s_suf);
  if (t == 0) {
    s_out[0] = -1;
    s_out[1] = (int)s_suf[0];  // total valid
  }
  __syncthreads();
  if (t < 256 && s_suf[0] > (uint32_t)T && s_suf[t] >= (uint32_t)T && s_suf[t + 1] < (uint32_t)T) {
    uint32_t cum = s_suf[t + 1];
    for (int i = PER - 1; i >= 0; --i) {
      const uint32_t c = h[t * PER + i];
      if (cum + c >= (uint32_t)T) {
        s_out[0] = t * PER + i;
        s_out[2] = (int)cum;
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
}

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

// ---- standalone histogram ------------------------------------------------------
__global__ __launch_bounds__(256) void k_hist(const float *scores, int32_t n_cols, int32_t chunk,
                                              uint32_t *hist) {
  __shared__ uint32_t lh[HIST_BINS];
  const int r = blockIdx.y;
  const int64_t c0 = (int64_t)blockIdx.x * chunk;
  const int64_t c1 = min(c0 + (int64_t)chunk, (int64_t)n_cols);
  for (int i = threadIdx.x; i < HIST_BINS; i += 256) lh[i] = 0;
  __syncthreads();
  const float *row = scores + (int64_t)r * n_cols;
  for (int64_t j = c0 + threadIdx.x; j < c1; j += 256) {
    const uint32_t k = score_key(row[j]);
    if (k > KEY_NEG_INF) atomicAdd(&lh[k >> HIST_SHIFT], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < HIST_BINS; i += 256)
    if (lh[i]) atomicAdd(&hist[(int64_t)r * HIST_BINS + i], lh[i]);
}

hipError_t launch_hist(const float *scores, int32_t n_cols, int rows, uint32_t *hist,
                       hipStream_t st) {
  const int32_t chunk = 8192;
  dim3 grid((unsigned)((n_cols + chunk - 1) / chunk), (unsigned)rows);
  hipLaunchKernelGGL(k_hist, grid, dim3(256), 0, st, scores, n_cols, chunk, hist);
  return hipGetLastError();
}

// ---- compaction against the threshold bin ----------------------------------------
__global__ __launch_bounds__(256) void k_compact(CompactArgs a) {
  __shared__ uint32_t lh[HIST_BINS];
  __shared__ uint32_t s_tmp[256], s_suf[257];
  __shared__ int s_out[4];
  const int r = blockIdx.y;
  const int32_t lim = row_limit(a.n_entries, a.q_pos, a.nq, r, a.n_cols);
  const int64_t c0 = (int64_t)blockIdx.x * a.chunk;
  if (c0 >= lim) return;
  const int64_t c1 = min(c0 + (int64_t)a.chunk, (int64_t)lim);
  for (int i = threadIdx.x; i < HIST_BINS; i += 256) lh[i] = a.hist[(int64_t)r * HIST_BINS + i];
  __syncthreads();
  find_threshold_bin(lh, a.T, s_tmp, s_suf, s_out);
  const int thr = s_out[0];
  const float *row = a.scores + (int64_t)r * a.n_cols;
  const int32_t *map = a.cand_map ? a.cand_map + (int64_t)r * a.n_cols : nullptr;
  int32_t *out = a.out + (int64_t)r * a.out_stride;
  int32_t *cand = a.cand_cols + (int64_t)r * a.n_cols;
  uint32_t *ctr = a.ctr + (int64_t)r * 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int64_t base = c0 + wave * 64; base < c1; base += 256) {
    const int64_t j = base + lane;
    bool up = false, eq = false;
    if (j < c1) {
      const uint32_t k = score_key(row[j]);
      if (k > KEY_NEG_INF) {
        const int bin = (int)(k >> HIST_SHIFT);
        up = (thr < 0) || (bin > thr);
        eq = (thr >= 0) && (bin == thr);
      }
    }
    const int p = wave_append(up, &ctr[0]);
    if (up && p < a.out_stride) out[p] = map ? map[j] : (int32_t)j;
    const int q = wave_append(eq, &ctr[1]);
    if (eq && q < a.n_cols) cand[q] = (int32_t)j;
  }
}

hipError_t launch_compact(const CompactArgs &a, int rows, hipStream_t st) {
  dim3 grid((unsigned)((a.n_cols + a.chunk - 1) / a.chunk), (unsigned)rows);
  hipLaunchKernelGGL(k_compact, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// ---- item accessors for the block radix select ------------------------------------
struct LdsItems {
  const uint32_t *key;
  const int32_t *id;
  __device__ void get(int i, uint32_t &k, int32_t &d) const { k = key[i]; d = id[i]; }
};
struct CandItems {  // candidate columns of a score row
  const float *row;
  const int32_t *cols;
  const int32_t *map;
  __device__ void get(int i, uint32_t &k, int32_t &d) const {
    const int32_t c = cols[i];
    k = score_key(row[c]);
    d = map ? map[c] : c;
  }
};
struct IdItems {  // a list of entry ids whose score sits at column = id
  const float *row;
  const int32_t *ids;
  __device__ void get(int i, uint32_t &k, int32_t &d) const {
    d = ids[i];
    k = score_key(row[d]);
  }
};

struct SelShared {
  uint32_t hist[256];
  uint32_t suf[257];
  int vars[8];
};

// Appends to dst the `need` best items (key desc, id asc) out of `count`.
// known_bits: number of leading key bits shared by every item (kpref0).
template <class Acc>
__device__ void block_select(const Acc &acc, int count, int need, uint32_t kpref0,
                             int known_bits, int32_t *dst, SelShared &sh) {
  const int t = threadIdx.x, nt = blockDim.x;
  if (t == 0) sh.vars[0] = 0;
  __syncthreads();
  if (need <= 0) return;
  if (need >= count) {
    for (int i = t; i < count; i += nt) {
      uint32_t k;
      int32_t d;
      acc.get(i, k, d);
      dst[atomicAdd((uint32_t *)&sh.vars[0], 1u)] = d;
    }
    __syncthreads();
    return;
  }
  uint32_t kpref = kpref0;
  uint32_t kmask = known_bits ? (0xFFFFFFFFu << (32 - known_bits)) : 0u;
  int bits_left = 32 - known_bits;
  int left = need;
  int eqcnt = count;
  while (bits_left > 0) {
    const int width = bits_left < 8 ? bits_left : 8;
    const int shift = bits_left - width;
    const uint32_t dmask = (1u << width) - 1u;
    if (t < 256) sh.hist[t] = 0;
    __syncthreads();
    for (int i = t; i < count; i += nt) {
      uint32_t k;
      int32_t d;
      acc.get(i, k, d);
      if ((k & kmask) == kpref) atomicAdd(&sh.hist[(k >> shift) & dmask], 1u);
    }
    __syncthreads();
    suffix_scan256(sh.hist, sh.suf);
    if (t < 256 && sh.suf[t] >= (uint32_t)left && sh.suf[t + 1] < (uint32_t)left) sh.vars[1] = t;
    __syncthreads();
    const int dsel = sh.vars[1];
    left -= (int)sh.suf[dsel + 1];
    eqcnt = (int)sh.hist[dsel];
    kpref |= (uint32_t)dsel << shift;
    kmask |= dmask << shift;
    bits_left -= width;
    __syncthreads();
  }
  uint32_t idthr = 0xFFFFFFFFu;
  if (left < eqcnt) {  // exact key ties at the boundary: keep the lowest ids
    uint32_t ipref = 0, imask = 0;
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (t < 256) sh.hist[t] = 0;
      __syncthreads();
      for (int i = t; i < count; i += nt) {
        uint32_t k;
        int32_t d;
        acc.get(i, k, d);
        if (k == kpref && ((uint32_t)d & imask) == ipref)
          atomicAdd(&sh.hist[((uint32_t)d >> shift) & 255u], 1u);
      }
      __syncthreads();
      suffix_scan256(sh.hist, sh.suf);
      // inclusive prefix(d) = suf[0] - suf[d + 1]
      if (t < 256) {
        const uint32_t pre = sh.suf[0] - sh.suf[t + 1];
        const uint32_t pre_prev = sh.suf[0] - sh.suf[t];
        if (pre >= (uint32_t)left && pre_prev < (uint32_t)left) sh.vars[1] = t;
      }
      __syncthreads();
      const int dsel = sh.vars[1];
      left -= (int)(sh.suf[0] - sh.suf[dsel]);
      ipref |= (uint32_t)dsel << shift;
      imask |= 255u << shift;
      __syncthreads();
    }
    idthr = ipref;
  }
  for (int i = t; i < count; i += nt) {
    uint32_t k;
    int32_t d;
    acc.get(i, k, d);
    if (k > kpref || (k == kpref && (uint32_t)d <= idthr))
      dst[atomicAdd((uint32_t *)&sh.vars[0], 1u)] = d;
  }
  __syncthreads();
}

// Sorts n distinct non-negative ids (n <= CSA2_MAX_K) held in global memory
// ascending, in place, then writes -1 to positions n..pad_to-1. Ids spanning
// at most 16 bitmap windows are placed through a bitmap and a prefix sum;
// wider ranges fall back to a bitonic sort in LDS.
__device__ void block_sort_ids(int32_t *ids, int n, int pad_to, uint32_t *bm, int32_t *sorted,
                               uint32_t *scan_buf, int *vars) {
  const int t = threadIdx.x, nt = blockDim.x;
  if (t == 0) {
    vars[2] = 0;
    vars[4] = 0x7FFFFFFF;
    vars[5] = 0;
  }
  __syncthreads();
  for (int i = t; i < n; i += nt) {
    atomicMin(&vars[4], ids[i]);
    atomicMax(&vars[5], ids[i]);
  }
  __syncthreads();
  const int64_t lo0 = (int64_t)(vars[4] & ~31), hi = (int64_t)vars[5];
  if (n > 0 && hi - lo0 < 16LL * BM_BITS) {
    for (int64_t lo = lo0; lo <= hi; lo += BM_BITS) {
      for (int i = t; i < BM_WORDS; i += nt) bm[i] = 0;
      __syncthreads();
      for (int i = t; i < n; i += nt) {
        const int64_t d = (int64_t)ids[i] - lo;
        if (d >= 0 && d < BM_BITS) atomicOr(&bm[d >> 5], 1u << (d & 31));
      }
      __syncthreads();
      const int per = BM_WORDS / nt;
      uint32_t cnt = 0;
      for (int i = 0; i < per; ++i) cnt += __popc(bm[t * per + i]);
      uint32_t total;
      const uint32_t off = block_exclusive_scan(cnt, scan_buf, &total);
      uint32_t pos = (uint32_t)vars[2] + off;
      for (int i = 0; i < per; ++i) {
        uint32_t word = bm[t * per + i];
        while (word) {
          const int bit = __ffs(word) - 1;
          word &= word - 1;
          sorted[pos++] = (int32_t)(lo + (int64_t)(t * per + i) * 32 + bit);
        }
      }
      __syncthreads();
      if (t == 0) vars[2] += (int)total;
      __syncthreads();
    }
  } else if (n > 0) {
    int np = 1;
    while (np < n) np <<= 1;
    for (int i = t; i < np; i += nt) sorted[i] = (i < n) ? ids[i] : 0x7FFFFFFF;
    __syncthreads();
    for (int kk = 2; kk <= np; kk <<= 1) {
      for (int j = kk >> 1; j > 0; j >>= 1) {
        for (int i = t; i < np; i += nt) {
          const int p = i ^ j;
          if (p > i) {
            const int32_t a = sorted[i], b = sorted[p];
            const bool up = (i & kk) == 0;
            if ((a > b) == up) {
              sorted[i] = b;
              sorted[p] = a;
            }
          }
        }
        __syncthreads();
      }
    }
  }
  __syncthreads();
  for (int i = t; i < n; i += nt) ids[i] = sorted[i];
  for (int i = n + t; i < pad_to; i += nt) ids[i] = -1;
  __syncthreads();
}

__global__ __launch_bounds__(FIN_NT) void k_final(FinalArgs a) {
  __shared__ uint32_t skey[FIN_ITEMS];
  __shared__ int32_t sid[FIN_ITEMS];
  __shared__ SelShared sh;
  __shared__ uint32_t scan_buf[FIN_NT];
  __shared__ int s_misc[4];
  const int r = blockIdx.x, t = threadIdx.x;
  const float *row = a.scores + (int64_t)r * a.n_cols;
  const int32_t *map = a.cand_map ? a.cand_map + (int64_t)r * a.n_cols : nullptr;
  int32_t *outT = a.outT + (int64_t)r * a.outT_stride;

  int selT;  // final size of the T-set
  if (a.hist) {
    // compact mode: ids in higher bins are already in outT[0..n_above)
    uint32_t part = 0;
    for (int i = t; i < HIST_BINS; i += FIN_NT) part += a.hist[(int64_t)r * HIST_BINS + i];
    uint32_t total;
    block_exclusive_scan(part, scan_buf, &total);
    const int n_above = (int)a.ctr[(int64_t)r * 4 + 0];
    const int n_cand = (int)a.ctr[(int64_t)r * 4 + 1];
    selT = (int)min((uint32_t)a.T, total);
    const int need = selT - n_above;
    const int32_t *cols = a.cand_cols + (int64_t)r * a.n_cols;
    if (need > 0) {
      if (n_cand <= FIN_ITEMS) {
        for (int i = t; i < n_cand; i += FIN_NT) {
          const int32_t c = cols[i];
          skey[i] = score_key(row[c]);
          sid[i] = map ? map[c] : c;
        }
        __syncthreads();
        block_select(LdsItems{skey, sid}, n_cand, need, 0u, 0, outT + n_above, sh);
      } else {
        block_select(CandItems{row, cols, map}, n_cand, need, 0u, 0, outT + n_above, sh);
      }
    }
  } else {
    // direct mode: every valid column of the row is an item (row fits in LDS)
    const int32_t lim = row_limit(a.n_entries, a.q_pos, a.nq, r, a.n_cols);
    if (t == 0) s_misc[0] = 0;
    __syncthreads();
    for (int base = (t >> 6) * 64; base < lim; base += FIN_NT) {
      const int j = base + (t & 63);
      bool ok = false;
      uint32_t k = 0;
      if (j < lim) {
        k = score_key(row[j]);
        ok = k > KEY_NEG_INF;
      }
      const uint64_t m = __ballot(ok);
      int basepos = 0;
      const int leader = m ? (__ffsll((unsigned long long)m) - 1) : 0;
      if (m && (t & 63) == leader) basepos = atomicAdd(&s_misc[0], __popcll(m));
      basepos = __shfl(basepos, leader);
      if (ok) {
        const uint32_t lo = (uint32_t)m, hi = (uint32_t)(m >> 32);
        const int p = basepos + __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0));
        skey[p] = k;
        sid[p] = map ? map[j] : j;
      }
    }
    __syncthreads();
    const int n_valid = s_misc[0];
    selT = min(a.T, n_valid);
    block_select(LdsItems{skey, sid}, n_valid, selT, 0u, 0, outT, sh);
  }
  __syncthreads();

  if (a.K2 > 0) {
    int32_t *outK = a.outK2 + (int64_t)r * a.K2_stride;
    const int selK = min(a.K2, selT);
    if (selT <= FIN_ITEMS) {
      for (int i = t; i < selT; i += FIN_NT) {
        const int32_t d = outT[i];
        sid[i] = d;
        skey[i] = score_key(row[d]);
      }
      __syncthreads();
      block_select(LdsItems{skey, sid}, selT, selK, 0u, 0, outK, sh);
    } else {
      block_select(IdItems{row, outT}, selT, selK, 0u, 0, outK, sh);
    }
    __syncthreads();
    block_sort_ids(outK, selK, a.K2, skey, sid, scan_buf, sh.vars);
    for (int i = selT + t; i < a.T; i += FIN_NT) outT[i] = -1;
  } else if (a.sortT) {
    block_sort_ids(outT, selT, a.T, skey, sid, scan_buf, sh.vars);
  } else {
    for (int i = selT + t; i < a.T; i += FIN_NT) outT[i] = -1;
  }
}

hipError_t launch_final(const FinalArgs &a, int rows, hipStream_t st) {
  hipLaunchKernelGGL(k_final, dim3((unsigned)rows), dim3(FIN_NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa2
