// Top-K selection for CSA2 on gfx950 (each selecting layer picks its own
// Top-K; a Full layer also keeps a candidate pool for the Reindex layers that
// follow: DeepSeek V4.1 Flash summaries, "DeepSeek V4.1 Flash深度解析" section on
// compressed attention gen. 2 and "DeepSeek V4.1 Flash 如何靠压缩 KV 缓存实现小模型
// 干翻大模型" section "CSA2").
//
// Order: score descending, entry id ascending on exact ties. Scores map to
// order-preserving 32-bit keys. A row is cut into chunks of `chunk` columns.
// For rows longer than fit in LDS, with one or two targets (the Full layer's
// pool and its top-K, both over every entry):
//  1. the scoring kernel adds each key's top 12 bits to a 4096-bin histogram
//     (LDS per workgroup, then fire-and-forget global atomics);
//  2. k_compact (one workgroup per chunk) finds every target's threshold bin
//     in that histogram, counts its keys above the bin, and writes its keys
//     in the bin, with their ids, grouped by key bits 19..12 (the "digit"),
//     plus a table of where each digit's group starts;
//  3. k_final (one workgroup per chunk again) reads every chunk's counts and
//     digit tables, finds the digit that holds the boundary, loads the few
//     keys of the row at that digit and settles the exact boundary among them
//     (radix select on the remaining key bits, then the id for exact ties),
//     and writes the selected ids of its own chunk in column order at the
//     offset given by the chunks before it.
// Plain stores only: on MI355X device-scope fences and value-returning global
// atomics cross the non-coherent per-XCD L2s and cost microseconds each.
// Output in column order is ascending id order whenever ids grow with the
// column (no candidate map, or an ascending one).
// Rows that fit in LDS use k_select_direct: one workgroup loads every key,
// selects, and writes ids through a bitmap sort. Rows of up to 16384 columns
// take k_sel_rowwise (k_select2.hip).
#include "csa2_dev.h"
#include "kernels.h"
#include "block_ops.h"

namespace csa2 {

#define FIN_NT 512
#define FIN_ITEMS 8192  // direct mode: items held in LDS
#define FB_ITEMS 1024   // compact mode: keys at the boundary digit held in LDS
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

// ---- standalone histogram ------------------------------------------------------
// Columns past a row's limit (visible entries, when n_entries is given) are
// not counted: they may hold nothing.
__global__ __launch_bounds__(256) void k_hist(const float *scores, int32_t n_cols, int32_t chunk,
                                              uint32_t *hist, const int32_t *n_entries,
                                              const int32_t *q_pos, int32_t nq) {
  __shared__ uint32_t lh[HIST_BINS];
  const int r = blockIdx.y;
  const int32_t lim = row_limit(n_entries, q_pos, nq, r, n_cols);
  const int64_t c0 = (int64_t)blockIdx.x * chunk;
  if (c0 >= lim) return;  // uniform
  const int64_t c1 = min(c0 + (int64_t)chunk, (int64_t)lim);
  for (int i = threadIdx.x; i < HIST_BINS; i += 256) lh[i] = 0;
  __syncthreads();
  const float *row = scores + (int64_t)r * n_cols;
  constexpr int U = 8;
  for (int64_t j0 = c0 + threadIdx.x; j0 < c1; j0 += 256 * U) {
    float v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = row[min(j0 + 256 * u, c1 - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t k = score_key(v[u]);
      if (j0 + 256 * u < c1 && k > KEY_NEG_INF) atomicAdd(&lh[k >> HIST_SHIFT], 1u);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < HIST_BINS; i += 256)
    if (lh[i]) atomicAdd(&hist[(int64_t)r * HIST_BINS + i], lh[i]);
}

hipError_t launch_hist(const float *scores, int32_t n_cols, int rows, uint32_t *hist,
                       hipStream_t st, const int32_t *n_entries, const int32_t *q_pos, int32_t nq) {
  const int32_t chunk = 8192;
  dim3 grid((unsigned)((n_cols + chunk - 1) / chunk), (unsigned)rows);
  hipLaunchKernelGGL(k_hist, grid, dim3(256), 0, st, scores, n_cols, chunk, hist, n_entries, q_pos, nq);
  return hipGetLastError();
}

__device__ __forceinline__ int key_digit(uint32_t k) { return (int)((k >> 12) & 0xFFu); }

// ---- compaction against the threshold bins ----------------------------------------
// NT threads, PER = chunk / NT columns per thread, NTG targets. Each lane
// owns PER consecutive columns: thread t holds c0 + t * PER + [0, PER),
// so (thread, item) is column order and a lane's place in an ordered output is
// an exclusive scan of per-lane counts. VEC: rows start 16-byte aligned
// (n_cols a multiple of 4), so the columns load as float4.
template <int PER, int NTG, bool VEC, int NT>
__global__ __launch_bounds__(NT) void k_compact(CompactArgs a) {
  __shared__ uint32_t lh[HIST_BINS];
  __shared__ uint32_t scan[8];
  __shared__ uint32_t dcnt[NTG][256];
  __shared__ int s_out[4], s_thr[NTG];
  const int r = blockIdx.y, w = blockIdx.x, tid = threadIdx.x;
  const int32_t lim = row_limit(a.n_entries, a.q_pos, a.nq, r, a.n_cols);
  const int64_t c0 = (int64_t)w * a.chunk;
  if (c0 >= lim && w != 0) return;  // uniform; workgroup 0 always publishes the thresholds
  const int64_t c1 = min(c0 + (int64_t)a.chunk, (int64_t)lim);
  const int64_t cb = c0 + (int64_t)tid * PER;
  const float *row = a.scores + (int64_t)r * a.n_cols;
  const int32_t *map = a.cand_map ? a.cand_map + (int64_t)r * a.n_cols : nullptr;
  // every load is issued unconditionally from an in-range address, so they are
  // all in flight together (a guarded load would be followed by a wait)
  float sv[PER];
  int32_t idv[PER];
  if constexpr (VEC) {
    const int64_t vmax = a.n_cols - 4;  // last aligned float4 inside the row
#pragma unroll
    for (int k = 0; k < PER / 4; ++k) {
      const v4f x = *(const v4f *)(row + min(cb + 4 * k, vmax));
      sv[4 * k] = x[0];
      sv[4 * k + 1] = x[1];
      sv[4 * k + 2] = x[2];
      sv[4 * k + 3] = x[3];
    }
    if (map) {
#pragma unroll
      for (int k = 0; k < PER / 4; ++k) {
        const v4i x = *(const v4i *)(map + min(cb + 4 * k, vmax));
        idv[4 * k] = x[0];
        idv[4 * k + 1] = x[1];
        idv[4 * k + 2] = x[2];
        idv[4 * k + 3] = x[3];
      }
    }
  } else {
    const int64_t jmax = a.n_cols - 1;
#pragma unroll
    for (int i = 0; i < PER; ++i) sv[i] = row[min(cb + i, jmax)];
    if (map) {
#pragma unroll
      for (int i = 0; i < PER; ++i) idv[i] = map[min(cb + i, jmax)];
    }
  }
  if (!map) {
#pragma unroll
    for (int i = 0; i < PER; ++i) idv[i] = (int32_t)(cb + i);
  }
  uint32_t hv[HIST_BINS / NT];
#pragma unroll
  for (int i = 0; i < HIST_BINS / NT; ++i) hv[i] = a.hist[(int64_t)r * HIST_BINS + tid + NT * i];
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint32_t k = score_key(sv[i]);
    key[i] = (cb + i < c1) ? k : 0u;
  }
#pragma unroll
  for (int i = 0; i < HIST_BINS / NT; ++i) lh[tid + NT * i] = hv[i];
  if (tid < 256) {
#pragma unroll
    for (int tg = 0; tg < NTG; ++tg) dcnt[tg][tid] = 0;
  }
  __syncthreads();
#pragma unroll
  for (int tg = 0; tg < NTG; ++tg) {
    hist_threshold_n<HIST_BINS, NT, true>(lh, (uint32_t)a.T[tg], scan, s_out);
    if (tid == 0) {
      s_thr[tg] = s_out[0];
      if (w == 0) {
        int32_t *info = a.info + ((int64_t)r * 2 + tg) * 4;
        info[0] = s_out[0];
        info[1] = s_out[1];
        info[2] = s_out[2];
      }
    }
  }
  __syncthreads();
  if (c0 >= lim) return;  // uniform: workgroup 0 of a row with nothing visible

  // classify with integer arithmetic (bit i of cbits: candidate, at or above
  // the threshold bin; of eqbits: in the bin); keys in the bin count towards
  // their digit
  uint32_t n_up[NTG], eqbits[NTG], cbits[NTG];
#pragma unroll
  for (int tg = 0; tg < NTG; ++tg) {
    const int thr = s_thr[tg];
    uint32_t eb = 0, ub = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const uint32_t valid = min(key[i] >> 23, 1u);                // key > KEY_NEG_INF
      const int bin = (int)(key[i] >> HIST_SHIFT);
      const uint32_t up = valid & ((uint32_t)(thr - bin) >> 31);   // bin > thr (any bin when thr < 0)
      const uint32_t iq = (thr >= 0 && bin == thr) ? valid : 0u;
      ub |= up << i;
      eb |= iq << i;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if ((eb >> i) & 1u) atomicAdd(&dcnt[tg][key_digit(key[i])], 1u);
    eqbits[tg] = eb;
    cbits[tg] = eb | ub;
    n_up[tg] = block_sum((uint32_t)__popc(ub), scan);
  }
#pragma unroll
  for (int tg = 0; tg < NTG; ++tg) {
    // thread t takes digit 255 - t: the exclusive scan in thread order is the
    // start of each digit's group when groups run from digit 255 down
    const int d = 255 - tid;
    const uint32_t c = (tid < 256) ? dcnt[tg][d] : 0u;
    uint32_t n_eq;
    const uint32_t start = block_exclusive_scan(c, scan, &n_eq);
    const int64_t slot = ((int64_t)r * 2 + tg) * a.max_wg + w;
    if (tid < 256) {
      a.suf[slot * 256 + d] = start + c;  // keys of this chunk in the bin with digit >= d
      dcnt[tg][d] = start;                // from here on: the group's write cursor
    }
    if (tid == 0) a.counts[slot] = n_up[tg] | (n_eq << 16);
  }
#pragma unroll
  for (int tg = 0; tg < NTG; ++tg) {
    uint64_t *list = a.list[tg] + (int64_t)r * a.seg_stride + c0;
    uint64_t *eq = a.eq[tg] + (int64_t)r * a.seg_stride + c0;
    const uint32_t cbit = cbits[tg], eb = eqbits[tg];
    // candidates in column order: this lane's first slot is the count before it
    uint32_t tot;
    uint32_t pos = block_exclusive_scan((uint32_t)__popc(cbit), scan, &tot);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const uint32_t c = (cbit >> i) & 1u;
      if (c) list[pos] = ((uint64_t)key[i] << 32) | (uint32_t)idv[i];
      pos += c;
    }
    // keys in the bin, grouped by digit: every slot first, then the stores
    uint32_t p[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      p[i] = 0;
      if ((eb >> i) & 1u) p[i] = atomicAdd(&dcnt[tg][key_digit(key[i])], 1u);
    }
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if ((eb >> i) & 1u) eq[p[i]] = ((uint64_t)key[i] << 32) | (uint32_t)idv[i];
  }
}

template <int NTG, bool VEC>
hipError_t launch_compact_n(const CompactArgs &a, dim3 grid, hipStream_t st) {
  switch (a.chunk) {
    case 2048: hipLaunchKernelGGL((k_compact<8, NTG, VEC, 256>), grid, dim3(256), 0, st, a); break;
    case 4096: hipLaunchKernelGGL((k_compact<16, NTG, VEC, 256>), grid, dim3(256), 0, st, a); break;
    case 8192: hipLaunchKernelGGL((k_compact<16, NTG, VEC, 512>), grid, dim3(512), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_compact(const CompactArgs &a, int rows, hipStream_t st) {
  dim3 grid((unsigned)((a.n_cols + a.chunk - 1) / a.chunk), (unsigned)rows);
  if ((int)grid.x > a.max_wg || a.max_wg > SEL_MAX_WG) return hipErrorInvalidValue;
  const bool vec = a.n_cols % 4 == 0 && ((uintptr_t)a.scores & 15) == 0 &&
                   (!a.cand_map || ((uintptr_t)a.cand_map & 15) == 0);
  if (a.ntarget == 1) return vec ? launch_compact_n<1, true>(a, grid, st) : launch_compact_n<1, false>(a, grid, st);
  if (a.ntarget == 2) return vec ? launch_compact_n<2, true>(a, grid, st) : launch_compact_n<2, false>(a, grid, st);
  return hipErrorInvalidValue;
}

// ---- final pass: one workgroup per chunk ------------------------------------------
// Workgroup of the flat index i in a prefix array (pre[w] <= i < pre[w+1]).
__device__ __forceinline__ int seg_of(const uint32_t *pre, int nwg, uint32_t i) {
  int lo = 0, hi = nwg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Keys at the boundary digit read from the chunks' groups in global memory
// (when there are too many for LDS).
struct FbGlobal {
  const uint64_t *eq;
  int32_t chunk;
  const uint32_t *pre, *start;
  int nwg;
  __device__ void get(int i, uint32_t &k, int32_t &d) const {
    const int w = seg_of(pre, nwg, (uint32_t)i);
    const uint64_t v = eq[(int64_t)w * chunk + start[w] + ((uint32_t)i - pre[w])];
    k = (uint32_t)(v >> 32);
    d = (int32_t)(uint32_t)v;
  }
};

// The chunk's candidates (keys at or above the threshold bin, in column
// order, from k_compact) are read two per thread per round; the first round's
// loads are issued with the others before anything else is known.
__global__ __launch_bounds__(FIN_NT) void k_final(FinalArgs a) {
  __shared__ uint16_t s_suf[SEL_MAX_WG * 256];
  __shared__ uint32_t s_cnt[SEL_MAX_WG];
  __shared__ uint32_t s_fpre[SEL_MAX_WG + 1], s_fstart[SEL_MAX_WG];
  __shared__ uint64_t s_fb[FB_ITEMS];
  __shared__ uint32_t s_tot[2][256], s_pre[2][256];
  __shared__ uint32_t s_wave[2][FIN_NT / 64];
  __shared__ SelShared<8> sh;
  const int w0 = blockIdx.x, r = blockIdx.y, tg = blockIdx.z, t = threadIdx.x;
  const int lane = t & 63, wv = t >> 6;
  const int T = a.T[tg];
  int32_t *out = a.out[tg] + (int64_t)r * a.out_stride[tg];
  const int32_t lim = row_limit(a.n_entries, a.q_pos, a.nq, r, a.n_cols);
  const int nwg = (int)((lim + a.chunk - 1) / a.chunk);
  const int32_t *info = a.info + ((int64_t)r * 2 + tg) * 4;
  const int thr = info[0], above = info[1], total = info[2];
  const int selT = min(T, total);
  for (int i = selT + w0 * FIN_NT + t; i < T; i += (int)gridDim.x * FIN_NT) out[i] = -1;
  if (w0 >= nwg) return;  // uniform: a chunk past the visible entries

  // ---- loads that do not depend on each other: candidates, counts, digit tables
  const uint64_t *list = a.list[tg] + (int64_t)r * a.seg_stride + (int64_t)w0 * a.chunk;
  uint64_t cv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) cv[u] = list[min(t + FIN_NT * u, a.chunk - 1)];
  const int64_t slot0 = ((int64_t)r * 2 + tg) * a.max_wg;
  {
    const uint32_t cw = a.counts[slot0 + min(t, nwg - 1)];
    if (t < nwg) s_cnt[t] = cw;
  }
  // digit tables of all chunks into LDS; thread t meets only digit t & 255
  // (of chunks 2u + t / 256), so it sums that digit's column on the way
  uint32_t sa = 0, sp = 0;
  if (thr >= 0) {  // uniform
    const uint32_t *suf = a.suf + slot0 * 256;
    const int n = nwg * 256;
    constexpr int U = 16;
    for (int i0 = 0; i0 < n; i0 += FIN_NT * U) {
      uint32_t v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = suf[min(i0 + t + FIN_NT * u, n - 1)];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int idx = i0 + t + FIN_NT * u;
        if (idx < n) {
          s_suf[idx] = (uint16_t)v[u];
          sa += v[u];
          sp += ((idx >> 8) < w0) ? v[u] : 0u;
        }
      }
    }
  }
  __syncthreads();
  const uint32_t up_before = block_sum((t < w0) ? (s_cnt[t] & 0xFFFFu) : 0u, sh.scan);
  const uint32_t n_list = (s_cnt[w0] & 0xFFFFu) + (s_cnt[w0] >> 16);

  // ---- boundary inside the threshold bin
  int fthr = 256;        // digits above fthr are taken whole
  bool fine_all = true;  // every key at digit fthr is taken
  SelRule rule{0u, 0u, 0xFFFFFFFFu};
  uint32_t gt_before = 0, fine_before = 0;
  if (thr >= 0) {
    const int need = selT - above;  // keys to take from the threshold bin (>= 1)
    s_tot[t >> 8][t & 255] = sa;
    s_pre[t >> 8][t & 255] = sp;
    __syncthreads();
    if (t < 256) {
      s_tot[0][t] += s_tot[1][t];
      s_pre[0][t] += s_pre[1][t];
    }
    __syncthreads();
    // keys with digit >= d, summed over the row, fall as d grows: the boundary
    // digit is the largest d at which they still reach `need`
    fthr = max((int)block_sum((t < 256 && s_tot[0][t] >= (uint32_t)need) ? 1u : 0u, sh.scan) - 1, 0);
    const uint32_t above2 = (fthr < 255) ? s_tot[0][fthr + 1] : 0u;
    const uint32_t need2 = (uint32_t)need - above2;
    const uint32_t F = s_tot[0][fthr] - above2;
    gt_before = (fthr < 255) ? s_pre[0][fthr + 1] : 0u;
    uint32_t fc = 0;
    if (t < nwg) {
      const uint32_t st = (fthr < 255) ? s_suf[t * 256 + fthr + 1] : 0u;
      s_fstart[t] = st;
      fc = s_suf[t * 256 + fthr] - st;
    }
    uint32_t ftot;
    const uint32_t fo = block_exclusive_scan(fc, sh.scan, &ftot);
    if (t < nwg) s_fpre[t] = fo;
    if (t == 0) s_fpre[nwg] = ftot;
    __syncthreads();
    const uint32_t fine_lim = s_fpre[w0];  // flat index of this chunk's first key at the digit
    if (need2 >= F) {
      fine_before = fine_lim;
    } else {
      fine_all = false;
      const uint64_t *eq = a.eq[tg] + (int64_t)r * a.seg_stride;
      if (F <= FB_ITEMS) {
        for (uint32_t i0 = 0; i0 < F; i0 += FIN_NT * 2) {
          uint64_t v[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const uint32_t i = min(i0 + t + FIN_NT * u, F - 1);
            const int w = seg_of(s_fpre, nwg, i);
            v[u] = eq[(int64_t)w * a.chunk + s_fstart[w] + (i - s_fpre[w])];
          }
#pragma unroll
          for (int u = 0; u < 2; ++u)
            if (i0 + t + FIN_NT * u < F) s_fb[i0 + t + FIN_NT * u] = v[u];
        }
        if (t == 0) {  // replaced by the last key taken (ids are distinct)
          sh.kmin = 0xFFFFFFFFu;
          sh.kmax = 0u;
        }
        __syncthreads();
        // rank of each key among the F at the digit (keys ahead of it: larger
        // key, or equal key and lower id); the one ranked need2 - 1 is the last
        // taken, and a key is taken iff it is not behind that one
        uint32_t c = 0;
        for (uint32_t i = t; i < F; i += FIN_NT) {
          const uint64_t vi = s_fb[i];
          const uint32_t ki = (uint32_t)(vi >> 32), di = (uint32_t)vi;
          uint32_t rank = 0;
          for (uint32_t j = 0; j < F; ++j) {
            const uint64_t vj = s_fb[j];
            const uint32_t kj = (uint32_t)(vj >> 32), dj = (uint32_t)vj;
            rank += (kj > ki || (kj == ki && dj < di)) ? 1u : 0u;
          }
          if (rank == need2 - 1) {
            sh.kmin = ki;
            sh.kmax = di;
          }
          c += (i < fine_lim && rank < need2) ? 1u : 0u;
        }
        fine_before = block_sum(c, sh.scan);
        rule = SelRule{0xFFFFFFFFu, sh.kmin, sh.kmax};
      } else {
        const FbGlobal acc{eq, a.chunk, s_fpre, s_fstart, nwg};
        rule = block_rule<8, FIN_NT>(acc, (int)F, (int)need2, sh);
        uint32_t c = 0;
        for (uint32_t i = t; i < fine_lim; i += FIN_NT) {
          uint32_t k;
          int32_t d;
          acc.get((int)i, k, d);
          c += rule_pass(rule, k, d) ? 1u : 0u;
        }
        fine_before = block_sum(c, sh.scan);
      }
    }
  }

  // ---- emit this chunk's selected candidates in column order
  uint32_t pos = up_before + gt_before + fine_before;
  for (uint32_t j0 = 0; j0 < n_list; j0 += 2 * FIN_NT) {
    if (j0 > 0) {  // uniform: more than 2 * FIN_NT candidates
#pragma unroll
      for (int u = 0; u < 2; ++u) cv[u] = list[min(j0 + t + FIN_NT * u, n_list - 1)];
    }
    bool pass[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t k = (uint32_t)(cv[u] >> 32);
      const int32_t d = (int32_t)(uint32_t)cv[u];
      bool ok = j0 + t + FIN_NT * u < n_list;
      if (thr >= 0) {
        const int bin = (int)(k >> HIST_SHIFT);
        const int dg = key_digit(k);
        ok = ok && (bin > thr || dg > fthr || (dg == fthr && (fine_all || rule_pass(rule, k, d))));
      }
      pass[u] = ok;
      const uint64_t m = __ballot(ok);
      if (lane == 0) s_wave[u][wv] = (uint32_t)__popcll(m);
    }
    __syncthreads();
    uint32_t tot0 = 0, before0 = 0, before1 = 0, tot1 = 0;
    for (int v = 0; v < FIN_NT / 64; ++v) {
      tot0 += s_wave[0][v];
      tot1 += s_wave[1][v];
      before0 += (v < wv) ? s_wave[0][v] : 0u;
      before1 += (v < wv) ? s_wave[1][v] : 0u;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint64_t m = __ballot(pass[u]);
      if (pass[u]) {
        const uint32_t p = pos + (u ? tot0 + before1 : before0) +
                           __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        if (p < (uint32_t)T) out[p] = (int32_t)(uint32_t)cv[u];
      }
    }
    pos += tot0 + tot1;
    __syncthreads();  // s_wave is rewritten next round
  }
}

hipError_t launch_final(const FinalArgs &a, int rows, int ntarget, hipStream_t st) {
  dim3 grid((unsigned)a.max_wg, (unsigned)rows, (unsigned)ntarget);
  if (a.max_wg > SEL_MAX_WG || a.chunk > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_final, grid, dim3(FIN_NT), 0, st, a);
  return hipGetLastError();
}

// ---- ascending output through a bitmap ----------------------------------------------
// Writes the n distinct non-negative ids held in LDS (n <= FIN_ITEMS) to
// `out` in ascending order, then -1 to positions n..pad_to-1. Ids spanning at
// most 16 bitmap windows are placed through a bitmap and a prefix sum; wider
// ranges fall back to a bitonic sort in LDS. bm: BM_WORDS words, sorted: at
// least the next power of two >= n entries (both LDS, distinct from ids).
__device__ void block_sort_out(const int32_t *ids, int n, int pad_to, int32_t *out, uint32_t *bm,
                               int32_t *sorted, uint32_t *scan_buf, int *vars) {
  const int t = threadIdx.x, nt = blockDim.x;
  if (t == 0) {
    vars[0] = 0;
    vars[1] = 0x7FFFFFFF;
    vars[2] = 0;
  }
  __syncthreads();
  {
    int lo = 0x7FFFFFFF, hi = 0;
    for (int i = t; i < n; i += nt) {
      lo = min(lo, ids[i]);
      hi = max(hi, ids[i]);
    }
    if (n > 0) {
      atomicMin(&vars[1], lo);
      atomicMax(&vars[2], hi);
    }
  }
  __syncthreads();
  const int64_t lo0 = (int64_t)(vars[1] & ~31), hi = (int64_t)vars[2];
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
      uint32_t pos = (uint32_t)vars[0] + off;
      for (int i = 0; i < per; ++i) {
        uint32_t word = bm[t * per + i];
        while (word) {
          const int bit = __ffs(word) - 1;
          word &= word - 1;
          if (pos < (uint32_t)n) sorted[pos] = (int32_t)(lo + (int64_t)(t * per + i) * 32 + bit);
          ++pos;
        }
      }
      __syncthreads();
      if (t == 0) vars[0] += (int)total;
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
            const int32_t x = sorted[i], y = sorted[p];
            const bool up = (i & kk) == 0;
            if ((x > y) == up) {
              sorted[i] = y;
              sorted[p] = x;
            }
          }
        }
        __syncthreads();
      }
    }
  }
  __syncthreads();
  for (int i = t; i < pad_to; i += nt) out[i] = (i < n) ? sorted[i] : -1;
  __syncthreads();
}

// ---- rows that fit in LDS: one workgroup per row and target -------------------------
struct LdsItems {
  const uint32_t *key;
  const int32_t *id;
  __device__ void get(int i, uint32_t &k, int32_t &d) const {
    k = key[i];
    d = id[i];
  }
};

#define DIR_U 8

__global__ __launch_bounds__(FIN_NT) void k_select_direct(DirectArgs a) {
  __shared__ uint32_t skey[FIN_ITEMS];
  __shared__ int32_t sid[FIN_ITEMS];
  __shared__ int32_t ssel[FIN_ITEMS];
  __shared__ SelShared<12> sh;
  __shared__ uint32_t s_n[2];
  const int r = blockIdx.x, tg = blockIdx.y, t = threadIdx.x;
  const float *row = a.scores + (int64_t)r * a.n_cols;
  const int32_t *map = a.cand_map ? a.cand_map + (int64_t)r * a.n_cols : nullptr;
  int32_t *gout = a.out[tg] + (int64_t)r * a.out_stride[tg];
  const int T = a.T[tg];
  const int32_t lim = min(row_limit(a.n_entries, a.q_pos, a.nq, r, a.n_cols), FIN_ITEMS);
  if (t == 0) {
    s_n[0] = 0;
    s_n[1] = 0;
  }
  __syncthreads();
  for (int base = 0; base < lim; base += FIN_NT * DIR_U) {
    float v[DIR_U];
    int32_t d[DIR_U];
#pragma unroll
    for (int u = 0; u < DIR_U; ++u) v[u] = row[min(base + t + FIN_NT * u, lim - 1)];
    if (map) {
#pragma unroll
      for (int u = 0; u < DIR_U; ++u) d[u] = map[min(base + t + FIN_NT * u, lim - 1)];
    } else {
#pragma unroll
      for (int u = 0; u < DIR_U; ++u) d[u] = base + t + FIN_NT * u;
    }
#pragma unroll
    for (int u = 0; u < DIR_U; ++u) {
      const uint32_t k = score_key(v[u]);
      const bool ok = base + t + FIN_NT * u < lim && k > KEY_NEG_INF;
      const int p = wave_append(ok, &s_n[0]);
      if (ok) {
        skey[p] = k;
        sid[p] = d[u];
      }
    }
  }
  __syncthreads();
  const int n_valid = (int)s_n[0];
  const int selT = min(T, n_valid);
  if (selT >= n_valid) {
    for (int i = t; i < n_valid; i += FIN_NT) ssel[i] = sid[i];
  } else {
    const LdsItems acc{skey, sid};
    const SelRule rule = block_rule<12, FIN_NT>(acc, n_valid, selT, sh);
    for (int i0 = 0; i0 < n_valid; i0 += FIN_NT) {
      const int i = i0 + t;
      uint32_t k = 0;
      int32_t d = 0;
      if (i < n_valid) acc.get(i, k, d);
      const bool ok = i < n_valid && rule_pass(rule, k, d);
      const int p = wave_append(ok, &s_n[1]);
      if (ok) ssel[p] = d;
    }
  }
  __syncthreads();
  block_sort_out(ssel, selT, T, gout, skey, sid, sh.scan, sh.out);
}

hipError_t launch_select_direct(const DirectArgs &a, int rows, int ntarget, hipStream_t st) {
  hipLaunchKernelGGL(k_select_direct, dim3((unsigned)rows, (unsigned)ntarget), dim3(FIN_NT), 0, st, a);
  return hipGetLastError();
}

// ---- ascending order for ids that did not come in column order ----------------------
// Row r of `ids` holds its selected ids first, then -1 up to T.
__global__ __launch_bounds__(FIN_NT) void k_sort_rows(int32_t *ids, int32_t stride, int32_t T) {
  __shared__ int32_t sin_[CSA2_MAX_K];
  __shared__ int32_t ssorted[CSA2_MAX_K];
  __shared__ uint32_t bm[BM_WORDS];
  __shared__ uint32_t scan[16];
  __shared__ int vars[4];
  const int t = threadIdx.x;
  int32_t *row = ids + (int64_t)blockIdx.x * stride;
  uint32_t c = 0;
  for (int i = t; i < T; i += FIN_NT) {
    const int32_t v = row[i];
    sin_[i] = v;
    c += v >= 0 ? 1u : 0u;
  }
  const uint32_t n = block_sum(c, scan);
  block_sort_out(sin_, (int)n, T, row, bm, ssorted, scan, vars);
}

hipError_t launch_sort_rows(int32_t *ids, int32_t stride, int32_t T, int rows, hipStream_t st) {
  if (T > CSA2_MAX_K) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_sort_rows, dim3((unsigned)rows), dim3(FIN_NT), 0, st, ids, stride, T);
  return hipGetLastError();
}

}  // namespace csa2
