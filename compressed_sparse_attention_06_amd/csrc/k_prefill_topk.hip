// Prefill chunk: lightning-indexer scoring fused with the per-query top-K, so
// the queries x entries score matrix never reaches memory (DeepSeek V4.1 Flash
// summaries: "DeepSeek V4.1 Flash 如何靠压缩 KV 缓存实现小模型干翻大模型",
// sections "CSA2" (each selecting layer picks its own top-K from the index
// scores) and "FP4 量化 + Bounded Replay" (FP4 indexer keys and queries);
// block-causal visibility as for the other scoring kernels).
//
// A workgroup owns 16 query rows of one request and every entry they see;
// its sixteen waves (four per SIMD, so at most 128 registers each) split the
// entries, and the queries' operands and head weights wait in LDS between
// sweeps rather than in registers.
// Scores are recomputed on the matrix cores in each pass instead of being
// stored; what a pass keeps is small and lives in LDS:
//   pass 0   a 2048-bin histogram per row over a fixed monotone map of the
//            fp32 score (64 bins per octave over [2^-12, 2^21), everything
//            below in bin 0, above in bin 2047);
//   pass 1+  the bin holding the K-th largest score is known, so every entry
//            above it is selected (one bit per entry id) and the entries
//            inside it, usually a few dozen to a few hundred, are collected
//            as candidates (in the row's histogram space) and ranked
//            exactly. A row whose threshold bin holds more than 512 entries
//            is refined by another histogram over that bin instead.
// Ranking and refinement work on the 64-bit composite (order key of the
// score, ~entry id): it is unique per entry and orders by score descending,
// then id ascending, so ties need no special case and every refinement step
// narrows the range by 2^11 until it holds at most 512 entries. Two rows
// share each histogram word (16-bit counts); a collecting row waits while
// the other row of its pair refines.
// The output is each row's selected ids in ascending order (a scan of the
// row's bitmap), then -1 pads.
//
// Matrix-core layout (v_mfma_f32_16x16x32_f16, both operands dequantised
// exactly to fp16 in registers): M = 4 query rows x 4 indexer heads, N = 16
// entries, K = one head's 64 channels in two steps; step ks, lane quarter g,
// element j stand for channel 16 g + 8 ks + j, so a lane's two steps cover
// one 16-channel scale group. C lane l holds the 4 heads of query row l/16
// for entry l%16, so ReLU, head weights and head sum stay in the lane. Four
// M tiles cover the 16 rows and share each dequantised key tile.
#include "csa2_dev.h"
#include "kernels.h"
#include "prefill_ops.h"
#include "block_ops.h"

namespace csa2 {

#define PT_R 16                        // query rows per workgroup
#define PT_MT (PT_R / 4)               // M tiles: 4 rows x 4 heads each
#define PT_WG_PER_CU 1                 // minimum waves per SIMD for the register budget
#define PT_NT 1024                     // threads (16 waves: four per SIMD)
#define PT_WAVES (PT_NT / 64)
static_assert(PT_WAVES >= PT_R, "one wave per row in the resolves");
#define PT_BINS 2048
#define PT_BIN_BITS 11
#define PT_CAND 512                    // candidates per row in a collect pass
#define PT_BITW (kPrefillTopkMaxCols / 32)
#define PT_PAGES 2048
#define PT_B 4                         // 16-entry tiles per batch (two batches in flight per wave)
#define PT_MAX_PASSES 12               // 1 histogram pass + at most 6 refinements + collect

// fixed monotone map of pass 0: IEEE bits of 2^-12, 64 bins per octave
#define PT_BITS0 0x39800000
#define PT_SHIFT0 17

enum { PT_DONE = 0, PT_ALL = 1, PT_HIST0 = 2, PT_HIST = 3, PT_COLLECT = 4 };
// sweep kinds: pass 0; collect passes whose ranges are plain score intervals;
// anything else (refinement histograms, composite bounds)
enum { SW_HIST0 = 0, SW_COLLECT_F = 1, SW_GENERAL = 2 };

struct PtShared {
  // pair p: histogram of rows 2p (low half of each word) and 2p+1 (high
  // half); in a collect pass, row 2p's candidates in words 0..1023 and row
  // 2p+1's in words 1024..2047 (512 composites each)
  uint32_t hist[PT_R / 2][PT_BINS];
  uint32_t bits[PT_R][PT_BITW];      // selected entry ids
  int32_t page[PT_PAGES];
  uint64_t rlo[PT_R], rhi[PT_R];     // composite range still open
  float flo[PT_R], fhi[PT_R];        // the same range as score bounds (when fb)
  int32_t mode[PT_R], shift[PT_R], need[PT_R], vis[PT_R], cnt[PT_R], fb[PT_R];
  int32_t next;                      // the next batch of a sweep (entries), taken by the waves in turn
  v8h qa[PT_MT][2][64];              // each lane's A operands (dequantised queries)
  float qw[PT_R][CSA2_HI];           // head weights of each row
};

__device__ __forceinline__ uint64_t *pt_cand(PtShared &sh, int r) {
  return (uint64_t *)&sh.hist[r >> 1][(r & 1) * (PT_BINS / 2)];
}

// the thread id through an opaque copy: indices and LDS addresses derived
// from it are computed where they are used, not once for the whole kernel
// and held (or spilled) across the passes
__device__ __forceinline__ int pt_tid() {
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  return tid;
}

__device__ __forceinline__ int pt_bin0(float s) {
  const int d = (__float_as_int(s) - PT_BITS0) >> PT_SHIFT0;  // arithmetic: negative scores < 0
  return min(max(d, 0), PT_BINS - 1);
}

// Composite range of bin T of the pass-0 map (keys of non-negative scores
// are their bits with the sign bit set).
__device__ __forceinline__ void pt_bin0_range(int T, uint64_t *lo, uint64_t *hi) {
  const uint32_t base = 0x80000000u + (uint32_t)PT_BITS0;
  const uint32_t klo = T == 0 ? 0u : base + ((uint32_t)T << PT_SHIFT0);
  const uint32_t khi = T == PT_BINS - 1 ? 0xFFFFFFFFu : base + ((uint32_t)(T + 1) << PT_SHIFT0) - 1u;
  *lo = (uint64_t)klo << 32;
  *hi = ((uint64_t)khi << 32) | 0xFFFFFFFFull;
}

// A composite range [lo, hi] that covers whole keys, with key bounds that are
// 0, 0xFFFFFFFF or keys of finite non-negative scores, is the score interval
// [flo, fhi]: key >= klo <=> s >= flo and key > khi <=> s > fhi (-0 ties +0).
__device__ __forceinline__ bool pt_float_bounds(uint64_t lo, uint64_t hi, float *flo, float *fhi) {
  const uint32_t klo = (uint32_t)(lo >> 32), khi = (uint32_t)(hi >> 32);
  const bool whole = (uint32_t)lo == 0u && (uint32_t)hi == 0xFFFFFFFFu;
  const bool lok = klo == 0u || klo >= 0x80000000u;
  const bool hok = khi == 0xFFFFFFFFu || (khi >= 0x80000000u && khi < 0xFF800000u);
  *flo = klo == 0u ? -INFINITY : __uint_as_float(klo & 0x7FFFFFFFu);
  *fhi = khi == 0xFFFFFFFFu ? INFINITY : __uint_as_float(khi & 0x7FFFFFFFu);
  return whole && lok && hok;
}

// wave sums and inclusive scans: the DPP / row-swap forms of block_ops.h
__device__ __forceinline__ uint32_t pt_wave_sum(uint32_t v) { return wave_sum(v); }
__device__ __forceinline__ uint32_t pt_wave_incl_scan(uint32_t v) { return wave_inclusive_scan(v); }

// Wave-level: in half `half` of the pair histogram h, the highest bin T whose
// count together with every higher bin reaches `need` (1 <= need <= total).
// *above = entries in bins above T, *cnt = entries in T. Lane j holds bins
// 256 i + 4 j + c (i < 8, c < 4), read as conflict-free 16-byte loads.
__device__ void pt_find_bin(const uint32_t *h, int half, uint32_t need, int *T, uint32_t *above,
                            uint32_t *cnt) {
  const int lane = pt_tid() & 63;
  uint32_t x[8][4];
  uint32_t seg[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const v4i w = *(const v4i *)(h + 256 * i + 4 * lane);
    uint32_t s = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      x[i][c] = half ? ((uint32_t)w[c] >> 16) : ((uint32_t)w[c] & 0xFFFFu);
      s += x[i][c];
    }
    seg[i] = pt_wave_sum(s);
  }
  uint32_t cum = 0;  // entries in segments above the chosen one
  int is = 0;
  bool found = false;
#pragma unroll
  for (int i = 7; i >= 0; --i) {
    if (!found) {
      if (cum + seg[i] >= need) {
        is = i;
        found = true;
      } else {
        cum += seg[i];
      }
    }
  }
  uint32_t xs[4], ss = 0, segs = 0;
#pragma unroll
  for (int c = 0; c < 4; ++c) xs[c] = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i == is) {
#pragma unroll
      for (int c = 0; c < 4; ++c) xs[c] = x[i][c];
      segs = seg[i];
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) ss += xs[c];
  const uint32_t incl = pt_wave_incl_scan(ss);
  const uint32_t ab = cum + (segs - incl);  // entries in this segment's higher lanes, and above
  const bool hit = ab < need && ab + ss >= need;
  int t = -1;
  uint32_t a = ab, cc = 0;
  if (hit) {
#pragma unroll
    for (int c = 3; c >= 0; --c) {
      if (t < 0) {
        if (a + xs[c] >= need) {
          t = 256 * is + 4 * lane + c;
          cc = xs[c];
        } else {
          a += xs[c];
        }
      }
    }
  }
  const uint64_t m = __ballot(hit);
  const int src = m ? (int)__ffsll((unsigned long long)m) - 1 : 0;  // uniform: from the ballot
  *T = __builtin_amdgcn_readlane(t, src);
  *above = (uint32_t)__builtin_amdgcn_readlane((int)a, src);
  *cnt = (uint32_t)__builtin_amdgcn_readlane((int)cc, src);
}

// Is row r taking part in a sweep of this kind? A collect row waits while
// the other row of its pair refines (they share the pair's LDS region).
__device__ __forceinline__ bool pt_open(const PtShared &sh, int kind, int r) {
  const int md = sh.mode[r];
  if (kind == SW_HIST0) return md == PT_HIST0;
  if (md == PT_HIST) return true;
  return md == PT_COLLECT && sh.mode[r ^ 1] != PT_HIST;
}

// One sweep over the entries of the open rows: recompute every score, then
// per the kind: pass-0 histogram; or, for a collect row, mark the entries
// above its range and keep those inside as candidates; for a refining row,
// the histogram of its range. TILEPAGE: pages of >= 16 entries, so a
// 16-entry tile lies in one page and its addresses are wave-uniform.
template <int KIND, bool TILEPAGE>
__device__ __forceinline__ void pt_sweep(const PrefillTopkArgs &a, PtShared &sh, int b) {
  const int tid = pt_tid();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 15, gq = lane >> 4;
  // the queries' A operands and the head weights of the lane's result rows
  // 4 mt + gq, from LDS for the sweep only (not held across the passes)
  v8h A[PT_MT][2];
  float W[PT_MT][CSA2_HI];
#pragma unroll
  for (int mt = 0; mt < PT_MT; ++mt) {
    A[mt][0] = sh.qa[mt][0][lane];
    A[mt][1] = sh.qa[mt][1][lane];
#pragma unroll
    for (int h = 0; h < CSA2_HI; ++h) W[mt][h] = sh.qw[4 * mt + gq][h];
  }
  // per M tile: the lane's result row (4 mt + gq) and its pass parameters
  int32_t vlim[PT_MT];
  uint32_t inc[PT_MT];
  uint64_t rlo[PT_MT], rhi[PT_MT];
  float flo[PT_MT], fhi[PT_MT];
  int32_t shf[PT_MT];
  bool coll[PT_MT];
  int32_t vmax = 0;
#pragma unroll
  for (int i = 0; i < PT_R; ++i)
    if (pt_open(sh, KIND, i)) vmax = max(vmax, sh.vis[i]);
#pragma unroll
  for (int mt = 0; mt < PT_MT; ++mt) {
    const int r = 4 * mt + gq;
    vlim[mt] = pt_open(sh, KIND, r) ? sh.vis[r] : 0;
    inc[mt] = 1u << (16 * (r & 1));
    rlo[mt] = sh.rlo[r];
    rhi[mt] = sh.rhi[r];
    flo[mt] = sh.flo[r];
    fhi[mt] = sh.fhi[r];
    shf[mt] = sh.shift[r];
    coll[mt] = sh.mode[r] == PT_COLLECT;
  }
  // refinement sweeps: lane g < 4 writes the bitmap halves of row 4 mt + g
  // when that row collects
  bool wbits[PT_MT];
#pragma unroll
  for (int mt = 0; mt < PT_MT; ++mt) {
    const int rr = 4 * mt + (lane & 3);
    wbits[mt] = lane < 4 && KIND != SW_HIST0 && pt_open(sh, KIND, rr) && sh.mode[rr] == PT_COLLECT;
  }
  // collect sweeps: lane L < 16 writes the bitmap half of row L for each tile
  const bool wrow = lane < PT_R && KIND == SW_COLLECT_F && pt_open(sh, KIND, lane) && sh.mode[lane] == PT_COLLECT;
  const int shift = a.c.page_shift;
  const int32_t pmask = (1 << shift) - 1;
  const int64_t bt_row = (int64_t)b * a.c.max_pages;
  const int offc = m * 32 + 8 * gq, offs = m * 4 + gq;  // lane's bytes within a 16-entry tile

  // key tiles of one batch: codes (8 bytes per lane), scale byte, validity
  struct Batch {
    v2f code[PT_B];
    uint32_t scb[PT_B];
    bool eok[PT_B];
  };
  auto load = [&](int32_t base, Batch &bt) {
    if (TILEPAGE) {
      // every page id of the batch first, then one wait
      int32_t pv[PT_B];
#pragma unroll
      for (int u = 0; u < PT_B; ++u) pv[u] = sh.page[min((base + 16 * u) >> shift, PT_PAGES - 1)];
#pragma unroll
      for (int u = 0; u < PT_B; ++u) {
        const int32_t et = base + 16 * u;
        const int32_t page = __builtin_amdgcn_readfirstlane(pv[u]);
        bt.eok[u] = et < vmax && page >= 0 && page < a.c.num_pages;  // uniform
        const int64_t row0 = bt.eok[u] ? ((int64_t)page << shift) + (et & pmask) : 0;
        bt.code[u] = *(const v2f *)(a.c.ix_codes + row0 * 32 + offc);
        bt.scb[u] = a.c.ix_scales[row0 * 4 + offs];
      }
    } else {
#pragma unroll
      for (int u = 0; u < PT_B; ++u) {
        const int32_t e = base + 16 * u + m, pg = e >> shift;
        const int32_t page = (e < vmax && pg < a.c.max_pages) ? a.c.block_table[bt_row + pg] : -1;
        bt.eok[u] = e < vmax && page >= 0 && page < a.c.num_pages;
        const int64_t crow = bt.eok[u] ? ((int64_t)page << shift) + (e & pmask) : 0;
        bt.code[u] = *(const v2f *)(a.c.ix_codes + crow * 32 + 8 * gq);
        bt.scb[u] = a.c.ix_scales[crow * 4 + gq];
      }
    }
  };
  // batches of 16 PT_B entries go to the waves as they ask (a wave that gets
  // fewer issue slots takes fewer), each wave holding two taken ahead
  auto take = [&]() {
    int32_t v = 0;
    if (lane == 0) v = atomicAdd(&sh.next, 16 * PT_B);
    return __builtin_amdgcn_readfirstlane(v);
  };
  Batch cur, nxt;
  int32_t base = take(), nb = take();
  load(base, cur);
  while (base < vmax) {
    // the next batch's loads are in flight while this one is scored; past
    // the end they read row 0 and are dropped (unconditional, so the waits
    // for this batch count the next batch's loads as still outstanding)
    load(nb, nxt);
    const int32_t nnb = take();
    __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of this batch's work
    // branch-free over the batch: tiles past the row ends or on missing pages
    // are masked per lane (their loads read row 0)
#pragma unroll
    for (int u = 0; u < PT_B; ++u) {
      const int32_t et = base + 16 * u;
      const _Float16 s = e4m3_to_f16(cur.scb[u]);
      const v8h b0 = fp4x8_dequant((uint32_t)__float_as_int(cur.code[u][0]), s);
      const v8h b1 = fp4x8_dequant((uint32_t)__float_as_int(cur.code[u][1]), s);
      const int32_t e = et + m;
      if constexpr (KIND == SW_COLLECT_F) {
        float scv[PT_MT];
        bool inrv[PT_MT];
        uint64_t bmv[PT_MT];
#pragma unroll
        for (int mt = 0; mt < PT_MT; ++mt) {
          v4f acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[mt][0], b0, (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[mt][1], b1, acc, 0, 0, 0);
          float sc = 0.f;
#pragma unroll
          for (int h = 0; h < CSA2_HI; ++h) sc = fmaf(W[mt][h], fmaxf(acc[h], 0.f), sc);
          const bool v = cur.eok[u] && e < vlim[mt];
          const bool sel = v && sc > fhi[mt];
          inrv[mt] = v && !sel && sc >= flo[mt];
          bmv[mt] = __ballot(sel);
          scv[mt] = sc;
        }
        if (et < vmax) {  // uniform
          const int gl = lane & 3, ml = (lane >> 2) & 3;
          uint64_t bsel = bmv[0];
          bsel = ml == 1 ? bmv[1] : bsel;
          bsel = ml == 2 ? bmv[2] : bsel;
          bsel = ml == 3 ? bmv[3] : bsel;
          if (wrow) ((uint16_t *)&sh.bits[lane][0])[et >> 4] = (uint16_t)(bsel >> (16 * gl));
        }
        if (__ballot(inrv[0] || inrv[1] || inrv[2] || inrv[3])) {  // uniform, and rare
#pragma unroll
          for (int mt = 0; mt < PT_MT; ++mt) {
            if (inrv[mt]) {
              const int r = 4 * mt + gq;
              const uint64_t comp = ((uint64_t)score_key(scv[mt]) << 32) | (uint64_t)(~(uint32_t)e);
              const uint32_t slot = atomicAdd((uint32_t *)&sh.cnt[r], 1u);
              if (slot < PT_CAND) pt_cand(sh, r)[slot] = comp;
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        continue;
      }
#pragma unroll
      for (int mt = 0; mt < PT_MT; ++mt) {
        v4f acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[mt][0], b0, (v4f){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[mt][1], b1, acc, 0, 0, 0);
        float sc = 0.f;
#pragma unroll
        for (int h = 0; h < CSA2_HI; ++h) sc = fmaf(W[mt][h], fmaxf(acc[h], 0.f), sc);
        const bool v = cur.eok[u] && e < vlim[mt];
        const int r = 4 * mt + gq;
        if (KIND == SW_HIST0) {
          atomicAdd(&sh.hist[r >> 1][pt_bin0(sc)], v ? inc[mt] : 0u);
          continue;
        }
        bool sel, inr;
        uint64_t comp = 0;
        if (KIND == SW_COLLECT_F) {
          sel = v && sc > fhi[mt];
          inr = v && !sel && sc >= flo[mt];
        } else {
          comp = ((uint64_t)score_key(sc) << 32) | (uint64_t)(~(uint32_t)e);
          sel = v && coll[mt] && comp > rhi[mt];
          inr = v && comp >= rlo[mt] && comp <= rhi[mt];
        }
        if (inr) {
          if (KIND == SW_COLLECT_F || coll[mt]) {
            if (KIND == SW_COLLECT_F) comp = ((uint64_t)score_key(sc) << 32) | (uint64_t)(~(uint32_t)e);
            const uint32_t slot = atomicAdd((uint32_t *)&sh.cnt[r], 1u);
            if (slot < PT_CAND) pt_cand(sh, r)[slot] = comp;
          } else {
            atomicAdd(&sh.hist[r >> 1][(uint32_t)((comp - rlo[mt]) >> shf[mt])], inc[mt]);
          }
        }
        // the 16 lanes of row 4 mt + g hold the 16 consecutive ids of one half
        // of a bitmap word; lane g (< 4) writes that half (each half belongs to
        // one tile, so a plain 16-bit store)
        const uint64_t bm = __ballot(sel);
        if (wbits[mt] && et < vmax)
          ((uint16_t *)&sh.bits[4 * mt + lane][0])[et >> 4] = (uint16_t)(bm >> (16 * lane));
      }
      __builtin_amdgcn_sched_barrier(0);  // one tile at a time: bounded register use
    }
    cur = nxt;
    base = nb;
    nb = nnb;
  }
}

// After a histogram pass: the next state of row r (one wave).
__device__ void pt_resolve_hist(PtShared &sh, int r) {
  const int lane = pt_tid() & 63;
  const int md = sh.mode[r];
  const uint32_t need = (uint32_t)sh.need[r];
  int T;
  uint32_t above, c;
  pt_find_bin(sh.hist[r >> 1], r & 1, need, &T, &above, &c);
  const uint64_t rlo = sh.rlo[r], rhi = sh.rhi[r];
  int nm = PT_COLLECT, nshift = 0;
  uint64_t nlo, nhi;
  uint32_t nneed;
  if (T < 0) {
    // fewer entries in the range than still needed (entries on missing pages
    // are never scored): take the whole range. Every composite is >= 1
    // (its low word is ~id), so nhi = 0 selects everything.
    nlo = rlo;
    nhi = rlo > 0 ? rlo - 1 : 0;
    nneed = 0;
  } else {
    uint64_t lo, hi;
    if (md == PT_HIST0) {
      pt_bin0_range(T, &lo, &hi);
    } else {
      const int sh_ = sh.shift[r];
      lo = rlo + ((uint64_t)T << sh_);
      const uint64_t span = rhi - lo, w = (1ull << sh_) - 1ull;
      hi = lo + (span < w ? span : w);
    }
    const uint32_t rest = need - above;  // entries still to take from bin T (>= 1)
    nlo = lo;
    nhi = hi;
    nneed = rest;
    if (c <= PT_CAND) {
      // collect the bin, rank it
    } else if (c == rest) {
      // every entry of the bin is taken: collect nothing, select down to lo
      nhi = lo > 0 ? lo - 1 : 0;
      nneed = 0;
    } else {
      nm = PT_HIST;
      const uint64_t d = hi - lo;
      const int bl = d ? 64 - __clzll((long long)d) : 0;
      nshift = bl > PT_BIN_BITS ? bl - PT_BIN_BITS : 0;
    }
  }
  float flo, fhi;
  const bool fb = pt_float_bounds(nlo, nhi, &flo, &fhi);
  if (lane == 0) {
    sh.mode[r] = nm;
    sh.rlo[r] = nlo;
    sh.rhi[r] = nhi;
    sh.flo[r] = flo;
    sh.fhi[r] = fhi;
    sh.fb[r] = fb ? 1 : 0;
    sh.shift[r] = nshift;
    sh.need[r] = (int32_t)nneed;
  }
}

// After a collect pass: select the `need` largest candidates (composites are
// unique, so exactly those at or above the need-th largest). The need-th
// largest is found bit by bit from the top (radix selection): every
// candidate lies in the row's range [rlo, rhi], so the bits above the
// highest bit where rlo and rhi differ are common; at each lower bit the
// count of candidates in the upper half of what is left decides that bit.
__device__ void pt_resolve_collect(PtShared &sh, int r) {
  const int lane = pt_tid() & 63;
  const int n = min(sh.cnt[r], PT_CAND);
  const uint32_t need = (uint32_t)sh.need[r];
  const uint64_t *cand = pt_cand(sh, r);
  const int kn = (n + 63) >> 6;  // candidate slots in use per lane (uniform)
  uint64_t mine[PT_CAND / 64];
#pragma unroll
  for (int k = 0; k < PT_CAND / 64; ++k) mine[k] = lane + 64 * k < n ? cand[lane + 64 * k] : 0ull;
  const uint64_t rlo = sh.rlo[r], rhi = sh.rhi[r];
  const uint64_t d = rlo ^ rhi;
  const int top = d ? 63 - __clzll((long long)d) : -1;
  uint64_t P = top >= 0 ? rlo & ~((2ull << top) - 1ull) : rlo;  // the common bits (none when top = 63)
  uint32_t above = 0;  // candidates above what is left
  for (int bt = top; bt >= 0; --bt) {
    const uint64_t hi = (P >> bt) | 1ull;
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < PT_CAND / 64; ++k) {
      if (k < kn) c += (uint32_t)__popcll(__ballot(lane + 64 * k < n && (mine[k] >> bt) == hi));
    }
    if (above + c >= need) P |= 1ull << bt;
    else above += c;
  }
#pragma unroll
  for (int k = 0; k < PT_CAND / 64; ++k) {
    if (lane + 64 * k < n && need > 0 && mine[k] >= P) {
      const uint32_t e = ~(uint32_t)mine[k];
      atomicOr(&sh.bits[r][e >> 5], 1u << (e & 31));
    }
  }
  if (lane == 0) sh.mode[r] = PT_DONE;
}

template <bool TILEPAGE>
__global__ __launch_bounds__(PT_NT, PT_WG_PER_CU) void k_prefill_topk(PrefillTopkArgs a) {
  __shared__ __attribute__((aligned(16))) PtShared sh;
  const int qb = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int K = a.k;

  if (tid < PT_R) {
    const int t = qb * PT_R + tid;
    int32_t V = 0;
    if (t < a.nq) V = min(visible_entries(a.c, a.q_pos, b, a.nq, t), a.n_cols);
    sh.vis[tid] = V;
    sh.need[tid] = K;
    sh.mode[tid] = t >= a.nq ? PT_DONE : (V <= K ? PT_ALL : PT_HIST0);
    sh.rlo[tid] = 0;
    sh.rhi[tid] = ~0ull;
    sh.flo[tid] = -INFINITY;
    sh.fhi[tid] = INFINITY;
    sh.fb[tid] = 0;
    sh.shift[tid] = 0;
    sh.cnt[tid] = 0;
  }
  if (tid == 0) sh.next = 0;
  {
    v4i z = {0, 0, 0, 0};
    for (int i = tid; i < PT_R * PT_BITW / 4; i += PT_NT) ((v4i *)&sh.bits[0][0])[i] = z;
    for (int i = tid; i < (PT_R / 2) * PT_BINS / 4; i += PT_NT) ((v4i *)&sh.hist[0][0])[i] = z;
  }
  __syncthreads();
  int32_t vmax = 0;
  bool any = false;
#pragma unroll
  for (int i = 0; i < PT_R; ++i) {
    vmax = max(vmax, sh.vis[i]);
    any |= sh.mode[i] == PT_HIST0;
  }
  if (TILEPAGE) {
    const int32_t npg = (vmax + (1 << a.c.page_shift) - 1) >> a.c.page_shift;
    for (int i = tid; i < npg && i < PT_PAGES; i += PT_NT)
      sh.page[i] = i < a.c.max_pages ? a.c.block_table[(int64_t)b * a.c.max_pages + i] : -1;
  }

  // A operands (rows 4 mt + m/4, head m%4) of every lane, by wave 0, and
  // the head weights of every row, into LDS
  if (wave == 0) {
    const int m = lane & 15, gq = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < PT_MT; ++mt) {
      const int ta = qb * PT_R + 4 * mt + (m >> 2), h = m & 3;
      const int64_t row_a = (int64_t)b * a.nq + min(ta, a.nq - 1);
      const v2f c = *(const v2f *)(a.qix_codes + (row_a * CSA2_HI + h) * 32 + 8 * gq);
      const uint32_t sb = a.qix_scales[(row_a * CSA2_HI + h) * 4 + gq];
      const _Float16 s = ta < a.nq ? e4m3_to_f16(sb) : (_Float16)0.f;
      sh.qa[mt][0][lane] = fp4x8_dequant((uint32_t)__float_as_int(c[0]), s);
      sh.qa[mt][1][lane] = fp4x8_dequant((uint32_t)__float_as_int(c[1]), s);
    }
    const int te = qb * PT_R + (lane >> 2);
    const int64_t row_e = (int64_t)b * a.nq + min(te, a.nq - 1);
    sh.qw[lane >> 2][lane & 3] = a.w[row_e * CSA2_HI + (lane & 3)];
  }
  __syncthreads();

  if (any) {
    pt_sweep<SW_HIST0, TILEPAGE>(a, sh, b);
    __syncthreads();
    if (wave < PT_R && sh.mode[wave] == PT_HIST0) pt_resolve_hist(sh, wave);  // one row per wave
    __syncthreads();
  }
  for (int pass = 1; pass < PT_MAX_PASSES; ++pass) {
    bool open = false, general = false;
#pragma unroll
    for (int i = 0; i < PT_R; ++i) {
      const int md = sh.mode[i];
      open |= md == PT_HIST || md == PT_COLLECT;
      general |= md == PT_HIST || (md == PT_COLLECT && !sh.fb[i]);
    }
    if (!open) break;  // uniform
    const int ptid = pt_tid(), pwave = __builtin_amdgcn_readfirstlane(ptid >> 6);
    // refining pairs start from an empty histogram; collect rows from no candidates
    for (int i = ptid; i < (PT_R / 2) * PT_BINS / 4; i += PT_NT) {
      const int p = i / (PT_BINS / 4);
      if (sh.mode[2 * p] == PT_HIST || sh.mode[2 * p + 1] == PT_HIST)
        ((v4i *)&sh.hist[0][0])[i] = (v4i){0, 0, 0, 0};
    }
    if (ptid < PT_R) sh.cnt[ptid] = 0;
    if (ptid == 0) sh.next = 0;
    __syncthreads();
    if (general) pt_sweep<SW_GENERAL, TILEPAGE>(a, sh, b);
    else pt_sweep<SW_COLLECT_F, TILEPAGE>(a, sh, b);
    __syncthreads();
    // one row per wave; the modes as the sweep saw them are read before any
    // row's resolve changes its own
    const int md = pwave < PT_R ? sh.mode[pwave] : PT_DONE, mdo = pwave < PT_R ? sh.mode[pwave ^ 1] : PT_DONE;
    __syncthreads();
    if (md == PT_HIST) pt_resolve_hist(sh, pwave);
    else if (md == PT_COLLECT && mdo != PT_HIST) pt_resolve_collect(sh, pwave);
    __syncthreads();
  }

  // ascending ids of each row, then -1 pads (one wave per row)
  for (int r = wave; r < PT_R; r += PT_WAVES) {
    const int t = qb * PT_R + r;
    if (t >= a.nq) continue;
    int32_t *out = a.idx_out + ((int64_t)b * a.nq + t) * K;
    const int32_t V = sh.vis[r];
    if (sh.mode[r] == PT_ALL) {
      for (int p = lane; p < K; p += 64) out[p] = p < V ? p : -1;
      continue;
    }
    const int nw = (V + 31) >> 5;
    int32_t pos = 0;
    for (int w0 = 0; w0 < nw; w0 += 64) {
      const int wi = w0 + lane;
      uint32_t x = wi < nw ? sh.bits[r][wi] : 0u;
      const uint32_t c = (uint32_t)__popc(x);
      const uint32_t incl = pt_wave_incl_scan(c);
      int32_t p = pos + (int32_t)(incl - c);
      while (x) {
        const int bit = __ffs(x) - 1;
        x &= x - 1;
        if (p < K) out[p] = wi * 32 + bit;
        ++p;
      }
      pos += __builtin_amdgcn_readlane((int)incl, 63);
    }
    for (int p = pos + lane; p < K; p += 64) out[p] = -1;
  }
}

hipError_t launch_prefill_topk(const PrefillTopkArgs &a, int batch, hipStream_t st) {
  if (a.n_cols < 1 || a.n_cols > kPrefillTopkMaxCols || a.k < 1 || a.nq < 1 || batch < 1)
    return hipErrorInvalidValue;
  dim3 grid((unsigned)((a.nq + PT_R - 1) / PT_R), (unsigned)batch);
  // pages of >= 16 entries: every 16-entry tile lies in one page, and the
  // page ids of a row (at most 32768 / 16) fit the LDS cache
  if (a.c.page_shift >= 4)
    hipLaunchKernelGGL(k_prefill_topk<true>, grid, dim3(PT_NT), 0, st, a);
  else
    hipLaunchKernelGGL(k_prefill_topk<false>, grid, dim3(PT_NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace csa2
