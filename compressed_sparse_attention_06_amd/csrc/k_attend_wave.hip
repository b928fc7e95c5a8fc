// Sparse attention over the selected compressed entries plus the sliding
// window, paired-wave form, gfx950 (DeepSeek V4.1 Flash summaries: "DeepSeek
// V4.1 Flash 如何靠压缩 KV 缓存实现小模型干翻大模型", section "CSA2": every mode
// attends with its own global Q and its own SWA KV; all heads share one
// compressed latent, so the latent row is both key and value).
//
// Same units and partials as k_attend_seg (units of 128 positions; the units
// of all rows, row after row, shared out over G workgroups; rows cut between
// workgroups combined by k_merge_seg), with another split inside a unit:
//  * eight waves (two per SIMD) form four pairs; pair p takes positions
//    32 p .. 32 p + 31 of every unit, as two tiles of 16, and keeps its own
//    online-softmax state for the row;
//  * the two waves of a pair split the 512 channels: wave half h owns
//    channels 256 h .. 256 h + 255 for the logits (a partial S over its
//    channels) and for the output (O[16 heads][its 256 channels], 64 fp32
//    registers per lane);
//  * lane (n, g) holds the 64 channels 256 h + 64 g .. + 63 of position n of
//    each tile (32 FP4 code bytes + 4 scale bytes, or 64 E4M3 bytes) and
//    dequantises them to fp16 eight at a time;
//  * S^T = R Q^T with v_mfma_f32_16x16x32_f16 (M = positions, N = the 16 heads,
//    K = the wave's 256 channels in 8 steps; step ks pairs channel
//    256 h + 64 g + 8 ks + e of R with the same channel of Q, whose fp16 hi and
//    lo halves stay in registers). Lane (n, g) receives S[head n][position
//    4 g + i] of each tile. The pair adds its two partial S through LDS, so
//    both waves hold the same logits and take the same softmax steps;
//  * the eight logits per lane are, after the softmax, the A operand
//    P[head n][k] of O += P R over the 32 positions, with k = 8 g + e standing
//    for position 16 (e / 4) + 4 g + e % 4;
//  * each wave writes its dequantised channels to its own LDS tile
//    [32 positions][256 channels] fp16 (rows padded by 16 bytes, so that the
//    16 rows of a store or of a transposed load start in 16 different bank
//    groups and every address is a lane base plus a constant), and
//    ds_read_b64_tr_b16 returns the B operand of the product (R with positions
//    along K) for each block of 16 of its output channels;
//  * O and the sum are rescaled only in chunks that raise some head's logit
//    more than 2^4 above its reference maximum (the weights are then at most
//    16, which fp16 holds exactly enough; the final normalisation divides by
//    the sum taken against the same reference).
// No workgroup barrier per unit: the two waves of a pair exchange their
// partial S through LDS with a handshake of their own (a posted and an
// acknowledged unit count per wave), so the four pairs run independently
// between the row's start and its end.
#include "csa2_dev.h"
#include "kernels.h"
#include "attend_common.h"

namespace csa2 {

#define PW_NT 512   // eight waves: four pairs
#define PW_RP 264   // halfs per LDS row of a wave's R tile (256 + 8)
#define PW_QP 520   // halfs per LDS row of the staged Q (512 + 8)
#define PW_SP 260   // floats per row of a wave's staged O at the row's end (256 + 4)
#define PW_SLACK 4.0f  // log2 of the largest weight before the reference maximum moves

struct PairShared {
  union {
    _Float16 r[8][32 * PW_RP];  // each wave's R tile: 32 positions x its 256 channels
    struct {
      _Float16 hi[CSA2_H * PW_QP];
      _Float16 lo[CSA2_H * PW_QP];
      float qexp[CSA2_H];
    } q;                                // Q of the row, staged once per row
    float stg[8][32 * PW_RP / 2];       // row end: each wave's O [16 heads][PW_SP], in its own R tile's storage
  };
  v4f sx[8][2][64];                     // each wave's partial S of its two tiles
  int sflag[8], sack[8];                // per wave: last unit whose partial S is posted / was read by the partner
  float wm[4][CSA2_H], wl[4][CSA2_H];   // each pair's running max and sum
};

// One lane's share of a tile position: 32 code bytes and 4 scale bytes of an
// entry, or the first 32 of its 64 E4M3 bytes of a window row (the other 32
// are loaded when the unit is computed, which keeps the prefetch buffer small).
struct PwSlice {
  v4i c[2];
  uint32_t w;  // entry: its 4 scale bytes; window row: its row scale (fp32 bits), when the window has them
  int kind;    // 0 no row, 1 entry, 2 window row
};

// The loads in flight for unit j, issued while unit j - 1 computes: the rows
// of unit j, the page words of unit j + 1 and the ids of unit j + 2 (for the
// lane's position in each of its pair's two tiles).
struct PwSet {
  PwSlice t[2];
  int32_t pg[2];
  int32_t id[2];
};

enum { PW_NONE = 0, PW_ENTRY = 1, PW_WINDOW = 2 };

// kind of the tile whose first position is p (uniform per wave)
__device__ __forceinline__ int pw_tile_type(int32_t p, int32_t kw, int32_t span) {
  return p < kw ? PW_ENTRY : (p < span ? PW_WINDOW : PW_NONE);
}

__device__ __forceinline__ float max_rows4(float t) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
  const float s = fmax_nc(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return fmax_nc(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// The loads of a unit always have the same count, each from an in-bounds
// address (a position that is not a row reads a fixed valid word or row),
// and nothing reads a loaded value before the unit is computed: the wait
// counts are then the same on every path, so the loads of the next unit stay
// in flight while the current one computes.

// id of position p of the row's set (ibase: the row's ids, or any valid word
// when use is false; use, ibase uniform)
__device__ __forceinline__ int32_t pw_fetch_id(const AttendArgs &a, const int32_t *ibase, bool use, int32_t p) {
  return ibase[use ? (uint32_t)min(p, a.k - 1) : 0u];
}

// block-table word of the page holding entry id (btab: the request's
// block-table row; the page index is clamped into it); use false (a tile
// with no entries): the row's first word, read without waiting for id
__device__ __forceinline__ int32_t pw_fetch_page(const AttendArgs &a, const int32_t *btab, bool use, int32_t id) {
  if (use) return btab[(uint32_t)min(max(id, 0) >> a.c.page_shift, a.c.max_pages - 1)];
  return btab[0];
}

// request-local window row of tile position p (0 when it has none)
__device__ __forceinline__ int32_t pw_window_row(int32_t p, int32_t kw, int32_t span, int32_t wf, int32_t wl,
                                                 bool &ok) {
  const int32_t jw = wf + (p - kw);
  ok = p < span && jw <= wl;
  return ok ? jw : 0;
}

// Rows of position p, channels cb .. cb + 63, of a tile of kind ty (uniform;
// PW_NONE past the row's units): an entry, a window row, or nothing; three
// loads in every case. cbase / sbase: the cache's code and scale arrays at the
// lane's channels; elim: the ids below it are visible entries with a page
// slot in the block table (the row's entry count, capped by the table);
// wcodes / wscale: the request's window rows and row scales (uniform). A
// position that is not a row (kind 0) loads physical row 0 (or window row 0)
// and is masked where the bytes are used: its entry scale word is taken as 0
// (E2M1 has no NaN or infinity, so its codes dequantise to 0), its window
// bytes as 0 and its row scale as 1.
__device__ __forceinline__ void pw_fetch_rows(const AttendArgs &a, int ty, int32_t p, int cb, int32_t elim,
                                              int32_t id, int32_t page, int32_t kw, int32_t span,
                                              const uint8_t *cbase, const uint8_t *sbase, const uint8_t *wcodes,
                                              const float *wscale, int32_t wf, int32_t wl, PwSlice &s) {
  if (ty == PW_WINDOW) {
    bool ok;
    const int32_t wr = pw_window_row(p, kw, span, wf, wl, ok);
    const uint8_t *cp = wcodes + (uint32_t)wr * CSA2_D + cb;
    const uint32_t *sp = wscale ? (const uint32_t *)(wscale + wr) : (const uint32_t *)a.c.kv_scales;
    s.c[0] = *(const v4i *)cp;
    s.c[1] = *(const v4i *)(cp + 16);
    s.w = *sp;
    s.kind = ok ? 2 : 0;
  } else {
    // cache rows number fewer than 2^31, so the row index fits 32 bits
    const int sh = a.c.page_shift;
    const bool ok = ty == PW_ENTRY && p < a.k && (uint32_t)id < (uint32_t)elim &&
                    (uint32_t)page < (uint32_t)a.c.num_pages;
    const uint32_t crow = ok ? ((uint32_t)page << sh) | ((uint32_t)id & ((1u << sh) - 1u)) : 0u;
    const uint8_t *cp = cbase + (uint64_t)crow * 256u;
    s.c[0] = *(const v4i *)cp;
    s.c[1] = *(const v4i *)(cp + 16);
    s.w = *(const uint32_t *)(sbase + (uint64_t)crow * 32u);
    s.kind = ok ? 1 : 0;
  }
}

// the other 32 of the lane's window bytes (raw; masked where they are used)
__device__ __forceinline__ void pw_window_tail(bool win, const uint8_t *wcodes, const uint8_t *qrow, int32_t wr,
                                               int cb, v4i *t) {
  const uint8_t *src = win ? wcodes + (uint32_t)wr * CSA2_D + cb + 32 : qrow;
  t[0] = *(const v4i *)src;
  t[1] = *(const v4i *)(src + 16);
}

// R operand of step ks: channels cb + 8 ks + e of the lane's position
template <int TY>
__device__ __forceinline__ v8h pw_operand(const PwSlice &f, const v2h *sc, const v4i *t, int ks) {
  if constexpr (TY == PW_WINDOW) {
    const int w0 = 2 * ks, w1 = 2 * ks + 1;
    const bool ok = f.kind == 2;  // no bytes of a position without a row
    const uint32_t x0 = ok ? (uint32_t)(w0 < 8 ? f.c[w0 / 4][w0 % 4] : t[(w0 - 8) / 4][w0 % 4]) : 0u;
    const uint32_t x1 = ok ? (uint32_t)(w1 < 8 ? f.c[w1 / 4][w1 % 4] : t[(w1 - 8) / 4][w1 % 4]) : 0u;
    const v4h h0 = e4m3x4_to_f16(x0), h1 = e4m3x4_to_f16(x1);
    return (v8h){h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
  } else {
    return fp4x8_dequant((uint32_t)f.c[ks / 4][ks % 4], sc[ks / 4][(ks / 2) % 2]);
  }
}

// QK of one tile over the wave's channels: partial S^T into acc (hi and lo
// products into one accumulator), the dequantised rows into the wave's R tile
// at wrow_lds; then the window row scales of positions 4 g + i (from the lanes
// that loaded them), gathered here, where the tile's loads have been waited for.
template <int TY>
__device__ __forceinline__ void pw_qk(const PwSlice &f, const v4i *t, const v8h *qh, const v8h *ql,
                                      _Float16 *wrow_lds, bool has_rs, v4f &acc, float *rs) {
  v2h sc[2];
  if constexpr (TY != PW_WINDOW) {
    const uint32_t sw = (f.kind == 1) ? f.w : 0u;  // zero scales for a position without a row
    sc[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
    sc[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, true);
  }
  acc = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const v8h r = pw_operand<TY>(f, sc, t, ks);
    *(v8h *)(wrow_lds + 8 * ks) = r;
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(r, qh[ks], acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(r, ql[ks], acc, 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);  // one step's operand at a time: the dequantised rows are not kept
  }
  const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    rs[i] = (TY == PW_WINDOW && has_rs) ? __shfl(f.kind == 2 ? __uint_as_float(f.w) : 1.f, 4 * g + i) : 1.f;
}

// Logits, online softmax and O += P R of one chunk, given the full S of both
// tiles (ty: tile kinds, for the window row scales).
template <bool WIN>
__device__ __forceinline__ void pw_softmax_pv(const _Float16 *rt, const v4f *S, const PwSlice *cur,
                                              const float (*rs)[4], float qs, uint32_t tr_base, float &m_run,
                                              float &l_run, v4f *o) {
  const int lane = threadIdx.x & 63, g = lane >> 4;
  // rows present at positions 4 g .. 4 g + 3 of each tile (lanes 0-15 hold positions 0-15)
  const uint32_t v0 = ((uint32_t)__ballot(cur[0].kind != 0) >> (4 * g)) & 15u;
  const uint32_t v1 = ((uint32_t)__ballot(cur[1].kind != 0) >> (4 * g)) & 15u;
  float z[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    z[0][i] = ((v0 >> i) & 1u) ? S[0][i] * (WIN ? qs * rs[0][i] : qs) : -INFINITY;
    z[1][i] = ((v1 >> i) & 1u) ? S[1][i] * (WIN ? qs * rs[1][i] : qs) : -INFINITY;
  }
  float cm = fmax_nc(fmax_nc(fmax_nc(z[0][0], z[0][1]), fmax_nc(z[0][2], z[0][3])),
                     fmax_nc(fmax_nc(z[1][0], z[1][1]), fmax_nc(z[1][2], z[1][3])));
  cm = max_rows4(cm);
  // m_run is the reference of the weights, not always the maximum: it moves
  // (every head to its own maximum, with O and the sum rescaled) only when
  // some head's logit exceeds it by more than PW_SLACK, so the weights stay
  // below 2^PW_SLACK and most chunks skip the rescale
  const float m_new = fmax_nc(m_run, cm);
  if (__ballot(m_new > m_run + PW_SLACK) != 0) {  // uniform
    const float mr = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - mr);  // 0 while m_run is -inf
    l_run *= alpha;
    float ah[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) ah[i] = __shfl(alpha, 4 * g + i);  // heads 4 g + i of the O blocks
#pragma unroll
    for (int q = 0; q < 16; ++q) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[q][i] *= ah[i];
    }
    m_run = m_new;
  }
  const float mref = (m_run == -INFINITY) ? 0.f : m_run;
  v8h pa;
  float ps = 0.f;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = __builtin_amdgcn_exp2f(z[t][i] - mref);  // 0 for a position without a row
      ps += p;
      pa[4 * t + i] = (_Float16)(WIN ? p * rs[t][i] : p);
    }
  }
  l_run += ps;
  // block q (channels 16 q .. 16 q + 15 of the wave): lane (c, rq) of row group
  // g reads channels 16 q + 4 rq .. + 3 of rows 4 g + c and 16 + 4 g + c
  // the reads run four blocks ahead of the products
  v4s t0[4], t1[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    t0[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(rt + tr_base + 16 * q));
    t1[q] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(rt + tr_base + 16 * PW_RP + 16 * q));
  }
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const v4h h0 = __builtin_bit_cast(v4h, t0[q & 3]), h1 = __builtin_bit_cast(v4h, t1[q & 3]);
    const v8h rb = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
    o[q] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, rb, o[q], 0, 0, 0);
    if (q + 4 < 16) {
      t0[q & 3] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(rt + tr_base + 16 * (q + 4)));
      t1[q & 3] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(rt + tr_base + 16 * PW_RP + 16 * (q + 4)));
    }
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // the first four blocks' reads
#pragma unroll
  for (int q = 0; q < 12; ++q) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one product
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // the reads of block q + 4
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
}

// Q of query row r: this thread's 16 fp32 values (head tid / 32, channels
// 16 (tid % 32) + [0, 16)).
__device__ __forceinline__ void pw_load_q16(const AttendArgs &a, int32_t r, float *qv) {
  const int tid = threadIdx.x;
  const float *src = a.q + ((int64_t)r * CSA2_H + (tid >> 5)) * CSA2_D + (tid & 31) * 16;
#pragma unroll
  for (int i = 0; i < 16; i += 4) {
    const v4f x = *(const v4f *)(src + i);
    qv[i] = x[0];
    qv[i + 1] = x[1];
    qv[i + 2] = x[2];
    qv[i + 3] = x[3];
  }
}

// The row ends in this workgroup: combine the four pairs' states (common
// reference: the largest of their maxima), then write the row whole
// (normalised, with its lse) or leave its partial in the workgroup's slot.
// Each wave stages its O in its own R tile's storage, which no other wave
// touches, so one barrier precedes the combine and one follows it (before
// the next row's rows overwrite the tiles).
__device__ __forceinline__ void pw_finish(const AttendArgs &a, const SegArgs &s, PairShared &sh, int wg,
                                          int32_t row, int32_t first_row, int64_t u_begin, int64_t u_end,
                                          float m_run, float l_run, const v4f *o) {
  // indices and LDS addresses from an opaque copy of the thread id, so that
  // none of them is computed once and kept live across the unit loop
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = tid >> 6, pair = wave >> 1, half = wave & 1;
  const int n = lane & 15, g = lane >> 4;
  const float l_tot = sum_rows4(l_run);
  if (half == 0 && g == 0) {  // both waves of a pair hold the same state
    sh.wm[pair][n] = m_run;
    sh.wl[pair][n] = l_tot;
  }
  asm volatile("" ::: "memory");  // after the wave's last reads of its R tile
  float *st = sh.stg[wave];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) st[(4 * g + i) * PW_SP + 16 * q + n] = o[q][i];
  }
  __syncthreads();
  const int64_t r0 = (int64_t)row * s.U;
  const bool whole = r0 >= u_begin && r0 + s.U <= u_end;
  const int slot = (row == first_row) ? 0 : 1;
  float *part = a.part + ((int64_t)wg * 2 + slot) * CSA2_H * kPartStride;
  // 16 x 512 outputs as 2048 float4, four per thread, summed over the pairs
  // (pair p's channel c is in wave 2 p + c / 256)
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int v = tid + PW_NT * jj, h = v >> 7, c = (v & 127) * 4, hf = c >> 8, cc = c & 255;
    const float M = fmax_nc(fmax_nc(sh.wm[0][h], sh.wm[1][h]), fmax_nc(sh.wm[2][h], sh.wm[3][h]));
    const float mr = (M == -INFINITY) ? 0.f : M;
    float f[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) f[p] = __builtin_amdgcn_exp2f(sh.wm[p][h] - mr);  // 0 for a pair with no row
    const v4f o0 = *(const v4f *)&sh.stg[hf][h * PW_SP + cc], o1 = *(const v4f *)&sh.stg[2 + hf][h * PW_SP + cc];
    const v4f o2 = *(const v4f *)&sh.stg[4 + hf][h * PW_SP + cc], o3 = *(const v4f *)&sh.stg[6 + hf][h * PW_SP + cc];
    const v4f x = (o0 * f[0] + o1 * f[1]) + (o2 * f[2] + o3 * f[3]);
    if (whole) {
      const float L = (sh.wl[0][h] * f[0] + sh.wl[1][h] * f[1]) + (sh.wl[2][h] * f[2] + sh.wl[3][h] * f[3]);
      const float inv = (L > 0.f) ? 1.f / L : 0.f;
      *(v4f *)&s.out[((int64_t)row * CSA2_H + h) * CSA2_D + c] = x * inv;
    } else {
      store_wt(&part[(int64_t)h * kPartStride + c], x);
    }
  }
  if (tid < CSA2_H) {
    const int h = tid;
    const float M = fmax_nc(fmax_nc(sh.wm[0][h], sh.wm[1][h]), fmax_nc(sh.wm[2][h], sh.wm[3][h]));
    const float mr = (M == -INFINITY) ? 0.f : M;
    const float L = (sh.wl[0][h] * __builtin_amdgcn_exp2f(sh.wm[0][h] - mr) +
                     sh.wl[1][h] * __builtin_amdgcn_exp2f(sh.wm[1][h] - mr)) +
                    (sh.wl[2][h] * __builtin_amdgcn_exp2f(sh.wm[2][h] - mr) +
                     sh.wl[3][h] * __builtin_amdgcn_exp2f(sh.wm[3][h] - mr));
    if (whole) {
      s.lse[(int64_t)row * CSA2_H + h] = (L > 0.f) ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
    } else {
      part[(int64_t)h * kPartStride + CSA2_D] = M;
      part[(int64_t)h * kPartStride + CSA2_D + 1] = L;
    }
  }
  __syncthreads();  // the staged O and the pair states are read before the next row
}

// Pair-level handshake through LDS (the two waves of a pair run on
// different SIMDs of the same compute unit, so the awaited wave always gets
// there); the wait gives up after ~2^22 polls, so no wave can hang on it.
__device__ __forceinline__ void pw_post(int *f, int v) {
  if ((threadIdx.x & 63) == 0) __hip_atomic_store(f, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void pw_wait(int *f, int v) {
  for (int it = 0; it < (1 << 22); ++it) {
    if (__hip_atomic_load(f, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= v) break;
    __builtin_amdgcn_s_sleep(1);
  }
}

__global__ __launch_bounds__(PW_NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attend_wave(AttendArgs a,
                                                                                                  SegArgs s) {
  __shared__ __attribute__((aligned(16))) PairShared sh;
  const int wg = s.xcd ? xcd_order(blockIdx.x, gridDim.x) : blockIdx.x;
  const int32_t U = s.U;
  const int64_t u_begin = (int64_t)wg * s.T / s.G, u_end = (int64_t)(wg + 1) * s.T / s.G;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = tid >> 6, pair = wave >> 1, half = wave & 1;
  const int n = lane & 15, g = lane >> 4;
  const int cb = 256 * half + 64 * g;  // the lane's first channel
  const uint8_t *cbase = a.c.kv_codes + cb / 2, *sbase = a.c.kv_scales + cb / 16;
  const int32_t first_row = (int32_t)(u_begin / U);
  const int32_t kw = seg_kw(a.k);
  const int32_t span = kw + (a.win_codes ? a.win_cap : 0);
  _Float16 *rt = sh.r[wave];
  // R tile addresses (in halfs): the lane's row n, channel 64 g; its
  // transposed-load row 4 g + c and channel 4 rq
  const uint32_t wr_base = (uint32_t)(n * PW_RP + 64 * g);
  const uint32_t tr_base = (uint32_t)((4 * g + (n >> 2)) * PW_RP + 4 * (n & 3));
  if (lane == 0) {
    sh.sflag[wave] = 0;
    sh.sack[wave] = 0;
  }
  __syncthreads();
  int useq = 0;  // units this wave has exchanged partial S for

  // The fetch context of a row: its ids, block-table row, window rows and
  // row scales, visible window range and entry bound; j_end: the end of its
  // units in this workgroup's range.
  struct PwRow {
    const int32_t *irow, *btab;
    const uint8_t *wcodes, *qrow;
    const float *wscale;
    int32_t wf, wl, elim, j_end;
  };
  auto row_ctx = [&](int32_t r) {
    PwRow c;
    const int bb = r / a.nq;
    c.j_end = (int32_t)(min(u_end, (int64_t)(r + 1) * U) - (int64_t)r * U);
    c.irow = a.idx + (int64_t)r * a.k;
    c.btab = a.c.block_table + (int64_t)bb * a.c.max_pages;
    c.wcodes = a.win_codes ? a.win_codes + (int64_t)bb * a.win_rows * CSA2_D : nullptr;
    c.wscale = a.win_row_scale ? a.win_row_scale + (int64_t)bb * a.win_rows : nullptr;
    window_range(a, r, bb, c.wf, c.wl);
    c.qrow = (const uint8_t *)(a.q + (int64_t)r * CSA2_H * CSA2_D);
    c.elim = min(a.c.n_entries[bb], a.c.max_pages << a.c.page_shift);
    return c;
  };
  int32_t row = first_row;
  int32_t j0 = (int32_t)(u_begin - (int64_t)row * U);
  PwRow cur = row_ctx(row);
  // The loads of the units of a row: unit j of the current row, or, for j
  // at or past its end, unit j - j_end of the next row when `cross` (the
  // next row's first units are fetched during this row's last ones, so that
  // its prologue does not wait for the id -> page -> row chain).
  PwRow nxt = cur;
  bool has_next = false, cross = false;
  // the next row in this workgroup's range, if any; its first three units
  // are entry tiles when kw >= 3 units (else they are fetched after the row)
  auto plan_next = [&]() {
    has_next = (int64_t)(row + 1) * U < u_end;
    cross = has_next && kw >= 3 * AS_UNIT;
    if (has_next) {
      const int bn = (row + 1) / a.nq, bc = row / a.nq;
      nxt.j_end = (int32_t)(min(u_end, (int64_t)(row + 2) * U) - (int64_t)(row + 1) * U);
      nxt.irow = a.idx + (int64_t)(row + 1) * a.k;
      nxt.btab = a.c.block_table + (int64_t)bn * a.c.max_pages;
      nxt.elim = bn == bc ? cur.elim : min(a.c.n_entries[bn], a.c.max_pages << a.c.page_shift);
    }
  };
  auto tinfo = [&](int32_t j, int t, bool &nx, int32_t &p) {
    nx = j >= cur.j_end;
    const int32_t jj = nx ? j - cur.j_end : j;
    p = jj * AS_UNIT + 32 * pair + 16 * t;  // first position of the tile in its row's set (uniform)
    const bool in = nx ? (cross && jj < nxt.j_end) : true;
    return in ? pw_tile_type(p, kw, span) : (int)PW_NONE;
  };
  auto fid = [&](int32_t j, int t) {
    bool nx;
    int32_t p;
    const int ty = tinfo(j, t, nx, p);
    return pw_fetch_id(a, nx ? nxt.irow : cur.irow, ty == PW_ENTRY, p + n);  // no entry: the row's first id
  };
  auto fpage = [&](int32_t j, int t, int32_t id) {
    bool nx;
    int32_t p;
    const int ty = tinfo(j, t, nx, p);
    return pw_fetch_page(a, nx ? nxt.btab : cur.btab, ty == PW_ENTRY, id);
  };
  // (the next row's tiles fetched here are all entries, so its window fields are not needed)
  auto frows = [&](int32_t j, int t, int32_t id, int32_t page, PwSlice &sl) {
    bool nx;
    int32_t p;
    const int ty = tinfo(j, t, nx, p);
    pw_fetch_rows(a, ty, p + n, cb, nx ? nxt.elim : cur.elim, id, page, kw, span, cbase, sbase, cur.wcodes,
                  cur.wscale, cur.wf, cur.wl, sl);
  };
  // the id, page and row loads of unit j0 into A, the ids of j0 + 1 into B
  auto prologue = [&](PwSet &A, PwSet &B) {
    int32_t id0[2], pg0[2];
    id0[0] = fid(j0, 0);
    id0[1] = fid(j0, 1);
    B.id[0] = fid(j0 + 1, 0);
    B.id[1] = fid(j0 + 1, 1);
    A.id[0] = fid(j0 + 2, 0);
    A.id[1] = fid(j0 + 2, 1);
    pg0[0] = fpage(j0, 0, id0[0]);
    pg0[1] = fpage(j0, 1, id0[1]);
    A.pg[0] = fpage(j0 + 1, 0, B.id[0]);
    A.pg[1] = fpage(j0 + 1, 1, B.id[1]);
    frows(j0, 0, id0[0], pg0[0], A.t[0]);
    frows(j0, 1, id0[1], pg0[1], A.t[1]);
  };
  PwSet A, B;
  float qv[16];
  pw_load_q16(a, row, qv);
  plan_next();
  prologue(A, B);
  for (;;) {
    // Q of the row (all eight waves convert, 32 threads per head): per-head
    // power-of-two normalisation, fp16 hi + lo halves
    {
      const int h = tid >> 5, part = tid & 31;
      float mx = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, fabsf(qv[i]));
      mx = row16_max(mx);  // then across the two rows of 16 lanes that hold the head
      const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmax_nc(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      int e = 0;
      if (mx > 0.f) frexpf(mx, &e);
      const float sc = ldexpf(1.f, -e);
#pragma unroll
      for (int i = 0; i < 16; i += 8) {
        v8h hv, lv;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float xq = qv[i + jj] * sc;
          const _Float16 hi = (_Float16)xq;
          hv[jj] = hi;
          lv[jj] = (_Float16)(xq - (float)hi);
        }
        *(v8h *)&sh.q.hi[h * PW_QP + part * 16 + i] = hv;
        *(v8h *)&sh.q.lo[h * PW_QP + part * 16 + i] = lv;
      }
      if (part == 0) sh.q.qexp[h] = (float)e;
    }
    __syncthreads();
    const float qs = ldexpf(a.sm_scale * 1.4426950408889634f, (int)sh.q.qexp[n]);
    // B operands of step ks: head n, channels cb + 8 ks + e
    v8h qh[8], ql[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qh[ks] = *(const v8h *)&sh.q.hi[n * PW_QP + cb + 8 * ks];
      ql[ks] = *(const v8h *)&sh.q.lo[n * PW_QP + cb + 8 * ks];
    }
    __syncthreads();  // the R tiles overwrite the staged Q
    float m_run = -INFINITY, l_run = 0.f;
    v4f o[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) o[q] = (v4f){0.f, 0.f, 0.f, 0.f};
    // Unit j with X = its set and Y = the set of unit j - 1, whose ids are
    // those of unit j + 1: the page words of j + 2, the ids of j + 3 and the
    // rows of j + 1 into Y, the window tails of unit j, then the compute.
    // Nothing loaded into Y is read before unit j + 1, and the two sets
    // alternate without copies, so the loads of j + 1 stay in flight while j
    // computes.
    auto unit = [&](int32_t j, PwSet &X, PwSet &Y) {
      const int32_t p0 = j * AS_UNIT + 32 * pair;  // first position of the pair's chunk
      // issue priority to the wave that lags the other wave on its SIMD (wave
      // ^ 4): by default the older wave wins every tie, so pairs 2 and 3 would
      // fall behind and pairs 0 and 1 wait for them at the row's end
      {
        const int sib = __hip_atomic_load(&sh.sflag[wave ^ 4], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (__builtin_amdgcn_readfirstlane(useq < sib ? 1 : 0)) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
      }
      const int ty0 = pw_tile_type(p0, kw, span), ty1 = pw_tile_type(p0 + 16, kw, span);
      const bool live = p0 < span;  // uniform per pair: the chunk holds some position of the row's set
      // page words and ids first: the rows of j + 1, issued at the start of
      // the next unit, then wait only for these, not for the rows of j + 1
      Y.pg[0] = fpage(j + 2, 0, X.id[0]);
      Y.pg[1] = fpage(j + 2, 1, X.id[1]);
      const int32_t idn0 = Y.id[0], idn1 = Y.id[1];  // ids of unit j + 1
      Y.id[0] = fid(j + 3, 0);
      Y.id[1] = fid(j + 3, 1);
      frows(j + 1, 0, idn0, X.pg[0], Y.t[0]);
      frows(j + 1, 1, idn1, X.pg[1], Y.t[1]);
      // the window tails of unit j, after the fixed set of loads above (their
      // wait, in window chunks only, then covers the next unit's loads too);
      // entry tiles load a fixed valid row instead, so that every path issues
      // the same loads and the waits for the rows of unit j stay exact
      v4i tail0[2], tail1[2];
      {
        bool ok;
        pw_window_tail(ty0 == PW_WINDOW, cur.wcodes, cur.qrow, pw_window_row(p0 + n, kw, span, cur.wf, cur.wl, ok), cb,
                       tail0);
        pw_window_tail(ty1 == PW_WINDOW, cur.wcodes, cur.qrow, pw_window_row(p0 + 16 + n, kw, span, cur.wf, cur.wl, ok),
                       cb, tail1);
      }
      v4f s0, s1;  // partial S of each tile over the wave's channels (hi and lo products)
      float rs[2][4];
      const bool has_rs = a.win_row_scale != nullptr;
      if (live) {
        if (ty0 == PW_WINDOW)
          pw_qk<PW_WINDOW>(X.t[0], tail0, qh, ql, rt + wr_base, has_rs, s0, rs[0]);
        else
          pw_qk<PW_ENTRY>(X.t[0], tail0, qh, ql, rt + wr_base, has_rs, s0, rs[0]);
        if (ty1 == PW_WINDOW)
          pw_qk<PW_WINDOW>(X.t[1], tail1, qh, ql, rt + wr_base + 16 * PW_RP, has_rs, s1, rs[1]);
        else
          pw_qk<PW_ENTRY>(X.t[1], tail1, qh, ql, rt + wr_base + 16 * PW_RP, has_rs, s1, rs[1]);
      } else {
        s0 = s1 = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) rs[0][i] = rs[1][i] = 1.f;
      }
      // the pair adds its two partial S (half 0 + half 1)
      // (only the two waves of the pair wait for each other: the other pairs
      // run on, which two workgroup barriers per unit did not allow)
      ++useq;
      pw_wait(&sh.sack[wave], useq - 1);  // the partner has read the previous unit's partial S
      sh.sx[wave][0][lane] = s0;
      sh.sx[wave][1][lane] = s1;
      pw_post(&sh.sflag[wave], useq);
      pw_wait(&sh.sflag[wave ^ 1], useq);
      const v4f p0r = sh.sx[wave ^ 1][0][lane], p1r = sh.sx[wave ^ 1][1][lane];
      pw_post(&sh.sack[wave ^ 1], useq);  // its slot may be written again
      if (live) {
        const v4f p0v = p0r, p1v = p1r;
        v4f Sf[2];
        Sf[0] = half ? p0v + s0 : s0 + p0v;
        Sf[1] = half ? p1v + s1 : s1 + p1v;
        if (ty0 == PW_WINDOW || ty1 == PW_WINDOW)
          pw_softmax_pv<true>(rt, Sf, X.t, rs, qs, tr_base, m_run, l_run, o);
        else
          pw_softmax_pv<false>(rt, Sf, X.t, rs, qs, tr_base, m_run, l_run, o);
      }
    };
    // the loads of unit j0 complete before the loop, so that the wait counts at
    // the loop head are those of the loop's own issue order on both entries
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    for (int32_t j = j0; j < cur.j_end; j += 2) {
      unit(j, A, B);
      if (j + 1 < cur.j_end) unit(j + 1, B, A);
    }
    if (has_next) pw_load_q16(a, row + 1, qv);  // in flight during the row's finish
    pw_finish(a, s, sh, wg, row, first_row, u_begin, u_end, m_run, l_run, o);
    if (!has_next) break;
    // the set of the next row's first unit is the one the last unit filled:
    // A after an even number of units, else B
    const bool odd = ((cur.j_end - j0) & 1) != 0, fetched = cross;
    ++row;
    j0 = 0;
    cur = row_ctx(row);
    plan_next();
    if (fetched) {
      if (odd) {
        const PwSet t = A;
        A = B;
        B = t;
      }
    } else {
      prologue(A, B);
    }
  }
}

hipError_t launch_attend_wave(const AttendArgs &a, const SegArgs &s, int max_slots, hipStream_t st) {
  if (s.G < 1 || s.G > kSegMaxWg || s.T < s.G || s.U < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_attend_wave, dim3((unsigned)s.G), dim3(PW_NT), 0, st, a, s);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge_seg(a, s, max_slots, st);
}

}  // namespace csa2
