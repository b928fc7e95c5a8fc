// Sparse attention over the selected compressed entries plus the sliding
// window, gfx950 (DeepSeek V4.1 Flash summaries: "DeepSeek V4.1 Flash 如何靠压缩
// KV 缓存实现小模型干翻大模型", section "CSA2": every mode attends with its own
// global Q and its own SWA KV; all heads share one compressed latent, so the
// latent row is both key and value).
//
// Layout of the work: see the segmented attention section below. Inside one
// unit of 128 positions, each of eight waves owns 16 rows:
//  * each lane holds one quarter (128 channels) of one row: the FP4 codes (64
//    bytes + 8 scale bytes) of a selected entry, or the E4M3 bytes of a window
//    row, loaded one unit ahead;
//  * S = Q R^T with v_mfma_f32_16x16x32_f16 (M = the 16 heads, N = the wave's
//    16 rows, K = 512 channels in 16 steps). The channel order inside a step
//    is free as long as both operands share it: step ks, lane quarter kq and
//    element j stand for channel 128 kq + 8 ks + j, so each lane dequantises
//    its own B operand straight from registers (E2M1 x E4M3 and E4M3 are exact
//    in fp16). Q is carried as an fp16 hi + lo pair after a per-head
//    power-of-two normalisation (about 22 significant bits); the hi halves
//    stay in registers, the lo halves are read from LDS at each step;
//  * the dequantised rows also go to an LDS tile [128][512] fp16 for
//    O += P R, where wave w owns output channels 64 w .. 64 w + 63 and reads R
//    with rows along K through ds_read_b64_tr_b16;
//  * online softmax in fp32 (base-2) across units; three workgroup barriers
//    per unit.
#include "csa2_dev.h"
#include "kernels.h"
#include "attend_common.h"

namespace csa2 {

#define AT_PITCH 520   // halfs per LDS row of the staged Q (512 + 8)

enum { SPLIT_ENTRIES = 0, SPLIT_WINDOW = 1 };

// ---- segmented attention: eight waves, 128 positions per step -----------------------
// The attention set of every query row (k selected entries, then from k
// rounded up to 16 up to win_cap window rows) is cut into units of 128 positions, and the units of all rows,
// row after row, are shared out evenly over G workgroups (G <= 256, one per
// compute unit: the 128-row R tile takes most of the LDS). A workgroup walks
// its units in order with one online-softmax state per row, loading the next
// unit's rows while it computes the current one (ids two units ahead,
// block-table words one ahead). Each of the eight waves takes 16 positions of a
// unit, so two waves share each SIMD and cover each other's latencies. A row
// whose units all fall to one workgroup is normalised and written there; a row
// cut between workgroups leaves one partial per workgroup (slot 0 for the
// workgroup's first row, slot 1 for its last), which k_merge_seg combines.
#define AS_PPITCH 136 // halfs per LDS row of P (128 + 8)
struct SegShared {
  union {
    _Float16 q[CSA2_H * AT_PITCH];  // hi halves of Q, staged once per row
    _Float16 r[AS_UNIT * AS_RPITCH];
  };
  _Float16 qlo[CSA2_H * AT_PITCH];  // lo halves of Q, read at every step
  _Float16 p[CSA2_H * AS_PPITCH];
  float wmax[CSA2_H][8], wsum[CSA2_H][8];  // [head][wave]
  float m[CSA2_H], l[CSA2_H], qexp[CSA2_H];
};

struct SegQ {
  v8h qa[16];
  float qs[4];  // logit scale (sm_scale * log2 e * 2^e) of heads 4g + i
};

// One lane's share of a unit row: the 64 code bytes and 8 scale bytes of a
// selected entry, or the first 64 E4M3 bytes of a window row (the other 64
// are loaded when the unit is computed, which keeps the prefetch buffer small).
struct SegSlice {
  v4i c[4];
  uint32_t s0, s1;
  float rs;     // window row scale (1 for entries)
  int32_t tag;  // entry id (checked against the request's entry count), or window row
  int kind;     // 0 no row, 1 entry, 2 window row
};

struct SegFetch {
  int32_t id, page;
};

// id of the lane's position in unit y (0 past the range or for window waves)
__device__ __forceinline__ int32_t seg_fetch_id(const AttendArgs &a, int64_t y, int64_t u_end, int32_t U,
                                                int prow) {
  if (y >= u_end) return 0;
  const int32_t r = (int32_t)(y / U), j = (int32_t)(y % U);
  if (j * AS_UNIT + (prow & ~15) >= seg_kw(a.k)) return 0;  // uniform per wave
  const int32_t pos = min(j * AS_UNIT + prow, a.k - 1);
  return a.idx[(int64_t)r * a.k + pos];
}

__device__ __forceinline__ int32_t seg_fetch_page(const AttendArgs &a, int64_t y, int64_t u_end, int32_t U,
                                                  int prow, int32_t id) {
  if (y >= u_end) return 0;
  const int32_t r = (int32_t)(y / U), j = (int32_t)(y % U);
  if (j * AS_UNIT + (prow & ~15) >= seg_kw(a.k)) return 0;
  const int b = r / a.nq;
  const int32_t pg = min(max(id, 0) >> a.c.page_shift, a.c.max_pages - 1);
  return a.c.block_table[(int64_t)b * a.c.max_pages + pg];
}

// The address depends only on the id and the page word (a position with no
// entry reads physical row 0, always in bounds). Its bytes must not reach the
// R tile: the scale words of such a position are zeroed, and since E2M1 has
// no NaN or infinity every code times a zero scale is 0. `use` is false for
// positions past k; ids at or past the request's entry count (`nent`, an
// unwritten slot) are not rows either.
__device__ __forceinline__ void seg_load_entry(const AttendArgs &a, int32_t id, int32_t page, int kq,
                                               int32_t nent, bool use, SegSlice &f) {
  const int sh = a.c.page_shift;
  const bool addr_ok = id >= 0 && (id >> sh) < a.c.max_pages && page >= 0 && page < a.c.num_pages;
  const int64_t crow = addr_ok ? ((int64_t)page << sh) + (id & ((1 << sh) - 1)) : 0;
  const uint8_t *cp = a.c.kv_codes + crow * 256 + kq * 64;
#pragma unroll
  for (int i = 0; i < 4; ++i) f.c[i] = *(const v4i *)(cp + 16 * i);
  const v2f sc = *(const v2f *)(a.c.kv_scales + crow * 32 + kq * 8);
  const bool ok = addr_ok && use && id < nent;
  f.s0 = ok ? (uint32_t)__float_as_int(sc[0]) : 0u;
  f.s1 = ok ? (uint32_t)__float_as_int(sc[1]) : 0u;
  f.rs = 1.f;
  f.tag = id;
  f.kind = ok ? 1 : 0;
}

// A window position with no visible row reads the request's row 0 (in
// bounds) and keeps zero codes and a unit row scale, so that a NaN byte or
// scale of an unwritten row never reaches the R tile or P.
__device__ __forceinline__ void seg_load_window(const AttendArgs &a, int b, int32_t j, bool ok, int kq,
                                                SegSlice &f) {
  const int32_t wr = b * a.win_rows + (ok ? j : 0);
  const uint8_t *src = a.win_codes + (int64_t)wr * CSA2_D + kq * 128;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v4i x = *(const v4i *)(src + 16 * i);
    f.c[i] = ok ? x : (v4i){0, 0, 0, 0};
  }
  f.s0 = f.s1 = 0u;
  const float rs = a.win_row_scale ? a.win_row_scale[wr] : 1.f;
  f.rs = ok ? rs : 1.f;
  f.tag = wr;
  f.kind = ok ? 2 : 0;
}

__device__ __forceinline__ void seg_fetch_rows(const AttendArgs &a, int64_t y, int64_t u_end, int32_t U,
                                               int prow, int kq, int32_t nent, const SegFetch &fe, SegSlice &s) {
  // a position with no row still feeds the R tile: zeros, never stale registers
#pragma unroll
  for (int i = 0; i < 4; ++i) s.c[i] = (v4i){0, 0, 0, 0};
  s.s0 = s.s1 = 0u;
  s.kind = 0;
  s.rs = 1.f;
  s.tag = 0;
  if (y >= u_end) return;
  const int32_t r = (int32_t)(y / U), j = (int32_t)(y % U);
  const int32_t pos = j * AS_UNIT + prow;
  const int32_t kw = seg_kw(a.k);
  if (j * AS_UNIT + (prow & ~15) < kw) {  // entry wave
    seg_load_entry(a, fe.id, fe.page, kq, nent, pos < a.k, s);
    return;
  }
  if (!a.win_codes) return;  // no window
  const int b = r / a.nq;
  int32_t wf, wl;
  window_range(a, r, b, wf, wl);
  const int32_t jw = wf + (pos - kw);
  seg_load_window(a, b, jw, pos < kw + a.win_cap && jw <= wl, kq, s);
}

// B operand of step KS from an entry: code word KS, scale of group KS / 2
// (the eight group scales of the lane's quarter, converted to fp16 in pairs)
template <int KS>
__device__ __forceinline__ v8h seg_entry_operand(const SegSlice &f, const v2h *sc) {
  return fp4x8_dequant((uint32_t)f.c[KS / 4][KS % 4], sc[KS / 4][(KS / 2) % 2]);
}

template <int KS>
__device__ __forceinline__ v8h seg_window_operand(const SegSlice &f, const v4i *h2) {
  uint32_t w0, w1;
  if constexpr (KS < 8) {
    w0 = (uint32_t)f.c[(2 * KS) / 4][(2 * KS) % 4];
    w1 = (uint32_t)f.c[(2 * KS + 1) / 4][(2 * KS + 1) % 4];
  } else {
    w0 = (uint32_t)h2[(2 * KS - 16) / 4][(2 * KS - 16) % 4];
    w1 = (uint32_t)h2[(2 * KS - 15) / 4][(2 * KS - 15) % 4];
  }
  const v4h h0 = e4m3x4_to_f16(w0), h1 = e4m3x4_to_f16(w1);
  const v8h r = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
  return r;
}

// S = Q R^T for the wave's 16 rows of the unit; the dequantised rows also go
// to the R tile. No barrier inside: entry or window is uniform per wave.
template <int KIND>
__device__ __forceinline__ void seg_qk(const AttendArgs &a, const SegShared &sh, const SegSlice &f, const SegQ &q,
                                       _Float16 *rtile, int prow, int n, int kq, v4f *acc) {
  v4i h2[4];
  if constexpr (KIND == SPLIT_WINDOW) {
    if (a.win_codes) {
      const bool ok = f.kind == 2;
      const int32_t wr = ok ? f.tag : 0;
      const uint8_t *src = a.win_codes + (int64_t)wr * CSA2_D + kq * 128 + 64;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const v4i x = *(const v4i *)(src + 16 * i);
        h2[i] = ok ? x : (v4i){0, 0, 0, 0};  // no bytes of a position without a row
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) h2[i] = (v4i){0, 0, 0, 0};
    }
  }
  // byte offset of the lane's chunk 0 in the R tile (row prow, block kq), swizzled
  const uint32_t rbase = (uint32_t)(prow * AS_RPITCH * 2 + kq * 256 + 16 * seg_rswz(prow));
  const _Float16 *qlo = &sh.qlo[n * AT_PITCH + kq * 128];
#define CSA2_QLO(KS) (*(const v8h *)(qlo + 8 * (KS)))
  v2h sc[4];
  if constexpr (KIND == SPLIT_ENTRIES) {
    sc[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.s0, 1.0f, false);
    sc[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.s0, 1.0f, true);
    sc[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.s1, 1.0f, false);
    sc[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(f.s1, 1.0f, true);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = (v4f){0.f, 0.f, 0.f, 0.f};
#define CSA2_SEG_STEP(KS)                                                                              \
  {                                                                                                    \
    v8h bop;                                                                                           \
    if constexpr (KIND == SPLIT_ENTRIES) bop = seg_entry_operand<KS>(f, sc);                           \
    else bop = seg_window_operand<KS>(f, h2);                                                          \
    *(v8h *)(rtile + ((rbase ^ (16 * (KS))) >> 1)) = bop;                                              \
    acc[(KS) & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(q.qa[KS], bop, acc[(KS) & 1], 0, 0, 0);      \
    acc[2 + ((KS) & 1)] = __builtin_amdgcn_mfma_f32_16x16x32_f16(CSA2_QLO(KS), bop, acc[2 + ((KS) & 1)], 0, 0, 0); \
  }
  CSA2_SEG_STEP(0) CSA2_SEG_STEP(1) CSA2_SEG_STEP(2) CSA2_SEG_STEP(3)
  CSA2_SEG_STEP(4) CSA2_SEG_STEP(5) CSA2_SEG_STEP(6) CSA2_SEG_STEP(7)
  CSA2_SEG_STEP(8) CSA2_SEG_STEP(9) CSA2_SEG_STEP(10) CSA2_SEG_STEP(11)
  CSA2_SEG_STEP(12) CSA2_SEG_STEP(13) CSA2_SEG_STEP(14) CSA2_SEG_STEP(15)
#undef CSA2_SEG_STEP
#undef CSA2_QLO
}

// Q of row r into the A operands (threads of waves 0-3 convert, all read).
__device__ __forceinline__ void seg_prepare_q(const AttendArgs &a, SegShared &sh, const float *qv, SegQ &q) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int n = lane & 15, g = lane >> 4;
  if (tid < 256) {  // waves 0-3
    const int h = tid >> 4, part = tid & 15;
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) mx = fmaxf(mx, fabsf(qv[i]));
    mx = row16_max(mx);
    int e = 0;
    if (mx > 0.f) frexpf(mx, &e);
    const float sc = ldexpf(1.f, -e);
#pragma unroll
    for (int i = 0; i < 32; i += 8) {
      v8h hv, lv;
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float x = qv[i + jj] * sc;
        const _Float16 hi = (_Float16)x;
        hv[jj] = hi;
        lv[jj] = (_Float16)(x - (float)hi);
      }
      *(v8h *)&sh.q[h * AT_PITCH + part * 32 + i] = hv;
      *(v8h *)&sh.qlo[h * AT_PITCH + part * 32 + i] = lv;
    }
    if (part == 0) {
      sh.qexp[h] = (float)e;
      sh.m[h] = -INFINITY;
      sh.l[h] = 0.f;
    }
  }
  __syncthreads();
  const float zscale = a.sm_scale * 1.4426950408889634f;
#pragma unroll
  for (int i = 0; i < 4; ++i) q.qs[i] = ldexpf(zscale, (int)sh.qexp[4 * g + i]);
#pragma unroll
  for (int ks = 0; ks < 16; ++ks) {
    q.qa[ks] = *(const v8h *)&sh.q[n * AT_PITCH + g * 128 + 8 * ks];
  }
  __syncthreads();  // the R tile overwrites the staged Q
}

__device__ __forceinline__ void seg_load_q(const AttendArgs &a, int r, float *qv) {
  const int tid = threadIdx.x;
  if (tid >= 256) return;  // uniform per wave
  load_q(a, r, qv);
}

// One unit: QK for the waves' 16 rows each, online softmax over the 128 rows,
// O = O * alpha + P R with wave w owning output channels 64 w .. 64 w + 63.
__device__ __forceinline__ void seg_unit(const AttendArgs &a, SegShared &sh, int32_t pos0, int32_t nent,
                                         const SegSlice &f, const SegQ &q, v4f *accO) {
  // lane indices and LDS addresses are recomputed per unit from an opaque copy
  // of the thread id instead of being kept live across the loop
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int prow = wave * 16 + n;
  v4f acc[4];
  if (pos0 + wave * 16 < seg_kw(a.k))  // uniform per wave
    seg_qk<SPLIT_ENTRIES>(a, sh, f, q, sh.r, prow, n, g, acc);
  else
    seg_qk<SPLIT_WINDOW>(a, sh, f, q, sh.r, prow, n, g, acc);
  // lane holds S[head 4g + i][row prow]
  const bool valid = (f.kind == 2) || (f.kind == 1 && f.tag < nent);
  const float rs = f.rs;
  float z[4], mx[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float sv = (acc[0][i] + acc[1][i]) + (acc[2][i] + acc[3][i]);
    z[i] = valid ? sv * q.qs[i] * rs : -INFINITY;
    mx[i] = z[i];
  }
  // maxima over the wave's 16 rows, the four heads' reductions interleaved
#pragma unroll
  for (int i = 0; i < 4; ++i) mx[i] = fmax_nc(mx[i], dpp_f32<0xB1>(mx[i]));
#pragma unroll
  for (int i = 0; i < 4; ++i) mx[i] = fmax_nc(mx[i], dpp_f32<0x4E>(mx[i]));
#pragma unroll
  for (int i = 0; i < 4; ++i) mx[i] = fmax_nc(mx[i], dpp_f32<0x141>(mx[i]));
#pragma unroll
  for (int i = 0; i < 4; ++i) mx[i] = fmax_nc(mx[i], dpp_f32<0x140>(mx[i]));
  if (n == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sh.wmax[4 * g + i][wave] = mx[i];
  }
  __syncthreads();  // R tile and the waves' maxima are in LDS
  // running maximum after this unit; a head with no finite logit yet keeps
  // reference 0 (its exponentials are all 0 and its state is empty)
  float alpha[4], mref[4], pv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * g + i;
    const v4f w0 = *(const v4f *)&sh.wmax[h][0], w1 = *(const v4f *)&sh.wmax[h][4];
    const float m_old = sh.m[h];
    const float m_new = fmax_nc(fmax_nc(fmax_nc(m_old, fmax_nc(w0[0], w0[1])), fmax_nc(fmax_nc(w0[2], w0[3]), fmax_nc(w1[0], w1[1]))),
                                fmax_nc(w1[2], w1[3]));
    mref[i] = (m_new == -INFINITY) ? 0.f : m_new;
    alpha[i] = __builtin_amdgcn_exp2f(m_old - mref[i]);  // 0 while m_old is -inf
    pv[i] = __builtin_amdgcn_exp2f(z[i] - mref[i]);      // 0 for an invalid row
  }
  float ps[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) ps[i] = pv[i] + dpp_f32<0xB1>(pv[i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) ps[i] += dpp_f32<0x4E>(ps[i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) ps[i] += dpp_f32<0x141>(ps[i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) ps[i] += dpp_f32<0x140>(ps[i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * g + i;
    if (n == 0) sh.wsum[h][wave] = ps[i];
    sh.p[h * AS_PPITCH + prow] = (_Float16)(pv[i] * rs);
  }
  __syncthreads();  // P and the row sums are in LDS; every read of m is done
  if (tid < CSA2_H) {
    const v4f w0 = *(const v4f *)&sh.wmax[tid][0], w1 = *(const v4f *)&sh.wmax[tid][4];
    const v4f s0 = *(const v4f *)&sh.wsum[tid][0], s1 = *(const v4f *)&sh.wsum[tid][4];
    const float m_old = sh.m[tid];
    const float m_new = fmax_nc(fmax_nc(fmax_nc(m_old, fmax_nc(w0[0], w0[1])), fmax_nc(fmax_nc(w0[2], w0[3]), fmax_nc(w1[0], w1[1]))),
                                fmax_nc(w1[2], w1[3]));
    const float mr = (m_new == -INFINITY) ? 0.f : m_new;
    const float sum = ((s0[0] + s0[1]) + (s0[2] + s0[3])) + ((s1[0] + s1[1]) + (s1[2] + s1[3]));
    sh.l[tid] = sh.l[tid] * __builtin_amdgcn_exp2f(m_old - mr) + sum;
    sh.m[tid] = m_new;
  }
  {
    const int c = n >> 2, rq = n & 3;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) accO[nt][i] *= alpha[i];
    }
    // lane reads channels n0 + 4 rq .. + 3 of rows 32 kstep + 8 g + c (+ 4):
    // chunk (8 wave + 2 nt + rq / 2) of the row, swizzled, half rq % 2
    const uint32_t cb = (uint32_t)((8 * wave) | (rq >> 1));
    const uint32_t a0 = (uint32_t)((8 * g + c) * AS_RPITCH * 2 + 8 * (rq & 1)) + 16 * (cb ^ seg_rswz(8 * g + c));
    const uint32_t a1 = (uint32_t)((8 * g + 4 + c) * AS_RPITCH * 2 + 8 * (rq & 1)) + 16 * (cb ^ seg_rswz(8 * g + 4 + c));
#pragma unroll
    for (int kstep = 0; kstep < 4; ++kstep) {
      const v8h pa = *(const v8h *)&sh.p[n * AS_PPITCH + 32 * kstep + 8 * g];
      v4s t0v[4], t1v[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const uint32_t o0 = (a0 ^ (32u * nt)) + 32u * AS_RPITCH * 2 * kstep;
        const uint32_t o1 = (a1 ^ (32u * nt)) + 32u * AS_RPITCH * 2 * kstep;
        t0v[nt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(sh.r + (o0 >> 1)));
        t1v[nt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(sh.r + (o1 >> 1)));
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const v4h h0 = __builtin_bit_cast(v4h, t0v[nt]), h1 = __builtin_bit_cast(v4h, t1v[nt]);
        const v8h rb = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
        accO[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, rb, accO[nt], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // the R tile and P are free for the next unit
}

// Row `row` is done in this workgroup: write it whole (normalised, with its
// lse), or leave its partial (unnormalised O, running max, running sum). The
// state goes through LDS (the R tile is free after the unit's last barrier) so
// that the stores are whole 16-byte vectors along each head's row.
__device__ __forceinline__ void seg_finish(const AttendArgs &a, const SegArgs &s, SegShared &sh, int w,
                                           int32_t row, int32_t first_row, int64_t u_begin, int64_t u_end,
                                           const v4f *accO) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  float *stage = (float *)sh.r;  // [16][kPartStride]
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int ch = wave * 64 + nt * 16 + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) stage[(4 * g + i) * kPartStride + ch] = accO[nt][i];
  }
  if (tid < CSA2_H) {
    stage[tid * kPartStride + CSA2_D] = sh.m[tid];
    stage[tid * kPartStride + CSA2_D + 1] = sh.l[tid];
  }
  __syncthreads();
  const int64_t r0 = (int64_t)row * s.U;
  if (r0 >= u_begin && r0 + s.U <= u_end) {
    // 16 x 512 outputs as 2048 float4, four per thread
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int v = tid + 512 * j, h = v >> 7, c = (v & 127) * 4;
      const float l = stage[h * kPartStride + CSA2_D + 1];
      const float inv = (l > 0.f) ? 1.f / l : 0.f;
      const v4f o = *(const v4f *)&stage[h * kPartStride + c];
      *(v4f *)&s.out[((int64_t)row * CSA2_H + h) * CSA2_D + c] = o * inv;
    }
    if (tid < CSA2_H) {
      const float l = stage[tid * kPartStride + CSA2_D + 1];
      s.lse[(int64_t)row * CSA2_H + tid] =
          (l > 0.f) ? (stage[tid * kPartStride + CSA2_D] + log2f(l)) * 0.6931471805599453f : -INFINITY;
    }
  } else {
    const int slot = (row == first_row) ? 0 : 1;
    float *part = a.part + ((int64_t)w * 2 + slot) * CSA2_H * kPartStride;
    // 16 x 516 floats as 2064 float4
    for (int v = tid; v < CSA2_H * kPartStride / 4; v += 512)
      store_wt(&part[4 * v], *(const v4f *)&stage[4 * v]);
  }
}

__global__ __launch_bounds__(512) void k_attend_seg(AttendArgs a, SegArgs s) {
  __shared__ __attribute__((aligned(16))) SegShared sh;
  const int w = s.xcd ? xcd_order(blockIdx.x, gridDim.x) : blockIdx.x;
  const int32_t U = s.U;
  const int64_t u_begin = (int64_t)w * s.T / s.G, u_end = (int64_t)(w + 1) * s.T / s.G;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, prow = wave * 16 + (lane & 15);
  const int32_t first_row = (int32_t)(u_begin / U);

  for (int64_t x = u_begin; x < u_end;) {
    // one row's units [x, xe): Q first, then the pipeline's prologue
    const int32_t row = (int32_t)(x / U);
    const int64_t xe = min(u_end, (int64_t)(row + 1) * U);
    // the first unit's rows are requested before Q is converted, so the id ->
    // page -> row chain and the conversion overlap
    SegQ q;
    SegFetch fc, fn;
    int32_t id2;
    SegSlice sc;
    const int32_t nent = a.c.n_entries[row / a.nq];
    {
      float qv[32];
      seg_load_q(a, row, qv);
      fc.id = seg_fetch_id(a, x, xe, U, prow);
      fn.id = seg_fetch_id(a, x + 1, xe, U, prow);
      id2 = seg_fetch_id(a, x + 2, xe, U, prow);
      fc.page = seg_fetch_page(a, x, xe, U, prow, fc.id);
      fn.page = seg_fetch_page(a, x + 1, xe, U, prow, fn.id);
      seg_fetch_rows(a, x, xe, U, prow, g, nent, fc, sc);
      seg_prepare_q(a, sh, qv, q);
    }
    // pipeline: rows of unit x in sc, id and page word of x + 1 in fn, id of x + 2 in id2
    v4f accO[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) accO[i] = (v4f){0.f, 0.f, 0.f, 0.f};
    for (; x < xe; ++x) {
      // rows of x + 1, page word of x + 2 and id of x + 3 load while unit x computes
      SegSlice sn;
      seg_fetch_rows(a, x + 1, xe, U, prow, g, nent, fn, sn);
      const int32_t pg2 = seg_fetch_page(a, x + 2, xe, U, prow, id2);
      const int32_t id3 = seg_fetch_id(a, x + 3, xe, U, prow);
      seg_unit(a, sh, (int32_t)(x % U) * AS_UNIT, nent, sc, q, accO);
      sc = sn;
      fn.id = id2;
      fn.page = pg2;
      id2 = id3;
    }
    seg_finish(a, s, sh, w, row, first_row, u_begin, u_end, accO);
    __syncthreads();  // m and l are read before the next row resets them
  }
}

// reductions over a wave: within rows of 16 lanes by DPP, then across the
// four rows through readlane (the result is uniform)
__device__ __forceinline__ float wave_max64(float v) {
  v = row16_max(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmax_nc(fmax_nc(r0, r1), fmax_nc(r2, r3));
}

__device__ __forceinline__ float wave_sum64(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Combine the partials of rows cut between workgroups of k_attend_seg (rows
// written whole are skipped). Workgroup w's partial for row r sits in slot 0
// when r is the first row of w's range, else in slot 1. One workgroup per
// (head, row), four channels per thread. The partials are taken BATCH at a
// time, and every load of a batch goes out before any is used: lane u of each
// wave reads the running max and sum of partial u (vector loads, so that the
// batch does not queue on scalar registers), each thread reads its four
// channels of every partial, and the weights reach the other lanes by
// readlane.
// (waves_per_eu: few merge waves share a SIMD, so the compiler may hold a
// whole batch in registers instead of recycling them between loads)
template <int BATCH>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(1, 2))) void k_merge_seg(MergeArgs a,
                                                                                              SegArgs s) {
  const int hr = s.xcd ? xcd_order(blockIdx.x, gridDim.x) : blockIdx.x;  // row-major (row, head)
  const int h = hr & (CSA2_H - 1), r = hr >> 4, t = threadIdx.x, lane = t & 63;
  const int64_t u0 = (int64_t)r * s.U, u1 = u0 + s.U - 1;
  const int32_t first = (int32_t)(((u0 + 1) * s.G + s.T - 1) / s.T - 1);
  const int32_t last = (int32_t)(((u1 + 1) * s.G + s.T - 1) / s.T - 1);
  if (first == last) return;  // written whole by its workgroup
  const int n = last - first + 1;
  // the first workgroup holds this row in slot 0 only when its range starts in it
  const int first_slot = ((int64_t)first * s.T / s.G / s.U == r) ? 0 : 1;
  // partial i of this row, head h: workgroup first + i, slot first_slot for i = 0, else 0
  const float *hb = a.part + (int64_t)h * kPartStride + 4 * t;
  float M = -INFINITY, L = 0.f;
  v4f o = {0.f, 0.f, 0.f, 0.f};
  for (int b0 = 0; b0 < n; b0 += BATCH) {
    const int cnt = min(BATCH, n - b0);
    float mu = -INFINITY, lu = 0.f;
    if (lane < cnt) {
      const int i = b0 + lane;
      const int slot = (i == 0) ? first_slot : 0;
      const float *ps = a.part + (((int64_t)(first + i) * 2 + slot) * CSA2_H + h) * kPartStride;
      mu = ps[CSA2_D];
      lu = ps[CSA2_D + 1];
    }
    v4f ov[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const int i = b0 + min(u, cnt - 1);  // repeats of the last partial weigh nothing
      const int slot = (i == 0) ? first_slot : 0;
      ov[u] = *(const v4f *)(hb + ((int64_t)(first + i) * 2 + slot) * CSA2_H * kPartStride);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load of the batch is issued before the first wait
    // no branch on the maxima, so that the loads above stay ahead of any use;
    // with nothing finite so far the reference is 0 and every weight is 0
    const float bm = fmaxf(M, wave_max64(mu));
    const float bref = (bm == -INFINITY) ? 0.f : bm;
    const float f = __builtin_amdgcn_exp2f(M - bref);  // 0 while M is -inf
    const float wu = __builtin_amdgcn_exp2f(mu - bref);  // 0 past the batch or for an empty partial
    L = L * f + wave_sum64(wu * lu);
    o *= f;
#pragma unroll
    for (int u = 0; u < BATCH; ++u)
      o += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wu), u)) * ov[u];
    M = bm;
  }
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  *(v4f *)&s.out[((int64_t)r * CSA2_H + h) * CSA2_D + 4 * t] = o * inv;
  if (t == 0)
    s.lse[(int64_t)r * CSA2_H + h] = (L > 0.f) ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
}

hipError_t launch_merge_seg(const AttendArgs &a, const SegArgs &s, int max_slots, hipStream_t st) {
  if (max_slots < 2) return hipSuccess;
  MergeArgs m{};
  m.part = a.part;
  const dim3 grid((unsigned)(CSA2_H * (s.T / s.U)));
  // one batch of loads covers up to 24 partials (the 1M decode rows have 17)
  if (max_slots <= 8)
    hipLaunchKernelGGL(k_merge_seg<8>, grid, dim3(128), 0, st, m, s);
  else if (max_slots <= 16)
    hipLaunchKernelGGL(k_merge_seg<16>, grid, dim3(128), 0, st, m, s);
  else
    hipLaunchKernelGGL(k_merge_seg<24>, grid, dim3(128), 0, st, m, s);
  return hipGetLastError();
}

hipError_t launch_attend_seg(const AttendArgs &a, const SegArgs &s, int max_slots, hipStream_t st) {
  if (s.G < 1 || s.G > kSegMaxWg || s.T < s.G || s.U < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_attend_seg, dim3((unsigned)s.G), dim3(512), 0, st, a, s);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_merge_seg(a, s, max_slots, st);
}

// ---- bit-exact dequantisation probes (same device helpers as above) ----
__global__ void k_dequant_fp4(const uint8_t *codes, const uint8_t *scales, int64_t n_groups,
                              uint16_t *out) {
  // one thread per 16-channel group
  for (int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gi < n_groups;
       gi += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t w0 = *(const uint32_t *)(codes + gi * 8);
    const uint32_t w1 = *(const uint32_t *)(codes + gi * 8 + 4);
    const _Float16 s = (_Float16)e4m3_to_f32(scales[gi]);
    v8h *o = (v8h *)(out + gi * 16);
    o[0] = fp4x8_dequant(w0, s);
    o[1] = fp4x8_dequant(w1, s);
  }
}

__global__ void k_dequant_e4m3(const uint8_t *bytes, int64_t n, float *out) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    out[i] = e4m3_to_f32(bytes[i]);
}

hipError_t launch_dequant_fp4(const uint8_t *codes, const uint8_t *scales, int64_t n_rows,
                              int32_t channels, uint16_t *out, hipStream_t st) {
  const int64_t n_groups = n_rows * (channels / 16);
  int64_t blocks = (n_groups + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL(k_dequant_fp4, dim3((unsigned)blocks), dim3(256), 0, st, codes, scales,
                     n_groups, out);
  return hipGetLastError();
}

hipError_t launch_dequant_e4m3(const uint8_t *bytes, int64_t n, float *out, hipStream_t st) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL(k_dequant_e4m3, dim3((unsigned)blocks), dim3(256), 0, st, bytes, n, out);
  return hipGetLastError();
}

}  // namespace csa2
