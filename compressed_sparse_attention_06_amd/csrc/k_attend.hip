// Sparse attention over the selected compressed entries plus the sliding
// window, gfx950 (DeepSeek V4.1 Flash summaries: "DeepSeek V4.1 Flash 如何靠压缩
// KV 缓存实现小模型干翻大模型", section "CSA2": every mode attends with its own
// global Q and its own SWA KV; all heads share one compressed latent, so the
// latent row is both key and value).
//
// One workgroup (4 waves) owns a (query row, split) pair: a contiguous slice of
// the attention set, processed in tiles of 64 rows, 16 per wave.
//  * each lane holds one quarter (128 channels) of one row of its wave's 16:
//    the FP4 codes (64 bytes + 8 scale bytes) of a selected entry, or the E4M3
//    bytes of a window row, all loaded before any compute;
//  * S = Q R^T with v_mfma_f32_16x16x32_f16 (M = the 16 heads, N = the wave's
//    16 rows, K = 512 channels in 16 steps). The channel order inside a step
//    is free as long as both operands share it: step ks, lane quarter kq and
//    element j stand for channel 128 kq + 8 ks + j, so each lane dequantises
//    its own B operand straight from registers (E2M1 x E4M3 and E4M3 are exact
//    in fp16). Q is carried as an fp16 hi + lo pair after a per-head
//    power-of-two normalisation (about 22 significant bits);
//  * the dequantised rows also go to an LDS tile [64][512] fp16 for O += P R,
//    where each wave owns 128 output channels and reads R with rows along K
//    through ds_read_b64_tr_b16;
//  * online softmax in fp32 (base-2) across tiles; three workgroup barriers
//    per tile.
// The partial (unnormalised O, running max, running sum) of each split goes to
// the workspace; k_merge combines the splits.
#include "csa2_dev.h"
#include "kernels.h"

namespace csa2 {

#define AT_ROWS 64     // rows per tile (4 waves x 16)
#define AT_PITCH 520   // halfs per LDS row of Q and of the R tile (512 + 8)
#define AT_PPITCH 72   // halfs per LDS row of P (64 + 8)

typedef __attribute__((address_space(3))) v4s *lds_v4s_ptr;

// One lane's quarter of one tile row. FP4 entry: c[0..3] hold the 64 code
// bytes, c[4].x and c[4].y the 8 group scales; window row: c[0..7] hold the
// 128 E4M3 bytes.
struct Slice {
  v4i c[8];
  float rs;   // window row scale (1 for entries)
  int kind;   // 0 no row, 1 entry, 2 window row
};

enum { SPLIT_ENTRIES = 0, SPLIT_WINDOW = 1, SPLIT_MIXED = 2 };

// Reductions over each row of 16 lanes with DPP moves (no LDS round trip):
// swap neighbours, swap pairs, mirror within 8 lanes, mirror within 16.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f32<0x140>(v));  // row_mirror
  return v;
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  return v;
}

// Loads are unconditional from clamped, in-range addresses (row 0 stands in
// for a missing row: its values are finite and get zero weight).
__device__ __forceinline__ void load_entry(const AttendArgs &a, int32_t id, int32_t page, bool in_range,
                                           int32_t nent, int kq, Slice &f) {
  const int sh = a.c.page_shift;
  const bool ok = in_range && id >= 0 && id < nent && (id >> sh) < a.c.max_pages && page >= 0 &&
                  page < a.c.num_pages;
  const int64_t crow = ok ? ((int64_t)page << sh) + (id & ((1 << sh) - 1)) : 0;
  const uint8_t *cp = a.c.kv_codes + crow * 256 + kq * 64;
#pragma unroll
  for (int i = 0; i < 4; ++i) f.c[i] = *(const v4i *)(cp + 16 * i);
  const v2f sc = *(const v2f *)(a.c.kv_scales + crow * 32 + kq * 8);
  f.c[4][0] = __float_as_int(sc[0]);
  f.c[4][1] = __float_as_int(sc[1]);
  f.rs = 1.f;
  f.kind = ok ? 1 : 0;
}

__device__ __forceinline__ void load_window(const AttendArgs &a, int b, int32_t j, bool ok, int kq, Slice &f) {
  const int64_t wr = (int64_t)b * a.win_rows + (ok ? j : 0);
  const uint8_t *src = a.win_codes + wr * CSA2_D + kq * 128;
#pragma unroll
  for (int i = 0; i < 8; ++i) f.c[i] = *(const v4i *)(src + 16 * i);
  f.rs = a.win_row_scale ? a.win_row_scale[wr] : 1.f;
  f.kind = ok ? 2 : 0;
}

// B operand of step ks: channels 128 kq + 8 ks + [0, 8) of the lane's row.
template <int KS>
__device__ __forceinline__ v8h entry_operand(const Slice &f) {
  const uint32_t word = (uint32_t)f.c[KS / 4][KS % 4];
  const uint32_t sw = (uint32_t)f.c[4][KS / 8];
  const _Float16 s = (_Float16)e4m3_to_f32((sw >> (8 * ((KS / 2) % 4))) & 0xFFu);
  return fp4x8_dequant(word, s);
}

template <int KS>
__device__ __forceinline__ v8h window_operand(const Slice &f) {
  const v4h h0 = e4m3x4_to_f16((uint32_t)f.c[(2 * KS) / 4][(2 * KS) % 4]);
  const v4h h1 = e4m3x4_to_f16((uint32_t)f.c[(2 * KS + 1) / 4][(2 * KS + 1) % 4]);
  const v8h r = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
  return r;
}

template <int KS, int KIND>
__device__ __forceinline__ v8h slice_operand(const Slice &f) {
  if constexpr (KIND == SPLIT_ENTRIES) return entry_operand<KS>(f);
  if constexpr (KIND == SPLIT_WINDOW) return window_operand<KS>(f);
  return (f.kind == 2) ? window_operand<KS>(f) : entry_operand<KS>(f);
}

// Q (hi, lo) is staged in LDS only until every lane holds its operands in
// registers; the R tile then reuses that space.
struct AttShared {
  union {
    struct {
      _Float16 q[CSA2_H * AT_PITCH];
      _Float16 qlo[CSA2_H * AT_PITCH];
    };
    _Float16 r[AT_ROWS * AT_PITCH];
  };
  _Float16 p[CSA2_H * AT_PPITCH];
  float wmax[4][CSA2_H], wsum[4][CSA2_H];
  float m[CSA2_H], l[CSA2_H], qexp[CSA2_H];
};

// Q of one query row: per-head power-of-two normalisation, fp16 hi + lo,
// staged in LDS and then held in registers as the A operands of every step
// (step ks: head n, channels 128 g + 8 ks + [0, 8)). qv: this thread's 32
// fp32 values (head tid / 16, channels 32 (tid % 16) + [0, 32)).
struct QOps {
  v8h qa[16], ql[16];
  float qs[4];  // logit scale (sm_scale * log2 e * 2^e) of heads 4g + i
};

__device__ __forceinline__ void prepare_q(const AttendArgs &a, AttShared &sh, const float *qv, QOps &q) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int n = lane & 15, g = lane >> 4;
  {
    const int h = tid >> 4, part = tid & 15;
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) mx = fmaxf(mx, fabsf(qv[i]));
    mx = row16_max(mx);  // the 16 threads of head h are one row of lanes
    int e = 0;
    if (mx > 0.f) frexpf(mx, &e);  // mx = f * 2^e, f in [0.5, 1)
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
    q.ql[ks] = *(const v8h *)&sh.qlo[n * AT_PITCH + g * 128 + 8 * ks];
  }
  __syncthreads();  // the R tile overwrites the staged Q
}

__device__ __forceinline__ void load_q(const AttendArgs &a, int r, float *qv) {
  const int tid = threadIdx.x;
  const float *src = a.q + ((int64_t)r * CSA2_H + (tid >> 4)) * CSA2_D + (tid & 15) * 32;
#pragma unroll
  for (int i = 0; i < 32; i += 4) {
    const v4f x = *(const v4f *)(src + i);
    qv[i] = x[0];
    qv[i + 1] = x[1];
    qv[i + 2] = x[2];
    qv[i + 3] = x[3];
  }
}

// One 64-row tile: S = Q R^T for the wave's 16 rows (the same operands fill
// the R tile), the online-softmax update, and O = O * alpha + P R with the
// wave owning output channels 128 wave .. +127.
template <int KIND>
__device__ __forceinline__ void attend_tile(AttShared &sh, const Slice &sl, const QOps &q, v4f *accO) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int trow = wave * 16 + n;
  v4f acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = (v4f){0.f, 0.f, 0.f, 0.f};
  _Float16 *rrow = &sh.r[trow * AT_PITCH + g * 128];
#define CSA2_QK_STEP(KS)                                                                              \
  {                                                                                                   \
    const v8h bop = slice_operand<KS, KIND>(sl);                                                      \
    *(v8h *)(rrow + 8 * (KS)) = bop;                                                                  \
    acc[(KS) & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(q.qa[KS], bop, acc[(KS) & 1], 0, 0, 0);     \
    acc[2 + ((KS) & 1)] = __builtin_amdgcn_mfma_f32_16x16x32_f16(q.ql[KS], bop, acc[2 + ((KS) & 1)], 0, 0, 0); \
  }
  CSA2_QK_STEP(0) CSA2_QK_STEP(1) CSA2_QK_STEP(2) CSA2_QK_STEP(3)
  CSA2_QK_STEP(4) CSA2_QK_STEP(5) CSA2_QK_STEP(6) CSA2_QK_STEP(7)
  CSA2_QK_STEP(8) CSA2_QK_STEP(9) CSA2_QK_STEP(10) CSA2_QK_STEP(11)
  CSA2_QK_STEP(12) CSA2_QK_STEP(13) CSA2_QK_STEP(14) CSA2_QK_STEP(15)
#undef CSA2_QK_STEP
  // lane holds S[head 4g + i][row n]
  const bool valid = sl.kind != 0;
  const float rs = sl.rs;
  float z[4], mx[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float sv = (acc[0][i] + acc[1][i]) + (acc[2][i] + acc[3][i]);
    z[i] = valid ? sv * q.qs[i] * rs : -INFINITY;
    mx[i] = row16_max(z[i]);  // over the wave's 16 rows
  }
  if (n == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sh.wmax[wave][4 * g + i] = mx[i];
  }
  __syncthreads();  // R tile and the waves' maxima are in LDS
  float alpha[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = 4 * g + i;
    const float m_old = sh.m[h];
    const float m_new =
        fmaxf(fmaxf(m_old, fmaxf(sh.wmax[0][h], sh.wmax[1][h])), fmaxf(sh.wmax[2][h], sh.wmax[3][h]));
    alpha[i] = (m_new == -INFINITY) ? 1.f : ((m_old == -INFINITY) ? 0.f : exp2f(m_old - m_new));
    const float pv = (z[i] == -INFINITY) ? 0.f : exp2f(z[i] - m_new);
    const float ps = row16_sum(pv);
    if (n == 0) sh.wsum[wave][h] = ps;
    sh.p[h * AT_PPITCH + trow] = (_Float16)(pv * rs);
  }
  __syncthreads();  // P and the row sums are in LDS; every read of m is done
  if (tid < CSA2_H) {
    const float m_old = sh.m[tid];
    const float m_new =
        fmaxf(fmaxf(m_old, fmaxf(sh.wmax[0][tid], sh.wmax[1][tid])), fmaxf(sh.wmax[2][tid], sh.wmax[3][tid]));
    const float al = (m_new == -INFINITY) ? 1.f : ((m_old == -INFINITY) ? 0.f : exp2f(m_old - m_new));
    sh.l[tid] = sh.l[tid] * al + ((sh.wsum[0][tid] + sh.wsum[1][tid]) + (sh.wsum[2][tid] + sh.wsum[3][tid]));
    sh.m[tid] = m_new;
  }
  {
    const int c = n >> 2, rq = n & 3;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) accO[nt][i] *= alpha[i];
    }
#pragma unroll
    for (int kstep = 0; kstep < 2; ++kstep) {
      const v8h pa = *(const v8h *)&sh.p[n * AT_PPITCH + 32 * kstep + 8 * g];
      v4s t0v[8], t1v[8];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int n0 = wave * 128 + nt * 16;
        const _Float16 *base0 = &sh.r[(32 * kstep + 8 * g + c) * AT_PITCH + n0 + 4 * rq];
        const _Float16 *base1 = &sh.r[(32 * kstep + 8 * g + 4 + c) * AT_PITCH + n0 + 4 * rq];
        t0v[nt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(base0));
        t1v[nt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(base1));
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        // whole-vector bit casts only: this clang mistranslates a bit cast of
        // a single vector element (it reads element 0)
        const v4h h0 = __builtin_bit_cast(v4h, t0v[nt]), h1 = __builtin_bit_cast(v4h, t1v[nt]);
        const v8h rb = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
        accO[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, rb, accO[nt], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // the R tile and P are free for the next tile
}

// Window geometry of query row r: rows w_first..w_last of its request's window.
__device__ __forceinline__ void window_range(const AttendArgs &a, int r, int b, int32_t &w_first,
                                             int32_t &w_last) {
  w_first = 0;
  w_last = -1;
  if (!a.win_codes) return;
  const int32_t len = a.win_len[b];
  if (a.win_pos0) {
    const int32_t pq = a.q_pos ? a.q_pos[r] : 0x7FFFFFFF;
    const int64_t rel = (int64_t)pq - a.win_pos0[b];
    w_first = (int32_t)max((int64_t)0, rel - a.win_window + 1);
    w_last = (int32_t)min(min((int64_t)len, (int64_t)a.win_rows) - 1, rel);
  } else {
    w_last = min(len, a.win_rows) - 1;
  }
}

template <int NT, int KIND>
__device__ __forceinline__ void attend_split(const AttendArgs &a, AttShared &sh, int r, int b, int split,
                                             int32_t p0, int32_t p1, int32_t nent, int32_t w_first,
                                             int32_t w_last) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;  // row of the wave's 16 / channel quarter; head group in C
  const int trow = wave * 16 + n;          // this lane's row inside a tile

  // ---- every global load of the split first: Q, then the rows level by level ----
  float qv[32];
  load_q(a, r, qv);
  Slice sl[NT];
  if constexpr (KIND == SPLIT_WINDOW) {
#pragma unroll
    for (int ti = 0; ti < NT; ++ti) {
      const int32_t pos = p0 + ti * AT_ROWS + trow;
      const int32_t j = w_first + (pos - a.k);
      load_window(a, b, j, pos < p1 && j <= w_last, g, sl[ti]);
    }
  } else {
    int32_t idv[NT], pgv[NT];
    const int32_t nent_c = max(nent, 1);
#pragma unroll
    for (int ti = 0; ti < NT; ++ti) {
      const int32_t pos = min(p0 + ti * AT_ROWS + trow, min(p1, a.k) - 1);
      idv[ti] = a.idx[(int64_t)r * a.k + pos];
    }
#pragma unroll
    for (int ti = 0; ti < NT; ++ti) {
      const int32_t pg = min(min(max(idv[ti], 0), nent_c - 1) >> a.c.page_shift, a.c.max_pages - 1);
      pgv[ti] = a.c.block_table[(int64_t)b * a.c.max_pages + pg];
    }
#pragma unroll
    for (int ti = 0; ti < NT; ++ti) {
      const int32_t pos = p0 + ti * AT_ROWS + trow;
      if constexpr (KIND == SPLIT_ENTRIES) {
        load_entry(a, idv[ti], pgv[ti], pos < p1, nent, g, sl[ti]);
      } else {
        // a lane reads an entry or a window row; both paths are issued
        Slice e, wr;
        load_entry(a, idv[ti], pgv[ti], pos < p1 && pos < a.k, nent, g, e);
        const int32_t j = w_first + (pos - a.k);
        load_window(a, b, j, pos < p1 && pos >= a.k && j <= w_last, g, wr);
        sl[ti] = (pos < a.k) ? e : wr;
      }
    }
  }
  QOps q;
  prepare_q(a, sh, qv, q);

  v4f accO[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) accO[i] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ti = 0; ti < NT; ++ti) {
    if (p0 + ti * AT_ROWS >= p1) break;  // uniform
    attend_tile<KIND>(sh, sl[ti], q, accO);
  }

  // ---- write this split's partial state ----
  float *part = a.part + ((int64_t)r * a.n_split + split) * CSA2_H * kPartStride;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const int ch = wave * 128 + nt * 16 + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) part[(4 * g + i) * kPartStride + ch] = accO[nt][i];
  }
  if (tid < CSA2_H) {
    part[tid * kPartStride + CSA2_D] = sh.m[tid];
    part[tid * kPartStride + CSA2_D + 1] = sh.l[tid];
  }
}

template <int NT>
__global__ __launch_bounds__(256) void k_attend(AttendArgs a) {
  __shared__ __attribute__((aligned(16))) AttShared sh;
  const int r = blockIdx.y, split = blockIdx.x;
  const int b = r / a.nq;
  const int32_t total_pos = a.k + a.win_cap;
  const int32_t p0 = split * (NT * AT_ROWS);
  const int32_t p1 = min(p0 + NT * AT_ROWS, total_pos);
  const int32_t nent = a.c.n_entries[b];
  int32_t w_first, w_last;
  window_range(a, r, b, w_first, w_last);
  // a split holds only selected entries, only window rows, or both
  if (p1 <= a.k)
    attend_split<NT, SPLIT_ENTRIES>(a, sh, r, b, split, p0, p1, nent, w_first, w_last);
  else if (p0 >= a.k)
    attend_split<NT, SPLIT_WINDOW>(a, sh, r, b, split, p0, p1, nent, w_first, w_last);
  else
    attend_split<NT, SPLIT_MIXED>(a, sh, r, b, split, p0, p1, nent, w_first, w_last);
}

// ---- one workgroup per query row, all tiles in turn ----------------------------------
// For calls with many query rows (a prefill chunk): no split partials and no
// merge; the row's tiles run in sequence, each tile's rows loaded while the
// previous tile computes (ids three tiles ahead, block-table words two
// ahead), and the workgroup writes out and lse itself.
struct TileFetch {
  int32_t id, page;
};

__device__ __forceinline__ int tile_kind(const AttendArgs &a, int t) {
  const int32_t t0 = t * AT_ROWS;
  return (t0 + AT_ROWS <= a.k) ? SPLIT_ENTRIES : (t0 >= a.k ? SPLIT_WINDOW : SPLIT_MIXED);
}

__device__ __forceinline__ int32_t fetch_id(const AttendArgs &a, int r, int t, int T, int trow) {
  if (t >= T || t * AT_ROWS >= a.k) return 0;  // uniform: no entries in this tile
  const int32_t pos = min(t * AT_ROWS + trow, a.k - 1);
  return a.idx[(int64_t)r * a.k + pos];
}

__device__ __forceinline__ int32_t fetch_page(const AttendArgs &a, int b, int32_t id, int32_t nent) {
  const int32_t pg = min(min(max(id, 0), max(nent, 1) - 1) >> a.c.page_shift, a.c.max_pages - 1);
  return a.c.block_table[(int64_t)b * a.c.max_pages + pg];
}

__device__ __forceinline__ void fetch_rows(const AttendArgs &a, int b, int t, int T, int trow, int g,
                                           const TileFetch &tf, int32_t nent, int32_t total_pos,
                                           int32_t w_first, int32_t w_last, Slice &sl) {
  if (t >= T) return;  // uniform
  const int32_t pos = t * AT_ROWS + trow;
  const int kind = tile_kind(a, t);
  if (kind == SPLIT_ENTRIES) {
    load_entry(a, tf.id, tf.page, pos < total_pos, nent, g, sl);
  } else if (kind == SPLIT_WINDOW) {
    const int32_t j = w_first + (pos - a.k);
    load_window(a, b, j, pos < total_pos && j <= w_last, g, sl);
  } else {
    Slice e, wr;
    load_entry(a, tf.id, tf.page, pos < a.k, nent, g, e);
    const int32_t j = w_first + (pos - a.k);
    load_window(a, b, j, pos < total_pos && pos >= a.k && j <= w_last, g, wr);
    sl = (pos < a.k) ? e : wr;
  }
}

__global__ __launch_bounds__(256) void k_attend_row(AttendArgs a, float *out, float *lse) {
  __shared__ __attribute__((aligned(16))) AttShared sh;
  const int r = blockIdx.x;
  const int b = r / a.nq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int trow = wave * 16 + n;
  const int32_t total_pos = a.k + a.win_cap;
  const int T = (total_pos + AT_ROWS - 1) / AT_ROWS;
  const int32_t nent = a.c.n_entries[b];
  int32_t w_first, w_last;
  window_range(a, r, b, w_first, w_last);

  float qv[32];
  load_q(a, r, qv);
  // ids three tiles ahead, block-table words two ahead, rows one ahead
  TileFetch f0, f1, f2;
  f0.id = fetch_id(a, r, 0, T, trow);
  f1.id = fetch_id(a, r, 1, T, trow);
  f2.id = fetch_id(a, r, 2, T, trow);
  f0.page = fetch_page(a, b, f0.id, nent);
  f1.page = fetch_page(a, b, f1.id, nent);
  Slice cur, nxt;
  cur.kind = 0;
  cur.rs = 1.f;
  fetch_rows(a, b, 0, T, trow, g, f0, nent, total_pos, w_first, w_last, cur);
  QOps q;
  prepare_q(a, sh, qv, q);

  v4f accO[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) accO[i] = (v4f){0.f, 0.f, 0.f, 0.f};
  for (int t = 0; t < T; ++t) {
    nxt.kind = 0;
    nxt.rs = 1.f;
    fetch_rows(a, b, t + 1, T, trow, g, f1, nent, total_pos, w_first, w_last, nxt);
    f2.page = fetch_page(a, b, f2.id, nent);
    const int32_t id3 = fetch_id(a, r, t + 3, T, trow);
    const int kind = tile_kind(a, t);  // uniform
    if (kind == SPLIT_ENTRIES)
      attend_tile<SPLIT_ENTRIES>(sh, cur, q, accO);
    else if (kind == SPLIT_WINDOW)
      attend_tile<SPLIT_WINDOW>(sh, cur, q, accO);
    else
      attend_tile<SPLIT_MIXED>(sh, cur, q, accO);
    cur = nxt;
    f1 = f2;
    f2.id = id3;
  }

  // ---- normalise and write the row's output ----
  float inv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float l = sh.l[4 * g + i];
    inv[i] = (l > 0.f) ? 1.f / l : 0.f;
  }
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    const int ch = wave * 128 + nt * 16 + n;
#pragma unroll
    for (int i = 0; i < 4; ++i) out[((int64_t)r * CSA2_H + 4 * g + i) * CSA2_D + ch] = accO[nt][i] * inv[i];
  }
  if (tid < CSA2_H) {
    const float l = sh.l[tid];
    lse[(int64_t)r * CSA2_H + tid] = (l > 0.f) ? (sh.m[tid] + log2f(l)) * 0.6931471805599453f : -INFINITY;
  }
}

// Combine split partials of one (row, head): out = sum_s 2^(m_s - M) O_s /
// sum_s 2^(m_s - M) l_s, one thread per channel. Splits are read 32 at a time
// (all loads in flight together) and folded into a running maximum.
__global__ __launch_bounds__(512) void k_merge(MergeArgs a) {
  constexpr int BATCH = 32;
  const int h = blockIdx.x, r = blockIdx.y, c = threadIdx.x;
  const float *base = a.part + (int64_t)r * a.n_split * CSA2_H * kPartStride + (int64_t)h * kPartStride;
  const int64_t sstride = (int64_t)CSA2_H * kPartStride;
  float M = -INFINITY, L = 0.f, o = 0.f;
  for (int s0 = 0; s0 < a.n_split; s0 += BATCH) {
    const int cnt = min(BATCH, a.n_split - s0);
    float mv[BATCH], lv[BATCH], ov[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const float *ps = base + (s0 + min(u, cnt - 1)) * sstride;
      mv[u] = ps[CSA2_D];
      lv[u] = ps[CSA2_D + 1];
      ov[u] = ps[c];
    }
    // repeats of the batch's last split weigh nothing: their max is -inf
#pragma unroll
    for (int u = 1; u < BATCH; ++u) mv[u] = (u < cnt) ? mv[u] : -INFINITY;
    float bm = M;
#pragma unroll
    for (int u = 0; u < BATCH; ++u) bm = fmaxf(bm, mv[u]);
    if (bm == -INFINITY) continue;
    const float f = exp2f(M - bm);  // 0 while M is -inf
    L *= f;
    o *= f;
#pragma unroll
    for (int u = 0; u < BATCH; ++u) {
      const float wgt = exp2f(mv[u] - bm);  // 0 for an empty split (m = -inf)
      L += wgt * lv[u];
      o += wgt * ov[u];
    }
    M = bm;
  }
  a.out[((int64_t)r * CSA2_H + h) * CSA2_D + c] = (L > 0.f) ? o / L : 0.f;
  if (c == 0)
    a.lse[(int64_t)r * CSA2_H + h] = (L > 0.f) ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
}

hipError_t launch_attend_rows(const AttendArgs &a, int rows, float *out, float *lse, hipStream_t st) {
  hipLaunchKernelGGL(k_attend_row, dim3((unsigned)rows), dim3(256), 0, st, a, out, lse);
  return hipGetLastError();
}

hipError_t launch_attend(const AttendArgs &a, int rows, hipStream_t st) {
  dim3 grid((unsigned)a.n_split, (unsigned)rows);
  if (a.rows_per_split == 64)
    hipLaunchKernelGGL(k_attend<1>, grid, dim3(256), 0, st, a);
  else if (a.rows_per_split == 128)
    hipLaunchKernelGGL(k_attend<2>, grid, dim3(256), 0, st, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs &a, int rows, hipStream_t st) {
  hipLaunchKernelGGL(k_merge, dim3(CSA2_H, (unsigned)rows), dim3(512), 0, st, a);
  return hipGetLastError();
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
