// Sparse attention over the selected compressed entries plus the sliding
// window, gfx950 (DeepSeek V4.1 Flash summaries: "DeepSeek V4.1 Flash 如何靠压缩
// KV 缓存实现小模型干翻大模型", section "CSA2": every mode attends with its own
// global Q and its own SWA KV; all heads share one compressed latent, so the
// latent row is both key and value).
//
// One workgroup (4 waves) owns a (query row, split) pair: a contiguous slice of
// the attention set, processed in tiles of 32 rows.
//  * gather: each thread fetches 64 channels of one row (32 code bytes + 4
//    scale bytes for an FP4 entry, 64 bytes for an E4M3 window row) and
//    dequantises them exactly to fp16 into an LDS tile [32][512];
//  * S = Q R^T with v_mfma_f32_16x16x32_f16 (M = the 16 heads), the 512
//    channels split across the 4 waves and summed through LDS; after a
//    per-head power-of-two normalisation Q is carried as an fp16 hi + lo pair
//    (about 22 significant bits), since a single fp16 rounding of Q shifts
//    every logit of a head coherently;
//  * online softmax in fp32 (base-2 exponent) per head;
//  * O += P R, each wave owning 128 output channels; the R operand of this
//    product needs rows along K, which ds_read_b64_tr_b16 reads straight out
//    of the row-major LDS tile.
// The partial (unnormalised O, running max, running sum) of each split goes to
// the workspace; k_merge combines the splits.
#include "csa2_dev.h"
#include "kernels.h"

namespace csa2 {

#define AT_TILE 32
#define AT_PITCH 520  // halfs per LDS row (512 + 8) to spread banks

typedef __attribute__((address_space(3))) v4s *lds_v4s_ptr;

// Inputs of one row slice of one tile: an FP4 entry uses c[0..1] (32 code
// bytes) and sc (4 scale bytes), a window row uses c[0..3] (64 E4M3 bytes).
struct RowFetch {
  v4i c[4];
  uint32_t sc;
  float rs;
  int kind;  // 0 none, 1 entry, 2 window row
};

// Loads of one slice are issued unconditionally from clamped, in-range
// addresses (row 0 stands in for a missing row) and level by level (ids, then
// block-table words, then data), so that no branch or wait separates loads
// that could be in flight together; validity is applied afterwards.
__device__ __forceinline__ void fetch_entry(const AttendArgs &a, int32_t id, int32_t page, bool in_range,
                                            int32_t nent, int gpart, RowFetch &f) {
  const int sh = a.c.page_shift;
  const bool ok = in_range && id >= 0 && id < nent && (id >> sh) < a.c.max_pages && page >= 0 &&
                  page < a.c.num_pages;
  const int64_t crow = ok ? ((int64_t)page << sh) + (id & ((1 << sh) - 1)) : 0;
  f.c[0] = *(const v4i *)(a.c.kv_codes + crow * 256 + gpart * 32);
  f.c[1] = *(const v4i *)(a.c.kv_codes + crow * 256 + gpart * 32 + 16);
  f.sc = *(const uint32_t *)(a.c.kv_scales + crow * 32 + gpart * 4);
  f.rs = 1.f;
  f.kind = ok ? 1 : 0;
}

__device__ __forceinline__ void fetch_window(const AttendArgs &a, int b, int32_t j, bool ok, int gpart,
                                             RowFetch &f) {
  const int64_t wr = (int64_t)b * a.win_rows + (ok ? j : 0);
  const uint8_t *src = a.win_codes + wr * CSA2_D + gpart * 64;
#pragma unroll
  for (int i = 0; i < 4; ++i) f.c[i] = *(const v4i *)(src + 16 * i);
  f.sc = 0;
  f.rs = a.win_row_scale ? a.win_row_scale[wr] : 1.f;
  f.kind = ok ? 2 : 0;
}

template <int RPS>
__global__ __launch_bounds__(256) void k_attend(AttendArgs a) {
  constexpr int NT = RPS / AT_TILE;
  __shared__ __attribute__((aligned(16))) _Float16 sQ[CSA2_H * AT_PITCH];
  __shared__ __attribute__((aligned(16))) _Float16 sQlo[CSA2_H * AT_PITCH];
  __shared__ __attribute__((aligned(16))) _Float16 sR[AT_TILE * AT_PITCH];
  __shared__ float sS[4][CSA2_H][AT_TILE];
  __shared__ __attribute__((aligned(16))) _Float16 sP[CSA2_H * 40];
  __shared__ int sValid[AT_TILE];
  __shared__ float sRscale[AT_TILE];
  __shared__ float sM[CSA2_H], sL[CSA2_H], sAlpha[CSA2_H], sQexp[CSA2_H];

  const int r = blockIdx.y, split = blockIdx.x;
  const int b = r / a.nq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t total_pos = a.k + a.win_cap;
  const int32_t p0 = split * RPS;
  const int32_t p1 = min(p0 + RPS, total_pos);
  const int32_t nent = a.c.n_entries[b];

  // window geometry for this query
  int32_t w_first = 0, w_last = -1;
  if (a.win_codes) {
    const int32_t len = a.win_len[b];
    if (a.win_pos0) {
      const int32_t pq = a.q_pos ? a.q_pos[r] : 0x7FFFFFFF;
      const int64_t rel = (int64_t)pq - a.win_pos0[b];
      w_first = (int32_t)max((int64_t)0, rel - a.win_window + 1);
      w_last = (int32_t)min(min((int64_t)len, (int64_t)a.win_rows) - 1, rel);
    } else {
      w_first = 0;
      w_last = min(len, a.win_rows) - 1;
    }
  }

  // ---- issue every global load of this slice first ----
  // A split holds only selected entries, only window rows, or (when k is not
  // a multiple of the split length) both; the first two take the batched
  // path, the mixed split fetches each tile just before it is used.
  const int grow = tid >> 3, gpart = tid & 7;
  const int kind = (p1 <= a.k) ? 0 : (p0 >= a.k ? 1 : 2);  // uniform per workgroup
  RowFetch pf[NT];
  if (kind == 0) {
    int32_t idv[NT], pgv[NT];
    const int32_t nent_c = max(nent, 1);
#pragma unroll
    for (int ti = 0; ti < NT; ++ti) {
      const int32_t pos = min(p0 + ti * AT_TILE + grow, p1 - 1);
      idv[ti] = a.idx[(int64_t)r * a.k + pos];
    }
#pragma unroll
    for (int ti = 0; ti < NT; ++ti) {
      const int32_t pg = min(min(max(idv[ti], 0), nent_c - 1) >> a.c.page_shift, a.c.max_pages - 1);
      pgv[ti] = a.c.block_table[(int64_t)b * a.c.max_pages + pg];
    }
#pragma unroll
    for (int ti = 0; ti < NT; ++ti)
      fetch_entry(a, idv[ti], pgv[ti], p0 + ti * AT_TILE + grow < p1, nent, gpart, pf[ti]);
  } else if (kind == 1) {
#pragma unroll
    for (int ti = 0; ti < NT; ++ti) {
      const int32_t pos = p0 + ti * AT_TILE + grow;
      const int32_t j = w_first + (pos - a.k);
      fetch_window(a, b, j, pos < p1 && j <= w_last, gpart, pf[ti]);
    }
  }

  // ---- Q: per-head power-of-two normalisation, fp16 hi + lo, into LDS ----
  {
    const int h = tid >> 4, part = tid & 15;
    const float *qh = a.q + ((int64_t)r * CSA2_H + h) * CSA2_D + part * 32;
    float v[32];
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 32; i += 4) {
      const v4f x = *(const v4f *)(qh + i);
      v[i] = x[0]; v[i + 1] = x[1]; v[i + 2] = x[2]; v[i + 3] = x[3];
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) mx = fmaxf(mx, fabsf(v[i]));
    mx = fmaxf(mx, __shfl_xor(mx, 1));
    mx = fmaxf(mx, __shfl_xor(mx, 2));
    mx = fmaxf(mx, __shfl_xor(mx, 4));
    mx = fmaxf(mx, __shfl_xor(mx, 8));
    int e = 0;
    if (mx > 0.f) frexpf(mx, &e);  // mx = f * 2^e, f in [0.5, 1)
    const float sc = ldexpf(1.f, -e);
#pragma unroll
    for (int i = 0; i < 32; i += 8) {
      v8h hv, lv;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = v[i + j] * sc;
        const _Float16 hi = (_Float16)x;
        hv[j] = hi;
        lv[j] = (_Float16)(x - (float)hi);
      }
      *(v8h *)&sQ[h * AT_PITCH + part * 32 + i] = hv;
      *(v8h *)&sQlo[h * AT_PITCH + part * 32 + i] = lv;
    }
    if (part == 0) {
      sQexp[h] = (float)e;
      sM[h] = -INFINITY;
      sL[h] = 0.f;
    }
  }
  const float kLog2e = 1.4426950408889634f;
  const float zscale = a.sm_scale * kLog2e;

  v4f accO[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) accO[i] = (v4f){0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int ti = 0; ti < NT; ++ti) {
    if (p0 + ti * AT_TILE >= p1) break;  // uniform
    if (kind == 2) {
      const int32_t pos = p0 + ti * AT_TILE + grow;
      if (pos < a.k) {
        const int32_t id = a.idx[(int64_t)r * a.k + pos];
        const int32_t pg = min(min(max(id, 0), max(nent, 1) - 1) >> a.c.page_shift, a.c.max_pages - 1);
        const int32_t page = a.c.block_table[(int64_t)b * a.c.max_pages + pg];
        fetch_entry(a, id, page, true, nent, gpart, pf[ti]);
      } else {
        const int32_t j = w_first + (pos - a.k);
        fetch_window(a, b, j, pos < p1 && j <= w_last, gpart, pf[ti]);
      }
    }
    // ---- dequantise this thread's slice of the tile into sR ----
    {
      _Float16 *dst = &sR[grow * AT_PITCH + gpart * 64];
      if (pf[ti].kind == 1) {
        const uint32_t sw = pf[ti].sc;
        const uint32_t cw[8] = {(uint32_t)pf[ti].c[0][0], (uint32_t)pf[ti].c[0][1], (uint32_t)pf[ti].c[0][2],
                                (uint32_t)pf[ti].c[0][3], (uint32_t)pf[ti].c[1][0], (uint32_t)pf[ti].c[1][1],
                                (uint32_t)pf[ti].c[1][2], (uint32_t)pf[ti].c[1][3]};
#pragma unroll
        for (int gi = 0; gi < 4; ++gi) {
          const _Float16 sg = (_Float16)e4m3_to_f32((sw >> (8 * gi)) & 0xFFu);
          *(v8h *)(dst + gi * 16) = fp4x8_dequant(cw[2 * gi], sg);
          *(v8h *)(dst + gi * 16 + 8) = fp4x8_dequant(cw[2 * gi + 1], sg);
        }
      } else if (pf[ti].kind == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const v4i x = pf[ti].c[i];
          const v4h h0 = e4m3x4_to_f16((uint32_t)x[0]), h1 = e4m3x4_to_f16((uint32_t)x[1]);
          const v4h h2 = e4m3x4_to_f16((uint32_t)x[2]), h3 = e4m3x4_to_f16((uint32_t)x[3]);
          const v8h lo = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
          const v8h hi = {h2[0], h2[1], h2[2], h2[3], h3[0], h3[1], h3[2], h3[3]};
          *(v8h *)(dst + 16 * i) = lo;
          *(v8h *)(dst + 16 * i + 8) = hi;
        }
      } else {
        const v8h zero = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 8; ++i) *(v8h *)(dst + 8 * i) = zero;
      }
      if (gpart == 0) {
        sValid[grow] = pf[ti].kind != 0;
        sRscale[grow] = pf[ti].rs;
      }
    }
    __syncthreads();

    // ---- S = Q R^T (partial over this wave's 128 channels) ----
    {
      v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
      const int m = lane & 15, kq = lane >> 4;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int c0 = wave * 128 + ks * 32 + kq * 8;
        const v8h qa = *(const v8h *)&sQ[m * AT_PITCH + c0];
        const v8h ql = *(const v8h *)&sQlo[m * AT_PITCH + c0];
        const v8h r0 = *(const v8h *)&sR[m * AT_PITCH + c0];
        const v8h r1 = *(const v8h *)&sR[(16 + m) * AT_PITCH + c0];
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa, r0, s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa, r1, s1, 0, 0, 0);
        s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql, r0, s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(ql, r1, s1, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sS[wave][4 * kq + i][m] = s0[i];
        sS[wave][4 * kq + i][16 + m] = s1[i];
      }
    }
    __syncthreads();

    // ---- online softmax (base 2): thread -> (head, two rows) ----
    {
      const int h = tid >> 4, rr = (tid & 15) * 2;
      const float qs = ldexpf(zscale, (int)sQexp[h]);
      float z[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int row = rr + u;
        const float sv = sS[0][h][row] + sS[1][h][row] + sS[2][h][row] + sS[3][h][row];
        z[u] = sValid[row] ? sv * qs * sRscale[row] : -INFINITY;
      }
      float tmax = fmaxf(z[0], z[1]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 1));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 2));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 4));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 8));
      const float m_old = sM[h];
      const float m_new = fmaxf(m_old, tmax);
      float alpha = 1.f, p[2] = {0.f, 0.f};
      if (m_new != -INFINITY) {
        alpha = (m_old == -INFINITY) ? 0.f : exp2f(m_old - m_new);
#pragma unroll
        for (int u = 0; u < 2; ++u) p[u] = (z[u] == -INFINITY) ? 0.f : exp2f(z[u] - m_new);
      }
      float ps = p[0] + p[1];
      ps += __shfl_xor(ps, 1);
      ps += __shfl_xor(ps, 2);
      ps += __shfl_xor(ps, 4);
      ps += __shfl_xor(ps, 8);
#pragma unroll
      for (int u = 0; u < 2; ++u) sP[h * 40 + rr + u] = (_Float16)(p[u] * sRscale[rr + u]);
      __syncthreads();  // everyone has read sM before it changes
      if ((tid & 15) == 0) {
        sM[h] = m_new;
        sL[h] = sL[h] * alpha + ps;
        sAlpha[h] = alpha;
      }
    }
    __syncthreads();

    // ---- O = O * alpha + P R  (wave owns channels 128*wave .. +127) ----
    {
      const int g = lane >> 4, j = lane & 15, c = j >> 2, rq = j & 3;
      const v8h pa = *(const v8h *)&sP[(lane & 15) * 40 + 8 * g];
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = sAlpha[4 * g + i];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int n0 = wave * 128 + nt * 16;
        const _Float16 *base0 = &sR[(8 * g + c) * AT_PITCH + n0 + 4 * rq];
        const _Float16 *base1 = &sR[(8 * g + 4 + c) * AT_PITCH + n0 + 4 * rq];
        const v4s t0v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(base0));
        const v4s t1v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(base1));
        // whole-vector bit casts only: this clang mistranslates a bit cast of
        // a single vector element (it reads element 0)
        const v4h h0 = __builtin_bit_cast(v4h, t0v), h1 = __builtin_bit_cast(v4h, t1v);
        const v8h rb = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
        v4f o = accO[nt];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] *= al[i];
        accO[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, rb, o, 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- write this split's partial state ----
  float *part = a.part + ((int64_t)r * a.n_split + split) * CSA2_H * kPartStride;
  {
    const int g = lane >> 4, j = lane & 15;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const int ch = wave * 128 + nt * 16 + j;
#pragma unroll
      for (int i = 0; i < 4; ++i) part[(4 * g + i) * kPartStride + ch] = accO[nt][i];
    }
  }
  if (tid < CSA2_H) {
    part[tid * kPartStride + CSA2_D] = sM[tid];
    part[tid * kPartStride + CSA2_D + 1] = sL[tid];
  }
}

// Combine split partials of one (row, head): out = sum_s 2^(m_s - M) O_s /
// sum_s 2^(m_s - M) l_s, one thread per channel. Splits are read in batches
// of 16 so their loads are in flight together.
__global__ __launch_bounds__(512) void k_merge(MergeArgs a) {
  constexpr int BATCH = 16;
  const int h = blockIdx.x, r = blockIdx.y, c = threadIdx.x;
  const float *base = a.part + (int64_t)r * a.n_split * CSA2_H * kPartStride + (int64_t)h * kPartStride;
  const int64_t sstride = (int64_t)CSA2_H * kPartStride;
  const int last = a.n_split - 1;
  float M = -INFINITY;
  for (int s0 = 0; s0 < a.n_split; s0 += BATCH) {
    float mv[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) mv[u] = base[min(s0 + u, last) * sstride + CSA2_D];
#pragma unroll
    for (int u = 0; u < BATCH; ++u) M = fmaxf(M, mv[u]);  // repeats of the last split change nothing
  }
  float L = 0.f, o = 0.f;
  if (M != -INFINITY) {
    for (int s0 = 0; s0 < a.n_split; s0 += BATCH) {
      float mv[BATCH], lv[BATCH], ov[BATCH];
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const float *ps = base + min(s0 + u, last) * sstride;
        mv[u] = ps[CSA2_D];
        lv[u] = ps[CSA2_D + 1];
        ov[u] = ps[c];
      }
#pragma unroll
      for (int u = 0; u < BATCH; ++u) {
        const float wgt = (s0 + u < a.n_split && mv[u] != -INFINITY) ? exp2f(mv[u] - M) : 0.f;
        L += wgt * lv[u];
        o += wgt * ov[u];
      }
    }
  }
  a.out[((int64_t)r * CSA2_H + h) * CSA2_D + c] = (L > 0.f) ? o / L : 0.f;
  if (c == 0)
    a.lse[(int64_t)r * CSA2_H + h] = (L > 0.f) ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
}

hipError_t launch_attend(const AttendArgs &a, int rows, hipStream_t st) {
  dim3 grid((unsigned)a.n_split, (unsigned)rows);
  if (a.rows_per_split == 128)
    hipLaunchKernelGGL(k_attend<128>, grid, dim3(256), 0, st, a);
  else if (a.rows_per_split == 256)
    hipLaunchKernelGGL(k_attend<256>, grid, dim3(256), 0, st, a);
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
