// Device helpers shared by the two attention kernels (k_attend.hip,
// k_attend_wave.hip): Q loading, window geometry, lane reductions and the
// R tile layout.
#pragma once

#include "csa2_dev.h"
#include "kernels.h"

namespace csa2 {

typedef __attribute__((address_space(3))) v4s *lds_v4s_ptr;

// DPP move within rows of 16 lanes (quad_perm / mirror controls only)
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Q of query row r: this thread's 32 fp32 values (head tid / 16, channels
// 32 (tid % 16) + [0, 32)).
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

#define AS_UNIT 128   // positions per unit of the attention work split
#define AS_RPITCH 512 // halfs per LDS row of the R tile (unpadded; 16-byte chunks are swizzled)

// R tile swizzle: in row r, the 16-byte chunk c of each 256-byte block is
// stored at chunk c ^ seg_rswz(r). Sixteen consecutive rows then fill every
// bank for the QK stores (same chunk, 16 rows) and eight rows x two chunks do
// the same for the PV transposed loads, with 32 or 64 banks.
__device__ __forceinline__ int seg_rswz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1) | (r & 8); }

// max of two non-NaN floats in one instruction: median of (a, b, +inf)
__device__ __forceinline__ float fmax_nc(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, INFINITY); }

// maximum over each row of 16 lanes: swap neighbours, swap pairs, mirror
// within 8 lanes, mirror within 16
__device__ __forceinline__ float row16_max(float v) {
  v = fmax_nc(v, dpp_f32<0xB1>(v));
  v = fmax_nc(v, dpp_f32<0x4E>(v));
  v = fmax_nc(v, dpp_f32<0x141>(v));
  v = fmax_nc(v, dpp_f32<0x140>(v));
  return v;
}

// Positions of a row's attention set: entries at [0, k), window rows from
// kw = k rounded up to 16, so that each wave's 16 positions are all entries
// (those at k and beyond hold nothing) or all window rows.
__device__ __forceinline__ int32_t seg_kw(int32_t k) { return (k + 15) & ~15; }

}  // namespace csa2
