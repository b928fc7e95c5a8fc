// Device-side helpers shared by the CSA2 HIP kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa2.h"

#define CSA2_D 512
#define CSA2_H 16
#define CSA2_HI 4
#define CSA2_DI 64

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));

// ---- stores that write through the L2 -----------------------------------------
// A vector global store with the sc0 sc1 cache policy: the data goes on to
// memory at once instead of staying dirty in the writing XCD's L2, so the
// release at the end of the kernel, which writes dirty L2 lines back before
// the next kernel may start, has less to write. Used for the attention's split
// partials, which only the next kernel reads (measured: the 1M attention call
// 14.5 -> 14.1 us). The same policy on the scores and candidate lists of the
// selection kernels made the step slower, so they keep plain stores.
__device__ __forceinline__ void store_wt(float *p, v4f x) {
  asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1" ::"v"(p), "v"(x) : "memory");
}

// ---- sums across the four 16-lane rows of a wave ------------------------------
// t(l) + t(l ^ 16) + t(l ^ 32) + t(l ^ 48) in every lane l, with gfx950's row
// swaps (VALU moves, no LDS round trip): a 16-lane swap of a register with
// itself leaves rows {0, 1} and {2, 3} split between the two results, so their
// sum is the pair sum; the 32-lane swap does the same for the halves. The
// additions pair the same operands as t += t(l ^ 16); t += t(l ^ 32), so the
// result is bit for bit the same.
__device__ __forceinline__ float sum_rows4(float t) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
  const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---- order-preserving keys for fp32 scores ---------------------------------
// Larger score -> larger key. -0 is folded onto +0 so that equal values tie.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
#define KEY_NEG_INF 0x007FFFFFu  // score_key(-inf); every finite score is above it
#define HIST_BITS 12
#define HIST_BINS (1 << HIST_BITS)
#define HIST_SHIFT (32 - HIST_BITS)

// ---- format decode -----------------------------------------------------------
// OCP E4M3 bytes b0 (low) and b1 of a 16-bit field -> two fp32 values. The
// gfx950 conversion with scale 1.0 is exact for every byte (checked bit by bit
// against the byte table in the parity tests).
__device__ __forceinline__ v2f e4m3x2_lo_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(word, 1.0f, false);
}
__device__ __forceinline__ v2f e4m3x2_hi_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(word, 1.0f, true);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t byte) {
  return e4m3x2_lo_to_f32(byte & 0xFFu)[0];
}

// E2M1 codes of one byte of `word` (low nibble first) -> two fp16 values. The
// hardware scale operand applies only its power-of-two part, so the conversion
// runs at scale 1.0 and the E4M3 block scale is applied by an fp16 multiply:
// E2M1 x E4M3 needs at most 6 significant bits and lies in [2^-10, 2688], so
// the product is exact in fp16.
template <int SEL>
__device__ __forceinline__ v2h fp4x2_to_f16(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, SEL);
}

// 8 FP4 channels (one dword of codes) of one 16-channel group with scale s.
__device__ __forceinline__ v8h fp4x8_dequant(uint32_t word, _Float16 s) {
  const v2h ss = {s, s};
  const v2h a = fp4x2_to_f16<0>(word) * ss;
  const v2h b = fp4x2_to_f16<1>(word) * ss;
  const v2h c = fp4x2_to_f16<2>(word) * ss;
  const v2h d = fp4x2_to_f16<3>(word) * ss;
  v8h r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

// 4 E4M3 bytes -> 4 fp16 (exact: every finite E4M3 value is an fp16 value).
__device__ __forceinline__ v4h e4m3x4_to_f16(uint32_t word) {
  v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, false);
  v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, true);
  v4h r = {a[0], a[1], b[0], b[1]};
  return r;
}

// ---- XCD-aware workgroup order ----------------------------------------------------
// MI355X hands the workgroups of a 1-D grid to its 8 XCDs (each with its own
// L2) in turn: workgroup b runs on XCD b % 8. xcd_order(b, n) renumbers them
// so that XCD x runs one contiguous block of the logical order (from
// x * (n / 8) + min(x, n % 8), the first n % 8 XCDs taking one more): logical
// neighbours, which read the same data (one query row's Q, one row's
// partials), then share one L2 and fetch it from memory once. A bijection of
// [0, n).
__device__ __forceinline__ int xcd_order(int b, int n) {
  const int x = b & 7, s = b >> 3, q = n >> 3, r = n & 7;
  return x * q + min(x, r) + s;
}

// ---- paged cache addressing ----------------------------------------------------
struct DevCache {
  const uint8_t *kv_codes, *kv_scales, *ix_codes, *ix_scales;
  const int32_t *block_table, *n_entries;
  int32_t page_shift, max_pages, num_pages;
};

// Physical row of entry s of request b, or -1 when the entry does not exist.
__device__ __forceinline__ int64_t cache_row(const DevCache &c, int b, int32_t s, int32_t n_ent) {
  if (s < 0 || s >= n_ent) return -1;
  int32_t pg = s >> c.page_shift;
  if (pg >= c.max_pages) return -1;
  int32_t page = c.block_table[(int64_t)b * c.max_pages + pg];
  if (page < 0 || page >= c.num_pages) return -1;
  return ((int64_t)page << c.page_shift) + (s & ((1 << c.page_shift) - 1));
}

// Entries visible to query t of request b.
__device__ __forceinline__ int32_t visible_entries(const DevCache &c, const int32_t *q_pos, int b,
                                                   int nq, int t) {
  int32_t V = c.n_entries[b];
  if (q_pos) {
    int64_t vp = ((int64_t)q_pos[(int64_t)b * nq + t] + 1) / CSA2_TOKENS_PER_ENTRY;
    if (vp < V) V = (int32_t)(vp < 0 ? 0 : vp);
  }
  return V;
}

// ---- wave helpers ---------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Wave-aggregated append: returns this lane's slot (valid only where pred).
__device__ __forceinline__ int wave_append(bool pred, uint32_t *counter) {
  uint64_t mask = __ballot(pred);
  if (mask == 0) return -1;
  int leader = __ffsll((unsigned long long)mask) - 1;
  int cnt = __popcll(mask);
  uint32_t base = 0;
  if (lane_id() == leader) base = atomicAdd(counter, (uint32_t)cnt);
  base = __shfl(base, leader);
  uint32_t lo = (uint32_t)mask, hi = (uint32_t)(mask >> 32);
  int before = __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, 0));
  return (int)base + before;
}
