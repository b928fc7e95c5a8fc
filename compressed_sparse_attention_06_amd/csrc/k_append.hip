// The write side of the cache, gfx950: quantising new compressed entries into
// FP4 (E2M1 values, one E4M3 scale per 16 channels) and new window tokens into
// E4M3 (DeepSeek V4.1 Flash summaries: "DeepSeek V4.1 Flash 如何靠压缩 KV 缓存
// 实现小模型干翻大模型", section "FP4 量化 + Bounded Replay": FP4 main KV and
// indexer Q/K with E4M3 scales per 16 channels and no second-level scale; the
// window keeps the last 128 tokens).
//
// Rounding (the pages give the formats only): nearest representable value,
// ties to the even mantissa, saturating at the largest finite value; the
// block scale is the E4M3 encoding of amax/6 (6 = the largest E2M1 magnitude)
// and each value is divided by the decoded scale in fp32; a window row with a
// row scale uses rs = amax/448. Encoding is integer arithmetic on the fp32
// bits, so it does not depend on the conversion instructions' modes.
#include "csa2_dev.h"
#include "kernels.h"

namespace csa2 {

// E4M3 byte of x: sign bit for x < 0, magnitude rounded to nearest even,
// saturating at 448 (0x7E).
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t sign = x < 0.f ? 0x80u : 0u;
  const float a = fabsf(x);
  uint32_t mag;
  if (!(a < 448.f)) {
    mag = 0x7Eu;
  } else if (a < 0.015625f) {
    // below the smallest normal 2^-6: multiples of 2^-9 (8 of them is 2^-6, byte 0x08)
    mag = (uint32_t)__builtin_rintf(a * 512.f);
  } else {
    const uint32_t u = __float_as_uint(a);
    const uint32_t m = u & 0x7FFFFFu;
    uint32_t q = ((((u >> 23) & 0xFFu) - 120u) << 3) | (m >> 20);  // biased exponent 127 -> 7
    const uint32_t rest = m & 0xFFFFFu;
    if (rest > 0x80000u || (rest == 0x80000u && (q & 1u))) q += 1u;  // carries into the exponent
    mag = min(q, 0x7Eu);
  }
  return sign | mag;
}

// E2M1 code of y (already divided by its block scale): the nearest of 0, 0.5,
// 1, 1.5, 2, 3, 4, 6, a midpoint going to the even code, saturating at 6;
// bit 3 is the sign of y.
__device__ __forceinline__ uint32_t e2m1_encode(float y) {
  const float a = fabsf(y);
  const uint32_t c = (a > 0.25f ? 1u : 0u) + (a >= 0.75f ? 1u : 0u) + (a > 1.25f ? 1u : 0u) +
                     (a >= 1.75f ? 1u : 0u) + (a > 2.5f ? 1u : 0u) + (a >= 3.5f ? 1u : 0u) +
                     (a > 5.0f ? 1u : 0u);
  return c | (y < 0.f ? 8u : 0u);
}

// One 16-channel group: 8 code bytes (channel 2j in the low nibble of byte j)
// and its scale byte.
__device__ __forceinline__ void quant_group(const float *x, uint8_t *codes, uint8_t *scale) {
  float v[16];
#pragma unroll
  for (int i = 0; i < 16; i += 4) {
    const v4f t = *(const v4f *)(x + i);
    v[i] = t[0];
    v[i + 1] = t[1];
    v[i + 2] = t[2];
    v[i + 3] = t[3];
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t sb = e4m3_encode(amax / 6.0f);
  const float s = e4m3_to_f32(sb);
  uint32_t w0 = 0, w1 = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t c = (s == 0.f) ? (v[i] < 0.f ? 8u : 0u) : e2m1_encode(v[i] / s);
    if (i < 8)
      w0 |= c << (4 * i);
    else
      w1 |= c << (4 * (i - 8));
  }
  *(uint2 *)codes = make_uint2(w0, w1);
  *scale = (uint8_t)sb;
}

__global__ void k_quant_fp4(const float *x, int64_t n_groups, int32_t groups_per_row, uint8_t *codes,
                            uint8_t *scales) {
  for (int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gi < n_groups;
       gi += (int64_t)gridDim.x * blockDim.x)
    quant_group(x + gi * 16, codes + gi * 8, scales + gi);
}

hipError_t launch_quant_fp4(const float *x, int64_t n_rows, int32_t channels, uint8_t *codes,
                            uint8_t *scales, hipStream_t st) {
  const int64_t n_groups = n_rows * (channels / 16);
  if (n_groups <= 0) return hipSuccess;
  int64_t blocks = (n_groups + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(k_quant_fp4, dim3((unsigned)blocks), dim3(256), 0, st, x, n_groups, channels / 16,
                     codes, scales);
  return hipGetLastError();
}

// One thread per 16-channel group of a new entry: groups 0..31 of the main-KV
// row, 32..35 of the indexer key.
__global__ void k_kv_append(AppendArgs a) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n_items = (int64_t)a.batch * a.n_new;
  const int gpe = a.ix ? 36 : 32;
  if (t >= n_items * gpe) return;
  const int64_t item = t / gpe;
  const int g = (int)(t % gpe);
  const int b = (int)(item / a.n_new);
  const int32_t s = a.entry[item];
  if (s < 0 || (s >> a.page_shift) >= a.max_pages) return;
  const int32_t page = a.block_table[(int64_t)b * a.max_pages + (s >> a.page_shift)];
  if (page < 0 || page >= a.num_pages) return;
  const int64_t row = ((int64_t)page << a.page_shift) + (s & ((1 << a.page_shift) - 1));
  if (g < 32)
    quant_group(a.kv + item * CSA2_D + 16 * g, a.kv_codes + row * (CSA2_D / 2) + 8 * g,
                a.kv_scales + row * (CSA2_D / 16) + g);
  else
    quant_group(a.ix + item * 64 + 16 * (g - 32), a.ix_codes + row * 32 + 8 * (g - 32),
                a.ix_scales + row * 4 + (g - 32));
}

hipError_t launch_kv_append(const AppendArgs &a, hipStream_t st) {
  const int64_t n = (int64_t)a.batch * a.n_new * (a.ix ? 36 : 32);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_kv_append, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

// One workgroup (128 threads, 4 channels each) per new window token.
__global__ __launch_bounds__(128) void k_window_append(uint8_t *codes, float *row_scale, int32_t rows,
                                                       const float *x, const int32_t *row, int32_t n_new) {
  __shared__ float smax[2];
  const int64_t item = blockIdx.x;
  const int b = (int)(item / n_new);
  const int32_t w = row[item];
  if (w < 0 || w >= rows) return;  // uniform
  const int t = threadIdx.x;
  const v4f v = *(const v4f *)(x + item * CSA2_D + 4 * t);
  float rs = 1.f;
  if (row_scale) {
    float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((t & 63) == 0) smax[t >> 6] = m;
    __syncthreads();
    const float amax = fmaxf(smax[0], smax[1]);
    rs = amax > 0.f ? amax / 448.f : 1.f;
    if (t == 0) row_scale[(int64_t)b * rows + w] = rs;
  }
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) word |= e4m3_encode(row_scale ? v[i] / rs : v[i]) << (8 * i);
  *(uint32_t *)(codes + ((int64_t)b * rows + w) * CSA2_D + 4 * t) = word;
}

hipError_t launch_window_append(uint8_t *codes, float *row_scale, int32_t rows, const float *x,
                                const int32_t *row, int32_t batch, int32_t n_new, hipStream_t st) {
  const int64_t n = (int64_t)batch * n_new;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_window_append, dim3((unsigned)n), dim3(128), 0, st, codes, row_scale, rows, x, row,
                     n_new);
  return hipGetLastError();
}

}  // namespace csa2
