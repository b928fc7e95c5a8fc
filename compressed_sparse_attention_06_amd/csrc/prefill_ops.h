// Helpers of the prefill kernels (gfx950 only).
#pragma once

#include "csa2_dev.h"

namespace csa2 {

// The E4M3 byte in bits 0..7 of `word` as fp16 (exact: every finite E4M3
// value is an fp16 value), in one conversion; the other bits of the word do
// not affect it.
__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, 1.0f, false)[0];
}

}  // namespace csa2
