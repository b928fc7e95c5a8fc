// Read-only streaming probe: the practical HBM read ceiling the decode
// kernels are measured against (their traffic is almost all reads). Not part
// of the method; measurement support only.
#include "csa2_dev.h"
#include "kernels.h"

namespace csa2 {

// Every lane streams 16-byte loads, eight in flight per iteration, over a
// grid-stride range and folds them with XOR; the result is stored only if it
// equals a value no input realistically produces, so the loads cannot be
// dropped and nothing is written in practice.
__global__ __launch_bounds__(256) void k_stream_read(const v4i *p, int64_t n16, uint32_t *sink) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  v4i acc = {0, 0, 0, 0};
  for (; i + 7 * stride < n16; i += 8 * stride) {
    v4i x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= x[u];
  }
  for (; i < n16; i += stride) acc ^= p[i];
  const uint32_t v = (uint32_t)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
  if (v == 0x9E3779B9u) sink[blockIdx.x & 1023] = v;
}

hipError_t launch_stream_read(const void *p, int64_t n_bytes, uint32_t *sink, int blocks, hipStream_t st) {
  if (n_bytes < 16 || blocks < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)blocks), dim3(256), 0, st, (const v4i *)p, n_bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace csa2
