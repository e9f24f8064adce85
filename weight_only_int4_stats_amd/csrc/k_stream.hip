// Plain streaming read of a device buffer: the rate that the W4A16 products,
// bound by loading the packed weights ("AWQ Math", "Weight-only quantization
// and where it breaks": decode is limited by moving the weights), are measured
// against at their own sizes and launch shapes.  Each wave reads P whole 1 KB
// units per step (64 lanes x 16 B, non-temporal), striding over the buffer;
// each block writes the XOR of every 32-bit word it read, so the result is
// defined and the loads cannot be dropped.
#include "awq_device.h"
#include "awq_internal.h"

namespace awqk {

template <int P>
__global__ __launch_bounds__(1024) void k_read_stream(const uint8_t* __restrict__ p, int64_t units,
                                                      uint32_t* __restrict__ block_xor) {
  __shared__ uint32_t part[16];
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int64_t waves = (int64_t)gridDim.x * 16;
  const int64_t w = (int64_t)blockIdx.x * 16 + wv;
  uint32_t acc = 0u;
  for (int64_t u = w * P; u < units; u += waves * P) {
    u32x4 v[P];
    // a unit past the end re-reads unit u (in range) and is not counted
#pragma unroll
    for (int q = 0; q < P; ++q) v[q] = ldg128_stream(p + (u + q < units ? u + q : u) * 1024 + lane * 16);
#pragma unroll
    for (int q = 0; q < P; ++q)
      if (u + q < units) acc ^= v[q][0] ^ v[q][1] ^ v[q][2] ^ v[q][3];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
  if (lane == 0) part[wv] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) t ^= part[i];
    block_xor[blockIdx.x] = t;
  }
}

}  // namespace awqk

namespace awq {

hipError_t launch_read_stream(const void* p, int64_t bytes, int blocks, int unroll, uint32_t* block_xor,
                              hipStream_t st) {
  using namespace awqk;
  const int64_t units = bytes / 1024;
  const uint8_t* b = (const uint8_t*)p;
  const dim3 grid((unsigned)blocks), block(1024);
  if (unroll == 1) hipLaunchKernelGGL(k_read_stream<1>, grid, block, 0, st, b, units, block_xor);
  else if (unroll == 2) hipLaunchKernelGGL(k_read_stream<2>, grid, block, 0, st, b, units, block_xor);
  else if (unroll == 4) hipLaunchKernelGGL(k_read_stream<4>, grid, block, 0, st, b, units, block_xor);
  else hipLaunchKernelGGL(k_read_stream<8>, grid, block, 0, st, b, units, block_xor);
  return hipGetLastError();
}

}  // namespace awq
