// The mixed-precision baseline that AWQ replaces ("AWQ vs. GPTQ:
// Understanding Weight Quantization Principles", sections on the central
// insight and on per-channel scaling): the salient weights are those of the
// input channels with the largest activation magnitudes, and keeping about 1 %
// of them in 16-bit greatly reduces the degradation, at the price of a
// mixed-precision layer.
//
// k_salient marks the n_keep channels with the largest mean |x| (ties: the
// lower index first) by an exact rank count,
//     rank_j = #{i : m_i > m_j} + #{i < j : m_i = m_j},  kept_j = rank_j < n_keep.
// A block of 16 waves takes 64 channels (one per lane); wave w counts over the
// w-th sixteenth of i, reading m_i with wave-uniform (scalar) loads, and the
// 16 partial counts are added in LDS.  O(K^2) comparisons, spread over K / 64
// blocks; it is not on the quantization path.
#include "awq_device.h"
#include "awq_internal.h"

namespace awqk {

constexpr int kSalWaves = 16;

__global__ __launch_bounds__(1024) void k_salient(const float* __restrict__ m, int64_t K,
                                                  int64_t n_keep, uint8_t* __restrict__ kept) {
  __shared__ int part[kSalWaves][64];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t j = (int64_t)blockIdx.x * 64 + lane;
  const float mj = j < K ? m[j] : 0.0f;
  const int64_t i0 = (int64_t)wv * K / kSalWaves, i1 = (int64_t)(wv + 1) * K / kSalWaves;
  int r = 0;
#pragma unroll 8
  for (int64_t i = i0; i < i1; ++i) {
    const float mi = m[i];                      // the same i in every lane
    r += (mi > mj) || (mi == mj && i < j);
  }
  part[wv][lane] = r;
  __syncthreads();
  if (wv == 0) {
    int64_t rank = 0;
#pragma unroll
    for (int w = 0; w < kSalWaves; ++w) rank += part[w][lane];
    if (j < K) kept[j] = rank < n_keep ? 1 : 0;
  }
}

}  // namespace awqk

namespace awq {

hipError_t launch_salient_channels(const float* mean_abs, int64_t K, int64_t n_keep, uint8_t* kept,
                                   hipStream_t st) {
  hipLaunchKernelGGL(awqk::k_salient, dim3((unsigned)((K + 63) / 64)), dim3(64 * awqk::kSalWaves), 0, st,
                     mean_abs, K, n_keep, kept);
  return hipGetLastError();
}

}  // namespace awq
