// Group-wise asymmetric 4-bit round-to-nearest of W' = W diag(s), packed 8
// codes per int32 ("AWQ Math", sections "Weight-only quantization and where
// it breaks", "The equivalent transform" and "Shapes, granularity, and
// complexity"; "AWQ > Benefits and Practical Considerations": one scale and one
// zero point per 128 weights).
//
// One thread per packed word (8 consecutive weights of a row); the 16 threads
// of an aligned 16-lane segment hold one group of 128 and find its min / max
// with cross-lane shuffles.  Loads are 128-bit and coalesced along K, the word
// stores are 32-bit and coalesced, and the first lane of each segment writes
// the group's fp16 step and uint8 zero point.
#include "awq_device.h"
#include "awq_internal.h"

namespace awqk {

template <int DT, bool HAS_S>
__global__ __launch_bounds__(256) void k_quantize_pack(const uint16_t* __restrict__ w, int64_t N,
                                                       int64_t K, const float* __restrict__ s,
                                                       uint32_t* __restrict__ qw,
                                                       uint16_t* __restrict__ scales,
                                                       uint8_t* __restrict__ zeros,
                                                       float* __restrict__ dbg) {
  const int64_t wpr = K >> 3;                  // words per row
  const int64_t total = N * wpr;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool in = idx < total;                 // whole 16-lane segments are in or out
  const int64_t n = in ? idx / wpr : 0;
  const int64_t c = in ? idx - n * wpr : 0;
  const int64_t k0 = c * 8;

  float v[8];
  if (in) {
    const u32x4 raw = ldg128(w + n * K + k0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = lo_f32<DT>(raw[j]);
      v[2 * j + 1] = hi_f32<DT>(raw[j]);
    }
    if constexpr (HAS_S) {
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(s + k0);
      const f32x4 s1 = *reinterpret_cast<const f32x4*>(s + k0 + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] *= s0[j];
        v[4 + j] *= s1[j];
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = 0.0f;
  }

  float mn = v[0], mx = v[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) {
    mn = fminf(mn, v[j]);
    mx = fmaxf(mx, v[j]);
  }
  seg16_minmax(mn, mx);
  const GroupGrid g = group_grid(mn, mx);

  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) word |= (uint32_t)quant_code(v[j], g) << (4 * j);

  if (in) {
    qw[idx] = word;
    if ((threadIdx.x & 15) == 0) {
      const int64_t G = K / kGroup;
      const int64_t gi = n * G + k0 / kGroup;
      scales[gi] = (uint16_t)g.step_bits;
      zeros[gi] = (uint8_t)g.z;
      if (dbg) dbg[gi] = g.d;
    }
  }
}

}  // namespace awqk

namespace awq {

hipError_t launch_quantize_pack(const void* w, int dt, int64_t N, int64_t K, const float* s,
                                uint32_t* qw, uint16_t* scales, uint8_t* zeros, float* dbg,
                                hipStream_t st) {
  using namespace awqk;
  const int64_t total = N * (K / 8);
  const dim3 grid((unsigned)((total + 255) / 256));
  const uint16_t* wp = (const uint16_t*)w;
  if (dt == DT_F16) {
    if (s) hipLaunchKernelGGL((k_quantize_pack<DT_F16, true>), grid, dim3(256), 0, st, wp, N, K, s, qw, scales, zeros, dbg);
    else   hipLaunchKernelGGL((k_quantize_pack<DT_F16, false>), grid, dim3(256), 0, st, wp, N, K, s, qw, scales, zeros, dbg);
  } else {
    if (s) hipLaunchKernelGGL((k_quantize_pack<DT_BF16, true>), grid, dim3(256), 0, st, wp, N, K, s, qw, scales, zeros, dbg);
    else   hipLaunchKernelGGL((k_quantize_pack<DT_BF16, false>), grid, dim3(256), 0, st, wp, N, K, s, qw, scales, zeros, dbg);
  }
  return hipGetLastError();
}

}  // namespace awq
