// Group-wise round-to-nearest of W' = W diag(s) ("AWQ Math", sections
// "Weight-only quantization and where it breaks", "The equivalent transform"
// and "Shapes, granularity, and complexity"; "AWQ > Benefits and Practical
// Considerations": one scale and one zero point per group of 128 weights).
//
// k_quantize_pack: the asymmetric 4-bit grid, packed 8 codes per int32, with
// groups of 64, 128 or 256 input channels.  k_quantize_codes: any grid of the
// quantizer family (N bits, asymmetric or symmetric), one byte per code.
//
// One thread per 8 consecutive weights of a row; the GL = group / 8 threads of
// an aligned GL-lane segment hold one group and find its min / max with
// cross-lane shuffles.  Loads are 128-bit and coalesced along K, the code
// stores are coalesced, and the first lane of each segment writes the group's
// fp16 step and uint8 zero point.
#include "awq_device.h"
#include "awq_internal.h"

namespace awqk {

// The 8 weights of thread slot idx (row n, word c) times s, as float; the
// group's grid from the segment's min / max.
template <int DT, bool HAS_S, int GL, bool SYM>
__device__ __forceinline__ GroupGrid load_group8(const uint16_t* __restrict__ w, int64_t K,
                                                 const float* __restrict__ s, bool in, int64_t n,
                                                 int64_t k0, QSpec q, float (&v)[8]) {
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
  seg_minmax<GL>(mn, mx);
  return group_grid<SYM>(mn, mx, q);
}

template <int DT, bool HAS_S, int GL>
__global__ __launch_bounds__(256) void k_quantize_pack(const uint16_t* __restrict__ w, int64_t N,
                                                       int64_t K, const float* __restrict__ s,
                                                       uint32_t* __restrict__ qw,
                                                       uint16_t* __restrict__ scales,
                                                       uint8_t* __restrict__ zeros,
                                                       float* __restrict__ dbg) {
  const int64_t wpr = K >> 3;                  // words per row
  const int64_t total = N * wpr;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool in = idx < total;                 // whole GL-lane segments are in or out
  const int64_t n = in ? idx / wpr : 0;
  const int64_t c = in ? idx - n * wpr : 0;

  float v[8];
  const GroupGrid g = load_group8<DT, HAS_S, GL, false>(w, K, s, in, n, c * 8, kQ4, v);
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) word |= (uint32_t)quant_code(v[j], g) << (4 * j);

  if (in) {
    qw[idx] = word;
    if ((threadIdx.x & (GL - 1)) == 0) {
      const int64_t gi = idx / GL;             // = n * (K / group) + c / GL
      scales[gi] = (uint16_t)g.step_bits;
      zeros[gi] = (uint8_t)g.z;
      if (dbg) dbg[gi] = g.d;
    }
  }
}

template <int DT, bool HAS_S, int GL, bool SYM>
__global__ __launch_bounds__(256) void k_quantize_codes(const uint16_t* __restrict__ w, int64_t N,
                                                        int64_t K, const float* __restrict__ s,
                                                        QSpec q, uint8_t* __restrict__ codes,
                                                        uint16_t* __restrict__ scales,
                                                        uint8_t* __restrict__ zeros) {
  const int64_t wpr = K >> 3;
  const int64_t total = N * wpr;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool in = idx < total;
  const int64_t n = in ? idx / wpr : 0;
  const int64_t c = in ? idx - n * wpr : 0;

  float v[8];
  const GroupGrid g = load_group8<DT, HAS_S, GL, SYM>(w, K, s, in, n, c * 8, q, v);
  uint2 out = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out.x |= (uint32_t)quant_code(v[j], g) << (8 * j);
    out.y |= (uint32_t)quant_code(v[4 + j], g) << (8 * j);
  }
  if (in) {
    *reinterpret_cast<uint2*>(codes + idx * 8) = out;
    if ((threadIdx.x & (GL - 1)) == 0) {
      scales[idx / GL] = (uint16_t)g.step_bits;
      zeros[idx / GL] = (uint8_t)g.z;
    }
  }
}

template <int GL>
void quantize_pack_gl(const uint16_t* wp, int dt, int64_t N, int64_t K, const float* s, uint32_t* qw,
                      uint16_t* scales, uint8_t* zeros, float* dbg, dim3 grid, hipStream_t st) {
  if (dt == DT_F16) {
    if (s) hipLaunchKernelGGL((k_quantize_pack<DT_F16, true, GL>), grid, dim3(256), 0, st, wp, N, K, s, qw, scales, zeros, dbg);
    else   hipLaunchKernelGGL((k_quantize_pack<DT_F16, false, GL>), grid, dim3(256), 0, st, wp, N, K, s, qw, scales, zeros, dbg);
  } else {
    if (s) hipLaunchKernelGGL((k_quantize_pack<DT_BF16, true, GL>), grid, dim3(256), 0, st, wp, N, K, s, qw, scales, zeros, dbg);
    else   hipLaunchKernelGGL((k_quantize_pack<DT_BF16, false, GL>), grid, dim3(256), 0, st, wp, N, K, s, qw, scales, zeros, dbg);
  }
}

template <int GL, bool SYM>
void quantize_codes_gl(const uint16_t* wp, int dt, int64_t N, int64_t K, const float* s, QSpec q,
                       uint8_t* codes, uint16_t* scales, uint8_t* zeros, dim3 grid, hipStream_t st) {
  if (dt == DT_F16) {
    if (s) hipLaunchKernelGGL((k_quantize_codes<DT_F16, true, GL, SYM>), grid, dim3(256), 0, st, wp, N, K, s, q, codes, scales, zeros);
    else   hipLaunchKernelGGL((k_quantize_codes<DT_F16, false, GL, SYM>), grid, dim3(256), 0, st, wp, N, K, s, q, codes, scales, zeros);
  } else {
    if (s) hipLaunchKernelGGL((k_quantize_codes<DT_BF16, true, GL, SYM>), grid, dim3(256), 0, st, wp, N, K, s, q, codes, scales, zeros);
    else   hipLaunchKernelGGL((k_quantize_codes<DT_BF16, false, GL, SYM>), grid, dim3(256), 0, st, wp, N, K, s, q, codes, scales, zeros);
  }
}

template <int GL>
void quantize_codes_g(const uint16_t* wp, int dt, int64_t N, int64_t K, const float* s, QSpec q,
                      uint8_t* codes, uint16_t* scales, uint8_t* zeros, dim3 grid, hipStream_t st) {
  if (q.sym) quantize_codes_gl<GL, true>(wp, dt, N, K, s, q, codes, scales, zeros, grid, st);
  else quantize_codes_gl<GL, false>(wp, dt, N, K, s, q, codes, scales, zeros, grid, st);
}

}  // namespace awqk

namespace awq {

hipError_t launch_quantize_pack(const void* w, int dt, int64_t N, int64_t K, const float* s, int group,
                                uint32_t* qw, uint16_t* scales, uint8_t* zeros, float* dbg,
                                hipStream_t st) {
  using namespace awqk;
  const int64_t total = N * (K / 8);
  const dim3 grid((unsigned)((total + 255) / 256));
  const uint16_t* wp = (const uint16_t*)w;
  if (group == 64) quantize_pack_gl<8>(wp, dt, N, K, s, qw, scales, zeros, dbg, grid, st);
  else if (group == 128) quantize_pack_gl<16>(wp, dt, N, K, s, qw, scales, zeros, dbg, grid, st);
  else if (group == 256) quantize_pack_gl<32>(wp, dt, N, K, s, qw, scales, zeros, dbg, grid, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_quantize_codes(const void* w, int dt, int64_t N, int64_t K, const float* s,
                                 QuantVariant qv, uint8_t* codes, uint16_t* scales, uint8_t* zeros,
                                 hipStream_t st) {
  using namespace awqk;
  const int64_t total = N * (K / 8);
  const dim3 grid((unsigned)((total + 255) / 256));
  const uint16_t* wp = (const uint16_t*)w;
  const QSpec q = qspec(qv.bits, qv.sym);
  if (qv.group == 64) quantize_codes_g<8>(wp, dt, N, K, s, q, codes, scales, zeros, grid, st);
  else if (qv.group == 128) quantize_codes_g<16>(wp, dt, N, K, s, q, codes, scales, zeros, grid, st);
  else if (qv.group == 256) quantize_codes_g<32>(wp, dt, N, K, s, q, codes, scales, zeros, grid, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace awq
