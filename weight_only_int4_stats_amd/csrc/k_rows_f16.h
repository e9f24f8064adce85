// Rows of 16-bit activations -> fp16 with an exact power-of-two scale per row.
#pragma once

#include "awq_device.h"

namespace awqk {

// exact power of two p with max|v| * 2^p < 2^14 (0 when max is 0)
__device__ __forceinline__ int pow2_exp_for(float amax) {
  if (!(amax > 0.0f)) return 0;
  int e;
  frexpf(amax, &e);
  return 14 - e;
}

constexpr int kRowsKeep = 8;   // 8-element chunks per thread kept in registers (K <= 16384)

// Activation rows -> fp16: y_row = fp16(x_row * r * 2^p_row), p_row from the
// row's max so the row sits in fp16's normal range.  One block per row.  With
// PERMUTE each 8-element chunk is stored as (k0,k4,k2,k6,k1,k5,k3,k7), the
// order in which the packed-nibble unpack yields weight pairs; with UNIT_T
// (K a multiple of 128) the 16 pieces of each 128-channel unit are also
// transposed 4 x 4, piece 4 b + i stored at 4 i + b, so that the pieces a
// 16 x 16 x 32 product's four 32-channel lane blocks read together (one i,
// b = 0..3) are adjacent.  A row of up to
// 256 KEEP chunks stays in registers between its max and its conversion (read
// once); a longer one is read twice.
template <int DT, bool HAS_R, bool PERMUTE, int KEEP = kRowsKeep, bool UNIT_T = false>
__device__ __forceinline__ void rows_f16_block(int64_t row, const uint16_t* __restrict__ src, int64_t K,
                                               int64_t ld, const float* __restrict__ r,
                                               uint16_t* __restrict__ dst, int* __restrict__ pexp) {
  const uint16_t* s = src + row * ld;
  const int64_t nch = K >> 3;
  auto load8 = [&](int64_t c, float v[8]) {
    const u32x4 raw = ldg128(s + c * 8);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = lo_f32<DT>(raw[j]);
      v[2 * j + 1] = hi_f32<DT>(raw[j]);
    }
    if constexpr (HAS_R) {
      const f32x4 r0 = *reinterpret_cast<const f32x4*>(r + c * 8);
      const f32x4 r1 = *reinterpret_cast<const f32x4*>(r + c * 8 + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[j] *= r0[j];
        v[4 + j] *= r1[j];
      }
    }
  };
  uint16_t* d = dst + row * K;
  auto store8 = [&](int64_t c, const float v[8], int p) {
    uint32_t h[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) h[j] = f32_to_f16_bits(ldexpf(v[j], p));
    u32x4 o;
    if constexpr (PERMUTE) {
      o[0] = h[0] | (h[4] << 16);
      o[1] = h[2] | (h[6] << 16);
      o[2] = h[1] | (h[5] << 16);
      o[3] = h[3] | (h[7] << 16);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = h[2 * j] | (h[2 * j + 1] << 16);
    }
    const int64_t pos = UNIT_T ? ((c & ~(int64_t)15) | ((c & 3) << 2) | ((c >> 2) & 3)) : c;
    *reinterpret_cast<u32x4*>(d + pos * 8) = o;
  };
  __shared__ float wmax[4];
  auto row_exp = [&](float amax) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
    __syncthreads();
    const int p = pow2_exp_for(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3])));
    if (threadIdx.x == 0) pexp[row] = p;
    return p;
  };
  float amax = 0.0f;
  if (nch <= 256 * KEEP) {
    // the row stays in registers between the max and the conversion
    float v[KEEP][8];
#pragma unroll
    for (int i = 0; i < KEEP; ++i) {
      const int64_t c = threadIdx.x + 256 * i;
      if (c < nch) {
        load8(c, v[i]);
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[i][j]));
      }
    }
    const int p = row_exp(amax);
#pragma unroll
    for (int i = 0; i < KEEP; ++i) {
      const int64_t c = threadIdx.x + 256 * i;
      if (c < nch) store8(c, v[i], p);
    }
    return;
  }
  for (int64_t c = threadIdx.x; c < nch; c += 256) {
    float v[8];
    load8(c, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
  }
  const int p = row_exp(amax);
  for (int64_t c = threadIdx.x; c < nch; c += 256) {
    float v[8];
    load8(c, v);
    store8(c, v, p);
  }
}
template <int DT, bool HAS_R, bool PERMUTE, bool UNIT_T = false>
__global__ __launch_bounds__(256) void k_rows_f16(const uint16_t* __restrict__ src, int64_t K,
                                                  int64_t ld, const float* __restrict__ r,
                                                  uint16_t* __restrict__ dst,
                                                  int* __restrict__ pexp) {
  rows_f16_block<DT, HAS_R, PERMUTE, kRowsKeep, UNIT_T>(blockIdx.x, src, K, ld, r, dst, pexp);
}

}  // namespace awqk
