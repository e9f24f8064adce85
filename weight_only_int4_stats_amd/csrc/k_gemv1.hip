// Batch-1 W4A16 GEMV ("AWQ > Benefits and Practical Considerations": the
// dequantization unpacks 4-bit integers, applies the group scale and zero
// point and optionally the per-channel inverse scale, fused with the multiply).
//
//   y[n] = sum_k step[n][g(k)] * (q[n][k] - z[n][g(k)]) * x[k] * r[k]
#include "awq_device.h"
#include "awq_internal.h"
#include "k_rows_f16.h"

namespace awqk {

constexpr uint32_t kMagic1024g1 = 0x64006400u;   // fp16 1024.0 in both halves

__device__ __forceinline__ float dot2h1(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

template <int YDT>
__device__ __forceinline__ void store_y1(void* y, int64_t idx, float v) {
  if constexpr (YDT == DT_F32) reinterpret_cast<float*>(y)[idx] = v;
  else reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)from_f32<YDT>(v);
}

// ---------------------------------------------------------------------------
// Batch-1 GEMV.  The block's waves are (K slice ks, row group rg): a lane owns
// one 128-bit chunk (32 codes) of K slice ks and walks the UL rows of its
// group.  The activation x * r is turned into fp16 once per block and staged
// in LDS (one thread per 8 consecutive k), so the 1/s and x reads are shared
// by every row of the block; those loads are issued before the weight loads
// (vector memory counters retire in order) so staging does not wait for the
// weights.  Each packed word is unpacked with one shift and four and-or
// operations: nibbles 0/4 and 2/6 become fp16 1024 + q, nibbles 1/5 and 3/7
// (still 4 bits up) become 1024 + 16 q; the factor 16 and the offsets are
// removed once per chunk with precomputed sums of the staged activations.
// Lanes reduce each row with a butterfly of shuffles; K slices combine
// through LDS in a fixed order.
// ---------------------------------------------------------------------------
constexpr int kG1Units = 4;          // rows per wave
constexpr int kG1MaxStage = 4;       // 8-element activation chunks staged per thread (K/8 <= 4 x threads)

template <int DT, int YDT, bool HAS_R>
__global__ __launch_bounds__(1024) void k_gemv1(
    const uint16_t* __restrict__ x, int64_t K, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int64_t N,
    const float* __restrict__ r, void* __restrict__ y, int nks) {
  constexpr int UL = kG1Units;
  extern __shared__ uint32_t lds1[];
  const int nwv = blockDim.x >> 6;
  const int nrg = nwv / nks;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int ks = wv % nks;
  const int rg = wv / nks;
  const int64_t CH = K >> 5;
  const int64_t ch = (int64_t)ks * 64 + lane;
  const bool valid = ch < CH;
  const int64_t chc = valid ? ch : 0;
  const int64_t G = K / kGroup;
  const int64_t gc = chc >> 2;
  const int64_t rowsb = (int64_t)nrg * UL;
  const int64_t row0 = (int64_t)blockIdx.x * rowsb + (int64_t)rg * UL;
  uint32_t* xpair = lds1;                                        // [CH][16] fp16 pairs
  float* xsum = reinterpret_cast<float*>(lds1 + CH * 16);        // [CH][4]: K0, S, 2^-p, -
  float* part = xsum + CH * 4;                                   // [nks][rowsb]

  // ---- 0. activation (and 1/s) loads for staging, issued first
  const int64_t n8 = K >> 3;
  const int64_t n8q = (n8 + 3) & ~int64_t(3);                    // whole quads of threads
  u32x4 sx[kG1MaxStage];
  f32x4 sr0[kG1MaxStage], sr1[kG1MaxStage];
#pragma unroll
  for (int i = 0; i < kG1MaxStage; ++i) {
    const int64_t c8 = threadIdx.x + (int64_t)i * blockDim.x;
    const int64_t c8c = c8 < n8 ? c8 : 0;
    if (c8 < n8q) {
      sx[i] = ldg128(x + c8c * 8);
      if constexpr (HAS_R) {
        sr0[i] = *reinterpret_cast<const f32x4*>(r + c8c * 8);
        sr1[i] = *reinterpret_cast<const f32x4*>(r + c8c * 8 + 4);
      }
    }
  }
  // ---- 1. weights, steps, zero points (branch-free: rows clamped, masked later)
  u32x4 wq[UL];
  uint32_t sraw[UL], zraw[UL];
#pragma unroll
  for (int u = 0; u < UL; ++u) {
    int64_t row = row0 + u;
    row = row < N ? row : N - 1;
    wq[u] = ldg128_stream(qw + row * (K >> 3) + chc * 4);
    sraw[u] = scales[row * G + gc];
    zraw[u] = zeros[row * G + gc];
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. stage fp16(x r 2^p) per 32-chunk (4 threads per chunk)
#pragma unroll
  for (int i = 0; i < kG1MaxStage; ++i) {
    const int64_t c8 = threadIdx.x + (int64_t)i * blockDim.x;
    if (c8 < n8q) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = lo_f32<DT>(sx[i][j]);
        v[2 * j + 1] = hi_f32<DT>(sx[i][j]);
      }
      if constexpr (HAS_R) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[j] *= sr0[i][j];
          v[4 + j] *= sr1[i][j];
        }
      }
      float amax = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
      amax = fmaxf(amax, __shfl_xor(amax, 1));
      amax = fmaxf(amax, __shfl_xor(amax, 2));
      int p = 0;
      if constexpr (DT == DT_BF16 || HAS_R) p = pow2_exp_for(amax);
      uint32_t h[8];
      float sa = 0.0f, sb = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        h[j] = (DT == DT_F16 && !HAS_R) ? (j & 1 ? sx[i][j >> 1] >> 16 : sx[i][j >> 1] & 0xFFFFu)
                                        : f32_to_f16_bits(ldexpf(v[j], p));
        if (j & 1) sb += f16_to_f32(h[j]);
        else sa += f16_to_f32(h[j]);
      }
      sa += __shfl_xor(sa, 1);
      sa += __shfl_xor(sa, 2);
      sb += __shfl_xor(sb, 1);
      sb += __shfl_xor(sb, 2);
      if (c8 < n8) {
        u32x4 o;
        o[0] = h[0] | (h[4] << 16);   // pairs with nibbles 0 / 4
        o[1] = h[2] | (h[6] << 16);   // nibbles 2 / 6 (word >> 8)
        o[2] = h[1] | (h[5] << 16);   // nibbles 1 / 5, held 16 q
        o[3] = h[3] | (h[7] << 16);   // nibbles 3 / 7, held 16 q
        *reinterpret_cast<u32x4*>(xpair + c8 * 4) = o;
        if ((c8 & 3) == 0) {
          f32x4 c;
          c[0] = 1024.0f * sa + 64.0f * sb;
          c[1] = sa + sb;
          c[2] = ldexpf(1.0f, -p);
          c[3] = 0.0f;
          *reinterpret_cast<f32x4*>(xsum + (c8 >> 2) * 4) = c;
        }
      }
    }
  }
  __syncthreads();
  u32x4 xr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xr[i] = *reinterpret_cast<const u32x4*>(xpair + chc * 16 + i * 4);
  const f32x4 xc = *reinterpret_cast<const f32x4*>(xsum + chc * 4);

  // ---- 3. dot products
  float val[UL];
#pragma unroll
  for (int u = 0; u < UL; ++u) {
    const bool rowok = valid && (row0 + u) < N;
    const float dz = rowok ? f16_to_f32(sraw[u]) * xc[2] : 0.0f;
    float Pa = 0.0f, Pb = 0.0f;
#pragma unroll
    for (int cw = 0; cw < 4; ++cw) {
      const uint32_t w = wq[u][cw];
      const uint32_t w8 = w >> 8;
      Pa = dot2h1((w & 0x000F000Fu) | kMagic1024g1, xr[cw][0], Pa);
      Pa = dot2h1((w8 & 0x000F000Fu) | kMagic1024g1, xr[cw][1], Pa);
      Pb = dot2h1((w & 0x00F000F0u) | kMagic1024g1, xr[cw][2], Pb);
      Pb = dot2h1((w8 & 0x00F000F0u) | kMagic1024g1, xr[cw][3], Pb);
    }
    const float P = __builtin_fmaf(Pb, 0.0625f, Pa) - __builtin_fmaf((float)zraw[u], xc[1], xc[0]);
    val[u] = dz * P;
  }
  // ---- 4. butterfly reduce-scatter over the wave (row index = top lane bits), then K slices
  constexpr int LB = 2;                          // log2(UL)
#pragma unroll
  for (int off = 32, n = UL; off >= 1; off >>= 1) {
    if (n > 1) {
      const bool upper = (lane & off) != 0;
#pragma unroll
      for (int i = 0; i < n / 2; ++i) {
        const float send = upper ? val[i] : val[i + n / 2];
        const float keep = upper ? val[i + n / 2] : val[i];
        val[i] = keep + __shfl_xor(send, off);
      }
      n >>= 1;
    } else {
      val[0] += __shfl_xor(val[0], off);
    }
  }
  if ((lane & ((64 >> LB) - 1)) == 0) part[ks * rowsb + rg * UL + (lane >> (6 - LB))] = val[0];
  __syncthreads();
  for (int t = threadIdx.x; t < rowsb; t += blockDim.x) {
    float tot = 0.0f;
    for (int k2 = 0; k2 < nks; ++k2) tot += part[k2 * rowsb + t];
    const int64_t row = (int64_t)blockIdx.x * rowsb + t;
    if (row < N) store_y1<YDT>(y, row, tot);
  }
}

template <int DT, int YDT, bool HAS_R>
hipError_t gemv1_dispatch(const uint16_t* x, int64_t K, const uint32_t* qw, const uint16_t* scales,
                          const uint8_t* zeros, int64_t N, const float* r, void* y, hipStream_t st) {
  const int64_t CH = K >> 5;
  const int nks = (int)((CH + 63) / 64);
  int nrg = nks >= 8 ? 1 : 8 / nks;
  if (nks * nrg > 16) nrg = 16 / nks;
  const int64_t rows = (int64_t)nrg * kG1Units;
  const int64_t threads = (int64_t)nks * nrg * 64;
  if (((K >> 3) + 3) / 4 * 4 > kG1MaxStage * threads) return hipErrorInvalidValue;
  const size_t lds = (size_t)CH * 16 * 4 + (size_t)CH * 4 * 4 + (size_t)nks * rows * 4;
  hipLaunchKernelGGL((k_gemv1<DT, YDT, HAS_R>), dim3((unsigned)((N + rows - 1) / rows)),
                     dim3((unsigned)(nks * nrg * 64)), lds, st, x, K, qw, scales, zeros, N, r, y, nks);
  return hipGetLastError();
}

}  // namespace awqk

namespace awq {

hipError_t launch_gemv1(const void* x, int xdt, int64_t K, const uint32_t* qw,
                        const uint16_t* scales, const uint8_t* zeros, int64_t N, const float* r,
                        void* y, int ydt, hipStream_t st) {
  using namespace awqk;
  const uint16_t* xp = (const uint16_t*)x;
#define AWQ_G1(DT, YDT)                                                                         \
  return r ? gemv1_dispatch<DT, YDT, true>(xp, K, qw, scales, zeros, N, r, y, st)               \
           : gemv1_dispatch<DT, YDT, false>(xp, K, qw, scales, zeros, N, r, y, st)
  if (xdt == DT_F16) {
    if (ydt == DT_F16) AWQ_G1(DT_F16, DT_F16);
    if (ydt == DT_BF16) AWQ_G1(DT_F16, DT_BF16);
    AWQ_G1(DT_F16, DT_F32);
  }
  if (ydt == DT_F16) AWQ_G1(DT_BF16, DT_F16);
  if (ydt == DT_BF16) AWQ_G1(DT_BF16, DT_BF16);
  AWQ_G1(DT_BF16, DT_F32);
#undef AWQ_G1
}

}  // namespace awq
