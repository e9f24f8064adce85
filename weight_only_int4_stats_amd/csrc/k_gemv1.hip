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
constexpr int kG1MaxStage = 4;       // 8-element activation chunks staged per thread (K/8 <= 4 x threads)

// Activation staging shared by the batch-1 kernels.  Thread t of the block
// handles the 8-element pieces t, t + blockDim, ... (NS of them): the loads are
// issued first (stage_load) and converted later (stage_store) into
//   xpair[c][16]: fp16(x r 2^p) of chunk c (32 elements) in unpack order,
//   xsum[c][4]:   (1024 (Sa + So), Sa + 16 So, 2^-p, 0),
// where even elements are stored as fp16(x r 2^p) and odd ones (which meet the
// nibbles held 16 q) as fp16(x r 2^(p - 4)), Sa / So are the sums of the stored
// even / odd values and p is the chunk's power of two (max |x r| 2^p < 2^14; 0
// for fp16 input without 1/s).
template <int DT, bool HAS_R, int NS>
__device__ __forceinline__ void stage_load(const uint16_t* __restrict__ x, const float* __restrict__ r,
                                           int64_t K, u32x4 (&sx)[NS], f32x4 (&sr0)[NS],
                                           f32x4 (&sr1)[NS]) {
  const int64_t n8 = K >> 3;
  const int64_t n8q = (n8 + 3) & ~int64_t(3);                    // whole quads of threads
#pragma unroll
  for (int i = 0; i < NS; ++i) {
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
}

template <int DT, bool HAS_R, int NS>
__device__ __forceinline__ void stage_store(int64_t K, const u32x4 (&sx)[NS], const f32x4 (&sr0)[NS],
                                            const f32x4 (&sr1)[NS], uint32_t* xpair, float* xsum) {
  const int64_t n8 = K >> 3;
  const int64_t n8q = (n8 + 3) & ~int64_t(3);
#pragma unroll
  for (int i = 0; i < NS; ++i) {
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
      amax = fmaxf(amax, quad_xor1(amax));
      amax = fmaxf(amax, quad_xor2(amax));
      int p = 0;
      if constexpr (DT == DT_BF16 || HAS_R) p = pow2_exp_for(amax);
      // even elements meet 1024 + q, odd ones 1024 + 16 q: the odd ones are
      // staged divided by 16 so one accumulator serves all four pairs
      uint32_t h[8];
      float sa = 0.0f, so = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j & 1) {
          h[j] = f32_to_f16_bits(ldexpf(v[j], p - 4));
          so += f16_to_f32(h[j]);
        } else {
          h[j] = (DT == DT_F16 && !HAS_R) ? (sx[i][j >> 1] & 0xFFFFu) : f32_to_f16_bits(ldexpf(v[j], p));
          sa += f16_to_f32(h[j]);
        }
      }
      sa += quad_xor1(sa);
      sa += quad_xor2(sa);
      so += quad_xor1(so);
      so += quad_xor2(so);
      if (c8 < n8) {
        u32x4 o;
        o[0] = h[0] | (h[4] << 16);   // pairs with nibbles 0 / 4
        o[1] = h[2] | (h[6] << 16);   // nibbles 2 / 6 (word >> 8)
        o[2] = h[1] | (h[5] << 16);   // nibbles 1 / 5, held 16 q
        o[3] = h[3] | (h[7] << 16);   // nibbles 3 / 7, held 16 q
        *reinterpret_cast<u32x4*>(xpair + c8 * 4) = o;
        if ((c8 & 3) == 0) {
          f32x4 c;
          c[0] = 1024.0f * (sa + so);   // the 1024 offsets of all 32 products
          c[1] = sa + 16.0f * so;       // sum of the effective activations
          c[2] = ldexpf(1.0f, -p);
          c[3] = 0.0f;
          *reinterpret_cast<f32x4*>(xsum + (c8 >> 2) * 4) = c;
        }
      }
    }
  }
}

// UL: rows per wave; NS: 8-element activation chunks staged per thread.
template <int DT, int YDT, bool HAS_R, int UL, int NS>
__global__ __launch_bounds__(1024) void k_gemv1_rows(
    const uint16_t* __restrict__ x, int64_t K, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int64_t N,
    const float* __restrict__ r, void* __restrict__ y, int nks, int gsh) {
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
  const int64_t G = K >> (gsh + 5);                              // groups per row
  const int64_t gc = chc >> gsh;                                 // this lane's group
  const int64_t rowsb = (int64_t)nrg * UL;
  const int64_t row0 = (int64_t)blockIdx.x * rowsb + (int64_t)rg * UL;
  uint32_t* xpair = lds1;                                        // [CH][16] fp16 pairs
  float* xsum = reinterpret_cast<float*>(lds1 + CH * 16);        // [CH][4]: K0, S, 2^-p, -
  float* part = xsum + CH * 4;                                   // [nks][rowsb]

  // ---- 0. activation (and 1/s) loads for staging, issued first
  u32x4 sx[NS];
  f32x4 sr0[NS], sr1[NS];
  stage_load<DT, HAS_R, NS>(x, r, K, sx, sr0, sr1);
  // ---- 1. weights, steps, zero points (branch-free: rows clamped, masked later)
  u32x4 wq[UL];
  uint32_t sraw[UL], zraw[UL];
  const uint32_t* qwl = qw + chc * 4;
  const uint16_t* scl = scales + gc;
  const uint8_t* zl = zeros + gc;
  const uint32_t KW = (uint32_t)(K >> 3), G32 = (uint32_t)G;
#pragma unroll
  for (int u = 0; u < UL; ++u) {
    const uint32_t row = (uint32_t)(row0 + u < N ? row0 + u : N - 1);
    wq[u] = ldg128_stream(qwl + (uint64_t)row * KW);
    sraw[u] = scl[(uint64_t)row * G32];
    zraw[u] = zl[(uint64_t)row * G32];
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. stage fp16(x r 2^p) per 32-chunk (4 threads per chunk)
  stage_store<DT, HAS_R, NS>(K, sx, sr0, sr1, xpair, xsum);
  __syncthreads();
  u32x4 xr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) xr[i] = *reinterpret_cast<const u32x4*>(xpair + chc * 16 + i * 4);
  const f32x4 xc = *reinterpret_cast<const f32x4*>(xsum + chc * 4);

  // ---- 3. dot products
  const uint32_t mlo = sgpr_const<0x000F000Fu>();
  const uint32_t mhi = sgpr_const<0x00F000F0u>();
  const uint32_t magic = vgpr_const<kMagic1024g1>();
  float val[UL];
#pragma unroll
  for (int u = 0; u < UL; ++u) {
    const bool rowok = valid && (row0 + u) < N;
    const float dz = rowok ? f16_to_f32(sraw[u]) * xc[2] : 0.0f;
    float P = 0.0f;
#pragma unroll
    for (int cw = 0; cw < 4; ++cw) {
      const uint32_t w = wq[u][cw];
      const uint32_t w8 = w >> 8;
      P = dot2h1((w & mlo) | magic, xr[cw][0], P);
      P = dot2h1((w8 & mlo) | magic, xr[cw][1], P);
      P = dot2h1((w & mhi) | magic, xr[cw][2], P);
      P = dot2h1((w8 & mhi) | magic, xr[cw][3], P);
    }
    P -= __builtin_fmaf((float)zraw[u], xc[1], xc[0]);
    val[u] = dz * P;
  }
  // ---- 4. reduce over the wave: rows split across lane halves, then 16-lane rows
  static_assert(UL == 1 || UL == 2 || UL == 4, "rows per wave");
  constexpr int LB = UL == 1 ? 0 : UL == 2 ? 1 : 2;   // log2(UL)
  float v;
  if constexpr (UL == 4) {
    const float a = pair_sum32(val[0], val[2]);      // lanes < 32: rows 0 / 1, upper: rows 2 / 3
    const float b = pair_sum32(val[1], val[3]);
    v = pair_sum16(a, b);                            // row index = lane >> 4
  } else if constexpr (UL == 2) {
    const float a = pair_sum32(val[0], val[1]);      // row index = lane >> 5
    v = pair_sum16(a, a);
  } else {
    const float a = pair_sum32(val[0], val[0]);
    v = pair_sum16(a, a);
  }
  v = row16_sum(v);
  val[0] = v;
  if ((lane & ((64 >> LB) - 1)) == 0) part[ks * rowsb + rg * UL + (lane >> (6 - LB))] = val[0];
  __syncthreads();
  for (int t = threadIdx.x; t < rowsb; t += blockDim.x) {
    float tot = 0.0f;
    for (int k2 = 0; k2 < nks; ++k2) tot += part[k2 * rowsb + t];
    const int64_t row = (int64_t)blockIdx.x * rowsb + t;
    if (row < N) store_y1<YDT>(y, row, tot);
  }
}

// ---------------------------------------------------------------------------
// Batch-1 GEMV, one block per compute unit.  Block b owns output rows
// [b N / B, (b + 1) N / B).  Its waves are (K slice ks, row group rg): a K
// slice is 128 chunks of 32 codes (4096 input channels), two chunks per lane
// (lane, lane + 64), and the wave's slice of the staged activation is held in
// registers for all of its rows.  Row group rg walks the block's rows
// rg, rg + nrg, ...; D rows of packed words, steps and zero points are kept in
// flight ahead of the row being reduced.  Each group of D row dot products is
// reduce-scattered across the wave; with one K slice the row sums are stored
// at once, otherwise the per-slice partial sums go to LDS and the slices are
// added in a fixed order at the end.
// ---------------------------------------------------------------------------
template <int DT, int YDT, bool HAS_R, int NS, int D, int C>
__global__ __launch_bounds__(1024) void k_gemv1_cu(
    const uint16_t* __restrict__ x, int64_t K, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int64_t N,
    const float* __restrict__ r, void* __restrict__ y, int nks, int nrg, int rows_max, int gsh) {
  static_assert(D >= 1 && D <= 4, "rows in flight");
  extern __shared__ uint32_t lds1[];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int ks = wv % nks;
  const int rg = wv / nks;
  const int64_t CH = K >> 5;
  const int64_t r0 = (int64_t)blockIdx.x * N / gridDim.x;
  const int nrows = (int)((int64_t)(blockIdx.x + 1) * N / gridDim.x - r0);
  const int nj = (rg < nrg && rg < nrows) ? (nrows - rg + nrg - 1) / nrg : 0;
  uint32_t* xpair = lds1;                                        // [CH][16]
  float* xsum = reinterpret_cast<float*>(lds1 + CH * 16);        // [CH][4]
  float* part = xsum + CH * 4;                                   // [nks][rows_max]

  int64_t chc[C];
  bool okc[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int64_t ch = (int64_t)ks * (64 * C) + c * 64 + lane;
    okc[c] = ch < CH;
    chc[c] = okc[c] ? ch : 0;
  }
  // ---- 0. staging loads, then the first D rows
  u32x4 sx[NS];
  f32x4 sr0[NS], sr1[NS];
  stage_load<DT, HAS_R, NS>(x, r, K, sx, sr0, sr1);

  // Buffer resources over this block's rows: an offset past the end reads 0
  // without touching memory, which masks missing rows and chunks.
  const uint32_t KW = (uint32_t)(K >> 3), G32 = (uint32_t)(K >> (gsh + 5));
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(qw + r0 * KW), (short)0, nrows * (int)KW * 4, kBufferWord3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(scales + r0 * G32), (short)0, nrows * (int)G32 * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(zeros + r0 * G32), (short)0, nrows * (int)G32, kBufferWord3);
  u32x4 wb[D][C];
  uint32_t sb[D][C], zb[D][C];
  auto load_row = [&](int slot, int j) {
    const bool rowok = j < nj;
    const uint32_t rl = (uint32_t)(rg + nrg * j);          // row within the block
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const bool ok = rowok && okc[c];
      const uint32_t g = (uint32_t)(chc[c] >> gsh);
      wb[slot][c] = __builtin_amdgcn_raw_buffer_load_b128(
          wrs, ok ? (rl * KW + (uint32_t)chc[c] * 4) * 4 : kBufferOob, 0, kBufferNt);
      sb[slot][c] = __builtin_amdgcn_raw_buffer_load_b16(srs, ok ? (rl * G32 + g) * 2 : kBufferOob, 0, 0);
      zb[slot][c] = __builtin_amdgcn_raw_buffer_load_b8(zrs, ok ? rl * G32 + g : kBufferOob, 0, 0);
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) load_row(d, d);
  __builtin_amdgcn_sched_barrier(0);

  // ---- 1. stage, then this wave's activation slice into registers
  stage_store<DT, HAS_R, NS>(K, sx, sr0, sr1, xpair, xsum);
  __syncthreads();
  u32x4 xr[C][4];
  f32x4 xc[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) xr[c][i] = *reinterpret_cast<const u32x4*>(xpair + chc[c] * 16 + i * 4);
    xc[c] = *reinterpret_cast<const f32x4*>(xsum + chc[c] * 4);
  }

  // ---- 2. rows: compute and reduce the D slots, then refill them while rows remain
  const uint32_t mlo = sgpr_const<0x000F000Fu>();
  const uint32_t mhi = sgpr_const<0x00F000F0u>();
  const uint32_t magic = vgpr_const<kMagic1024g1>();
  if (nj > 0) {
    int j0 = 0;
    while (true) {
      float val[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (j0 + d < nj) {                           // wave-uniform: padding slot
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < C; ++c) {
          float P = 0.0f;
#pragma unroll
          for (int cw = 0; cw < 4; ++cw) {
            const uint32_t w = wb[d][c][cw];
            const uint32_t w8 = w >> 8;
            P = dot2h1((w & mlo) | magic, xr[c][cw][0], P);
            P = dot2h1((w8 & mlo) | magic, xr[c][cw][1], P);
            P = dot2h1((w & mhi) | magic, xr[c][cw][2], P);
            P = dot2h1((w8 & mhi) | magic, xr[c][cw][3], P);
          }
          P -= __builtin_fmaf((float)zb[d][c], xc[c][1], xc[c][0]);
          // a chunk past K reads step 0 (out-of-range buffer offset)
          acc = __builtin_fmaf(f16_to_f32(sb[d][c]) * xc[c][2], P, acc);
        }
        val[d] = acc;
        }
      }
      float v;
      if constexpr (D >= 3) {
        v = pair_sum16(pair_sum32(val[0], val[2]), pair_sum32(val[1], val[3]));   // row j0 + (lane >> 4)
      } else if constexpr (D == 2) {
        const float a = pair_sum32(val[0], val[1]);                               // row j0 + (lane >> 5)
        v = pair_sum16(a, a);
      } else {
        const float a = pair_sum32(val[0], val[0]);
        v = pair_sum16(a, a);
      }
      v = row16_sum(v);
      constexpr int LB = D >= 3 ? 2 : D == 2 ? 1 : 0;
      const int jd = j0 + (lane >> (6 - LB));
      if ((lane & ((64 >> LB) - 1)) == 0 && jd < nj && jd < j0 + D) {
        if (nks == 1) store_y1<YDT>(y, r0 + rg + nrg * jd, v);   // one K slice: the row is complete
        else part[ks * rows_max + rg + nrg * jd] = v;
      }
      j0 += D;
      if (j0 >= nj) break;                           // wave-uniform
      for (int d = 0; d < D; ++d) load_row(d, j0 + d);
    }
  }
  if (nks == 1) return;                             // block-uniform
  __syncthreads();
  for (int t = threadIdx.x; t < nrows; t += blockDim.x) {
    float tot = 0.0f;
    for (int k2 = 0; k2 < nks; ++k2) tot += part[k2 * rows_max + t];
    store_y1<YDT>(y, r0 + t, tot);
  }
}

constexpr size_t kCuLdsReserve = 81 * 1024;


template <int DT, int YDT, bool HAS_R, int NS, int D, int C>
hipError_t gemv1_cu_launch(const uint16_t* x, int64_t K, const uint32_t* qw, const uint16_t* scales,
                         const uint8_t* zeros, int64_t N, int gsh, const float* r, void* y, int nblk,
                         int nrg_max, hipStream_t st) {
  const int64_t CH = K >> 5;
  const int nks = (int)((CH + 64 * C - 1) / (64 * C));
  if (nks > 16 || nblk <= 0 || nrg_max <= 0) return hipErrorInvalidValue;
  const int nrg = 16 / nks < nrg_max ? 16 / nks : nrg_max;
  const int64_t threads = (int64_t)nks * nrg * 64;
  if (((K >> 3) + 3) / 4 * 4 > NS * threads) return hipErrorInvalidValue;
  if (nblk > N) nblk = (int)N;
  const int rows_max = (int)((N + nblk - 1) / nblk);
  size_t lds = (size_t)CH * 16 * 4 + (size_t)CH * 4 * 4 + (size_t)nks * rows_max * 4;
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  // Over half of a compute unit's 160 KB of LDS: no two blocks share a unit,
  // so the grid of one block per unit spreads over all of them.
  if (lds < kCuLdsReserve) lds = kCuLdsReserve;
  hipLaunchKernelGGL((k_gemv1_cu<DT, YDT, HAS_R, NS, D, C>), dim3((unsigned)nblk), dim3((unsigned)threads),
                     lds, st, x, K, qw, scales, zeros, N, r, y, nks, nrg, rows_max, gsh);
  return hipGetLastError();
}

// Launch with nrg row groups per block; the block stages the whole activation
// (NS chunks of 8 per thread must cover K / 8, rounded up to whole quads).
template <int DT, int YDT, bool HAS_R, int UL, int NS>
hipError_t gemv1_rows_launch(const uint16_t* x, int64_t K, const uint32_t* qw, const uint16_t* scales,
                        const uint8_t* zeros, int64_t N, int gsh, const float* r, void* y, int nrg,
                        hipStream_t st) {
  const int64_t CH = K >> 5;
  const int nks = (int)((CH + 63) / 64);
  const int64_t rows = (int64_t)nrg * UL;
  const int64_t threads = (int64_t)nks * nrg * 64;
  if (threads > 1024 || ((K >> 3) + 3) / 4 * 4 > NS * threads) return hipErrorInvalidValue;
  const size_t lds = (size_t)CH * 16 * 4 + (size_t)CH * 4 * 4 + (size_t)nks * rows * 4;
  hipLaunchKernelGGL((k_gemv1_rows<DT, YDT, HAS_R, UL, NS>), dim3((unsigned)((N + rows - 1) / rows)),
                     dim3((unsigned)threads), lds, st, x, K, qw, scales, zeros, N, r, y, nks, gsh);
  return hipGetLastError();
}

constexpr int64_t kRowsMaxK = 24576;      // row-block kernel: staged activation <= 64 KB of LDS
constexpr int64_t kCuMaxK = 32768;        // per-CU kernel: 4 staged pieces per thread, <= 80 KB of LDS
constexpr int kCuMinRowsPerCu = 24;       // below this the row-block kernel is faster

// Which batch-1 kernel serves (K, N): 2 = per-CU, 1 = row-block, 0 = neither.
// The row-block kernel stages the whole activation (and 1/s: 6 bytes per
// channel) in every block; once its blocks' staging reads exceed twice the
// packed weights (few rows per block and a long K, as 4096 x 11008), the
// per-CU kernel, which stages once per compute unit, is faster.
inline int gemv1_path(int64_t K, int64_t N) {
  const int64_t cus = awq::device_cus();
  const int64_t nblk = N < cus ? N : cus;
  const int64_t rows_max = (N + nblk - 1) / nblk;
  const int64_t CH = K >> 5;
  const int64_t nks = (CH + 127) / 128;
  const bool cu_ok = K <= kCuMaxK && CH * 80 + nks * rows_max * 4 <= 160 * 1024 &&
                     rows_max * (K >> 1) < (int64_t(1) << 31);
  const int64_t rks = (CH + 63) / 64;                            // row-block kernel's K slices
  int64_t rnrg = rks >= 8 ? 1 : 8 / rks;
  if (rks * rnrg > 16) rnrg = 16 / rks;
  const int64_t rblocks = (N + 4 * rnrg - 1) / (4 * rnrg);
  const bool rows_staging_heavy = rblocks * K * 6 > 2 * (N * K / 2);
  if (cu_ok && (N >= kCuMinRowsPerCu * cus || K > kRowsMaxK || rows_staging_heavy)) return 2;
  if (K <= kRowsMaxK) return 1;
  return cu_ok ? 2 : 0;
}

// gsh: log2 of the 32-code chunks per group (1, 2, 3 for groups of 64, 128, 256)
template <int DT, int YDT, bool HAS_R>
hipError_t gemv1_dispatch(const uint16_t* x, int64_t K, const uint32_t* qw, const uint16_t* scales,
                          const uint8_t* zeros, int64_t N, int gsh, const float* r, void* y,
                          hipStream_t st) {
  const int path = gemv1_path(K, N);
  const int64_t need = ((K >> 3) + 3) / 4 * 4;     // staged 8-element pieces, whole quads
  if (path == 2) {
    // rows in flight per wave: one for K <= 4096 (the staging loads then wait
    // behind less weight traffic), two up to 16384, four beyond (a long
    // staging phase, with few rows per wave to cover it)
    const int nblk = awq::device_cus();
    const int64_t nks = ((K >> 5) + 127) / 128;
    const int64_t threads = nks * (16 / nks) * 64;
    if (need <= threads) {
      if (K <= 4096)
        return gemv1_cu_launch<DT, YDT, HAS_R, 1, 1, 2>(x, K, qw, scales, zeros, N, gsh, r, y, nblk, 16, st);
      return gemv1_cu_launch<DT, YDT, HAS_R, 1, 2, 2>(x, K, qw, scales, zeros, N, gsh, r, y, nblk, 16, st);
    }
    if (need <= 2 * threads)
      return gemv1_cu_launch<DT, YDT, HAS_R, 2, 2, 2>(x, K, qw, scales, zeros, N, gsh, r, y, nblk, 16, st);
    return gemv1_cu_launch<DT, YDT, HAS_R, 4, 4, 2>(x, K, qw, scales, zeros, N, gsh, r, y, nblk, 16, st);
  }
  if (path == 0) return hipErrorInvalidValue;
  const int64_t CH = K >> 5;
  const int nks = (int)((CH + 63) / 64);
  int nrg = nks >= 8 ? 1 : 8 / nks;
  if (nks * nrg > 16) nrg = 16 / nks;
  const int64_t threads = (int64_t)nks * nrg * 64;
  if (need <= threads) return gemv1_rows_launch<DT, YDT, HAS_R, 4, 1>(x, K, qw, scales, zeros, N, gsh, r, y, nrg, st);
  if (need <= 2 * threads) return gemv1_rows_launch<DT, YDT, HAS_R, 4, 2>(x, K, qw, scales, zeros, N, gsh, r, y, nrg, st);
  return gemv1_rows_launch<DT, YDT, HAS_R, 4, kG1MaxStage>(x, K, qw, scales, zeros, N, gsh, r, y, nrg, st);
}

}  // namespace awqk

namespace awq {

int device_cus() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

bool gemv1_supported(int64_t K, int64_t N) { return awqk::gemv1_path(K, N) != 0; }

hipError_t launch_gemv1(const void* x, int xdt, int64_t K, const uint32_t* qw,
                        const uint16_t* scales, const uint8_t* zeros, int64_t N, int group,
                        const float* r, void* y, int ydt, hipStream_t st) {
  using namespace awqk;
  const uint16_t* xp = (const uint16_t*)x;
  const int gsh = group == 64 ? 1 : group == 128 ? 2 : group == 256 ? 3 : -1;
  if (gsh < 0) return hipErrorInvalidValue;
#define AWQ_G1(DT, YDT)                                                                         \
  return r ? gemv1_dispatch<DT, YDT, true>(xp, K, qw, scales, zeros, N, gsh, r, y, st)          \
           : gemv1_dispatch<DT, YDT, false>(xp, K, qw, scales, zeros, N, gsh, r, y, st)
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
