// Fused W4A16 product ("AWQ > Benefits and Practical Considerations": the
// dequantization unpacks 4-bit integers, applies a group scale and zero point
// and optionally the per-channel inverse scale, fused with the matrix
// multiply so the fp16 weight matrix is never materialised).
//
//   y[m][n] = sum_k step[n][g(k)] * (q[n][k] - z[n][g(k)]) * x[m][k] * r[k]
//
// Two kernels:
//
// * k_gemv (M <= 8): bandwidth-bound split-K GEMV.  A lane owns a fixed
//   128-bit chunk of every row (32 codes = a quarter group), so its slice of
//   x stays in registers for all rows; a wave covers 64 consecutive chunks
//   (2048 codes) of a row, a block's waves cover the row's K slices, and the
//   block walks a tile of rows with all of its 128-bit weight loads in flight.
//   Dequantization is exact and cheap: the nibble pair (q_j, q_j+4) of a word
//   becomes two fp16 values 1024 + q by OR-ing the exponent bits of 1024 into
//   them; a packed fp16 dot product with the matching x pair accumulates in
//   fp32, and the group epilogue subtracts (1024 + z) * sum(x) and applies the
//   step.  The lane's x slice is fp16: as given for fp16 input, otherwise
//   (bf16 input or a 1/s factor) x * r is scaled by an exact power of two per
//   lane and rounded to fp16 once.  Partial sums are reduced across lanes and
//   waves through LDS in a fixed order.
//
// * k_gemm (M > 8): fp16 matrix-core GEMM on 128x128 output tiles, one
//   128-wide group per K step.  A pre-pass rounds each activation row x * r,
//   scaled by an exact power of two, to fp16 (exact for bf16 input without
//   1/s) in the order the nibble unpack produces; a second pre-pass picks a
//   power of two per weight row so that step * 15 stays inside fp16.  Each
//   lane dequantizes its packed word of the B fragment to step * (q - z)
//   rounded once to fp16 and feeds v_mfma_f32_32x32x16_f16; the epilogue
//   undoes both powers of two exactly.
#include "awq_device.h"
#include "awq_internal.h"
#include "k_rows_f16.h"

namespace awqk {

// ===========================================================================
// GEMV
// ===========================================================================
constexpr int kGvVals = 16;      // partial sums per lane per block (units x M)
constexpr int64_t kGemvMaxK = 30720;   // 15 waves of 64 chunks: reduction buffers stay in 64 KB LDS
constexpr int64_t kGemvMaxK8 = 16384;  // 8 waves for 2..8 activation rows

constexpr uint32_t kMagic1024 = 0x64006400u;   // fp16 1024.0 in both halves
constexpr float kOff1024 = 1024.0f;

__device__ __forceinline__ float dot2h(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
}

template <int YDT>
__device__ __forceinline__ void store_y(void* y, int64_t idx, float v) {
  if constexpr (YDT == DT_F32) reinterpret_cast<float*>(y)[idx] = v;
  else reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)from_f32<YDT>(v);
}

// Row units (RPS rows side by side) whose weights a lane loads up front, per
// activation-row count.  More units put more bytes in flight per wave; the
// activation registers limit them for larger MT.
template <int MT>
constexpr int gemv_units() { return MT <= 2 ? 8 : 4; }

// LPR: lanes per row segment (16, 32 or 64); MT: activation rows (1, 2, 4, 8).
// Loads are issued in the order activations, 1/s, weights / steps / zero
// points, all branch-free (out-of-range rows and chunks read a valid address
// and are masked afterwards), so every load of the block is in flight before
// the first wait; the activation slice is converted while the weights arrive.
template <int DT, int YDT, int LPR, int MT, bool HAS_R>
__global__ __launch_bounds__(LPR < 64 ? 64 : (MT == 1 ? 1024 : 512)) void k_gemv(
    const uint16_t* __restrict__ x, int M, int64_t K, int64_t ldx, const uint32_t* __restrict__ qw,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ zeros, int64_t N,
    const float* __restrict__ r, void* __restrict__ y, int64_t ldy) {
  constexpr int RPS = 64 / LPR;                // rows processed side by side per wave
  constexpr int UL = gemv_units<MT>();         // row units loaded per lane
  constexpr int UP = kGvVals / MT;             // row units per reduction pass
  constexpr int NPASS = (UL + UP - 1) / UP;
  constexpr int ROWS = UL * RPS;               // rows per block
  constexpr int NOUT = kGvVals * RPS;          // outputs per reduction pass
  constexpr bool kScaled = (DT == DT_BF16) || HAS_R;

  extern __shared__ float red[];               // [nw][kGvVals][64] then [nw][NOUT]
  const int nw = blockDim.x >> 6;
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int sub = lane / LPR;
  const int cl = lane % LPR;
  const int64_t CH = K >> 5;                   // 16-byte chunks per row
  const int64_t ch = (int64_t)wv * LPR + cl;
  const bool valid = ch < CH;
  const int64_t chc = valid ? ch : 0;          // in-bounds chunk for masked lanes
  const int64_t G = K / kGroup;
  const int64_t gc = chc >> 2;
  const int64_t row0 = (int64_t)blockIdx.x * ROWS;

  // ---- 1. activation (and 1/s) loads
  u32x4 xraw[MT][4];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int cw = 0; cw < 4; ++cw)
      xraw[m][cw] = ldg128(x + (int64_t)(m < M ? m : 0) * ldx + chc * 32 + cw * 8);
  f32x4 rr[8];
  if constexpr (HAS_R) {
#pragma unroll
    for (int i = 0; i < 8; ++i) rr[i] = *reinterpret_cast<const f32x4*>(r + chc * 32 + i * 4);
  }

  // ---- 2. weights, steps, zero points of all the block's rows
  u32x4 wq[UL];
  uint32_t sraw[UL], zraw[UL];
#pragma unroll
  for (int u = 0; u < UL; ++u) {
    int64_t row = row0 + u * RPS + sub;
    row = row < N ? row : N - 1;
    wq[u] = ldg128_stream(qw + row * (K >> 3) + chc * 4);
    sraw[u] = scales[row * G + gc];
    zraw[u] = zeros[row * G + gc];
  }
  // keep every load above this point: nothing below may be hoisted between
  // them, so all of them are in flight before the first wait
  __builtin_amdgcn_sched_barrier(0);

  // ---- 3. activation slice -> fp16 pairs (x_j, x_j+4) per word, sum, scale
  uint32_t xp[MT][16];
  float xs[MT], xscale[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    uint32_t h[32];
    xscale[m] = 1.0f;
    if constexpr (kScaled) {
      float v[32];
#pragma unroll
      for (int cw = 0; cw < 4; ++cw)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[cw * 8 + 2 * j] = lo_f32<DT>(xraw[m][cw][j]);
          v[cw * 8 + 2 * j + 1] = hi_f32<DT>(xraw[m][cw][j]);
        }
      if constexpr (HAS_R) {
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] *= rr[i >> 2][i & 3];
      }
      float amax = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
      const int p = pow2_exp_for(amax);
      xscale[m] = ldexpf(1.0f, -p);
#pragma unroll
      for (int i = 0; i < 32; ++i) h[i] = f32_to_f16_bits(ldexpf(v[i], p));
    } else {
#pragma unroll
      for (int cw = 0; cw < 4; ++cw)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          h[cw * 8 + 2 * j] = xraw[m][cw][j] & 0xFFFFu;
          h[cw * 8 + 2 * j + 1] = xraw[m][cw][j] >> 16;
        }
    }
    const bool live = valid && m < M;
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) sum += f16_to_f32(h[i]);
    xs[m] = live ? sum : 0.0f;
#pragma unroll
    for (int cw = 0; cw < 4; ++cw)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        xp[m][cw * 4 + j] = live ? (h[cw * 8 + j] | (h[cw * 8 + j + 4] << 16)) : 0u;
  }

  // ---- 4. dot products and the reduction, one pass of UP row units at a time
  constexpr int LPO = 64 / NOUT;               // lanes per output in the LDS reduction: 4, 2 or 1
  float* rw = red + wv * (kGvVals * 64);
  float* r2 = red + nw * (kGvVals * 64);
#pragma unroll
  for (int pass = 0; pass < NPASS; ++pass) {
    float val[kGvVals];
#pragma unroll
    for (int uu = 0; uu < UP; ++uu) {
      const int u = pass * UP + uu;
      if (u >= UL) {
#pragma unroll
        for (int m = 0; m < MT; ++m) val[uu * MT + m] = 0.0f;
        continue;
      }
      const bool rowok = valid && (row0 + u * RPS + sub) < N;
      const float dz = rowok ? f16_to_f32(sraw[u]) : 0.0f;
      const float cz = kOff1024 + (float)zraw[u];
      float P[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m) P[m] = 0.0f;
#pragma unroll
      for (int cw = 0; cw < 4; ++cw) {
        const uint32_t wword = wq[u][cw];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t pr = ((wword >> (4 * j)) & 0x000F000Fu) | kMagic1024;
#pragma unroll
          for (int m = 0; m < MT; ++m) P[m] = dot2h(pr, xp[m][cw * 4 + j], P[m]);
        }
      }
#pragma unroll
      for (int m = 0; m < MT; ++m)
        val[uu * MT + m] = (dz * __builtin_fmaf(-cz, xs[m], P[m])) * xscale[m];
    }

    if (pass > 0) __syncthreads();               // the previous pass has read its LDS
#pragma unroll
    for (int v = 0; v < kGvVals; ++v) rw[v * 64 + lane] = val[v];
    __syncthreads();
    {
      const int o = lane / LPO;
      const int jj = lane % LPO;
      const int v = o / RPS;
      const int osub = o % RPS;
      const float* src = rw + v * 64 + osub * LPR + jj * 16;
      float t = 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) t += src[i];
#pragma unroll
      for (int off = LPO / 2; off >= 1; off >>= 1) t += __shfl_xor(t, off);
      if (jj == 0) r2[wv * NOUT + o] = t;
    }
    __syncthreads();
    if ((int)threadIdx.x < NOUT) {
      const int oo = threadIdx.x;
      float tot = 0.0f;
      for (int w = 0; w < nw; ++w) tot += r2[w * NOUT + oo];
      const int vv = oo / RPS;
      const int uu = vv / MT;
      const int m = vv % MT;
      const int u = pass * UP + uu;
      const int64_t row = row0 + (int64_t)u * RPS + (oo % RPS);
      if (u < UL && row < N && m < M) store_y<YDT>(y, (int64_t)m * ldy + row, tot);
    }
  }
}

// ===========================================================================
// matrix-core GEMM
// ===========================================================================

// Per weight row n: e_n with max_g step[n][g] * 2^e_n in [2^-10, 2^-9), so that
// D' = step 2^e_n times 2^24 is a finite fp16 and D' (q - z) is a normal fp16.
__global__ void k_step_exp(const uint16_t* __restrict__ scales, int64_t N, int64_t G,
                           int* __restrict__ eexp) {
  const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  float mx = 0.0f;
  for (int64_t g = 0; g < G; ++g) mx = fmaxf(mx, f16_to_f32(scales[n * G + g]));
  int e = 0;
  if (mx > 0.0f) {
    int ex;
    frexpf(mx, &ex);        // mx < 2^ex
    e = -9 - ex;            // mx * 2^e in [2^-10, 2^-9): D' 2^24 stays finite in fp16
  }
  eexp[n] = e;
}

__device__ __forceinline__ f32x16 mfma32h(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// One packed word (codes of k = 8c + j in bits 4j..4j+3) -> 8 fp16 operands
// D' (q - z), k order (0,4 | 2,6 | 1,5 | 3,7).  The masked nibbles are read
// as fp16 subnormals q 2^-24 (nibbles 1/3/5/7 still 4 bits up: q 2^-20); one
// packed fma with the fp16 constants D' 2^24 (or D' 2^20) and -D' z gives
// D' q - D' z with one rounding.  Shift, 4 ands and 4 fmas per word.
__device__ __forceinline__ u32x4 dequant_word_f16(uint32_t w, f16x2 c24, f16x2 c20, f16x2 nzd) {
  const uint32_t w8 = w >> 8;
  u32x4 out;
  out[0] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(
      __builtin_bit_cast(f16x2, w & 0x000F000Fu), c24, nzd));
  out[1] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(
      __builtin_bit_cast(f16x2, w8 & 0x000F000Fu), c24, nzd));
  out[2] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(
      __builtin_bit_cast(f16x2, w & 0x00F000F0u), c20, nzd));
  out[3] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(
      __builtin_bit_cast(f16x2, w8 & 0x00F000F0u), c20, nzd));
  return out;
}

// 256 x 256 output tile per block of 8 waves (2 along m x 4 along n, each wave
// 128 x 64 = 4 x 2 blocks of 32 x 32), 64 k per LDS stage, two LDS stages so
// that the next stage's global loads are in flight during the current
// stage's matrix-core work (one barrier per stage).
constexpr int kMT = 256;                // tile rows (m)
constexpr int kNT = 256;                // tile columns (n)
constexpr int kBK = 64;                 // k per stage
constexpr int kALd = kBK + 8;           // x tile row stride (16-bit elements)
constexpr int kBLd = 12;                // packed-word tile row stride (words; 8 used)

template <int YDT>
__global__ __launch_bounds__(512) void k_gemm(const uint16_t* __restrict__ xq, int64_t M, int64_t K,
                                              const int* __restrict__ pm,
                                              const uint32_t* __restrict__ qw,
                                              const uint16_t* __restrict__ scales,
                                              const uint8_t* __restrict__ zeros,
                                              const int* __restrict__ en, int64_t N,
                                              void* __restrict__ y, int64_t ldy) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kMT * kALd];
  __shared__ __attribute__((aligned(16))) uint32_t Bq[2][kNT * kBLd];
  __shared__ __attribute__((aligned(16))) uint32_t Bc[2][kNT * 4];   // D'2^24, D'2^20, -D'z (fp16 pairs)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv >> 2, wn = wv & 3;
  const int64_t m0 = (int64_t)blockIdx.y * kMT;
  const int64_t n0 = (int64_t)blockIdx.x * kNT;
  const int64_t G = K / kGroup;
  const int64_t S = K / kBK;
  const int bcol = tid & 255;                    // column this thread stages (B side)
  const bool bcol_ok = n0 + bcol < N;
  const int64_t bcol_c = bcol_ok ? n0 + bcol : 0;
  const int ecol = bcol_ok ? en[bcol_c] : 0;

  // per-thread source pointers (advanced by k0 each stage)
  const uint16_t* asrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 512 * i;
    const int64_t mr = m0 + (c >> 3);
    asrc[i] = xq + (mr < M ? mr : 0) * K + (c & 7) * 8;
  }
  const uint32_t* bsrc = qw + bcol_c * (K >> 3);
  const uint16_t* ssrc = scales + bcol_c * G;
  const uint8_t* zsrc = zeros + bcol_c * G;

  f32x16 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

  u32x4 ra[4];              // staged x chunks
  u32x4 rb0, rb1;           // staged packed words (threads < 256)
  uint32_t rs = 0, rz = 0;  // staged step / zero (threads >= 256)

  auto gload = [&](int64_t s) {
    const int64_t k0 = s * kBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) ra[i] = ldg128(asrc[i] + k0);
    if (tid < 256) {
      rb0 = ldg128_stream(bsrc + (k0 >> 3));
      rb1 = ldg128_stream(bsrc + (k0 >> 3) + 4);
    } else {
      rs = ssrc[k0 / kGroup];
      rz = zsrc[k0 / kGroup];
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 512 * i;
      // rows past M hold row 0's data: output rows are independent and those are never stored
      *reinterpret_cast<u32x4*>(&As[buf][(c >> 3) * kALd + (c & 7) * 8]) = ra[i];
    }
    if (tid < 256) {
      // word order (0,2,4,6 | 1,3,5,7): a lane's four k steps are one 16-byte read
      // columns past N hold column 0's words; their outputs are never stored
      const u32x4 e = {rb0[0], rb0[2], rb1[0], rb1[2]};
      const u32x4 o = {rb0[1], rb0[3], rb1[1], rb1[3]};
      *reinterpret_cast<u32x4*>(&Bq[buf][bcol * kBLd]) = e;
      *reinterpret_cast<u32x4*>(&Bq[buf][bcol * kBLd + 4]) = o;
    } else {
      u32x4 c = {0u, 0u, 0u, 0u};
      if (bcol_ok) {
        const float D = ldexpf(f16_to_f32(rs), ecol);        // D' (exact: power-of-two scaling)
        const uint32_t h24 = f32_to_f16_bits(D * 16777216.0f);
        const uint32_t h20 = f32_to_f16_bits(D * 1048576.0f);
        const uint32_t hz = f32_to_f16_bits(-(D * (float)rz));
        c[0] = h24 | (h24 << 16);
        c[1] = h20 | (h20 << 16);
        c[2] = hz | (hz << 16);
      }
      *reinterpret_cast<u32x4*>(&Bc[buf][bcol * 4]) = c;
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int64_t s = 0; s < S; ++s) {
    const int buf = (int)(s & 1);
    if (s + 1 < S) gload(s + 1);
    f16x2 c24[2], c20[2], nzd[2];
    u32x4 bw[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int col = wn * 64 + nb * 32 + (lane & 31);
      const u32x4 c = *reinterpret_cast<const u32x4*>(&Bc[buf][col * 4]);
      c24[nb] = as_f16x2(c[0]);
      c20[nb] = as_f16x2(c[1]);
      nzd[nb] = as_f16x2(c[2]);
      bw[nb] = *reinterpret_cast<const u32x4*>(&Bq[buf][col * kBLd + (lane >> 5) * 4]);
    }
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      u32x4 a[4], b[2];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        a[mb] = *reinterpret_cast<const u32x4*>(
            &As[buf][(wm * 128 + mb * 32 + (lane & 31)) * kALd + ks * 16 + 8 * (lane >> 5)]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) b[nb] = dequant_word_f16(bw[nb][ks], c24[nb], c20[nb], nzd[nb]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32h(a[mb], b[nb], acc[mb][nb]);
    }
    if (s + 1 < S) lstore(buf ^ 1);
    __syncthreads();
  }

  // 32x32 accumulator layout: column = lane % 32, row = 8 (v / 4) + 4 (lane / 32) + v % 4
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int64_t n = n0 + wn * 64 + nb * 32 + (lane & 31);
    if (n >= N) continue;
    const int e = en[n];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + wm * 128 + mb * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (m < M) store_y<YDT>(y, m * ldy + n, ldexpf(acc[mb][nb][v], -(pm[m] + e)));
      }
  }
}

// ---------------------------------------------------------------------------
template <int DT, int YDT, bool HAS_R>
hipError_t gemv_dispatch(const uint16_t* x, int M, int64_t K, int64_t ldx, const uint32_t* qw,
                         const uint16_t* scales, const uint8_t* zeros, int64_t N, const float* r,
                         void* y, int64_t ldy, hipStream_t st) {
  const int64_t CH = K >> 5;
  const int lpr = CH >= 64 ? 64 : (CH > 16 ? 32 : 16);
  const int64_t nw = (CH + lpr - 1) / lpr;   // <= 15 (K <= kGemvMaxK)
  const int rps = 64 / lpr;
  const int mt = M <= 1 ? 1 : (M <= 2 ? 2 : (M <= 4 ? 4 : 8));
  const int rows = (mt <= 2 ? gemv_units<1>() : gemv_units<8>()) * rps;
  const dim3 grid((unsigned)((N + rows - 1) / rows));
  const dim3 block((unsigned)(nw * 64));
  const size_t lds = (size_t)nw * kGvVals * 64 * 4 + (size_t)nw * kGvVals * rps * 4;
#define AWQ_GV(LPR, MT)                                                                        \
  hipLaunchKernelGGL((k_gemv<DT, YDT, LPR, MT, HAS_R>), grid, block, lds, st, x, M, K, ldx, qw, \
                     scales, zeros, N, r, y, ldy)
#define AWQ_GV_M(LPR)            \
  switch (mt) {                  \
    case 1: AWQ_GV(LPR, 1); break; \
    case 2: AWQ_GV(LPR, 2); break; \
    case 4: AWQ_GV(LPR, 4); break; \
    default: AWQ_GV(LPR, 8); break; \
  }
  if (lpr == 64) { AWQ_GV_M(64) }
  else if (lpr == 32) { AWQ_GV_M(32) }
  else { AWQ_GV_M(16) }
#undef AWQ_GV_M
#undef AWQ_GV
  return hipGetLastError();
}

struct GemmWs {
  uint16_t* xq;
  int* pm;
  int* en;
  size_t bytes;
};

inline GemmWs gemm_ws(void* ws, int64_t M, int64_t N, int64_t K) {
  GemmWs w{};
  char* base = (char*)ws;
  size_t off = 0;
  auto take = [&](size_t b) {
    char* p = base ? base + off : nullptr;
    off += awq::align_up(b, 256);
    return p;
  };
  w.xq = (uint16_t*)take((size_t)M * K * 2);
  w.pm = (int*)take((size_t)M * 4);
  w.en = (int*)take((size_t)N * 4);
  w.bytes = off;
  return w;
}

inline bool use_gemv(int64_t M, int64_t K) {
  return (M == 1 && K <= kGemvMaxK) || (M <= 8 && K <= kGemvMaxK8);
}

template <int DT, int YDT, bool HAS_R>
hipError_t gemm_dispatch(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint32_t* qw,
                         const uint16_t* scales, const uint8_t* zeros, int64_t N, const float* r,
                         void* y, int64_t ldy, void* ws, hipStream_t st) {
  const GemmWs w = gemm_ws(ws, M, N, K);
  hipLaunchKernelGGL((k_rows_f16<DT, HAS_R, true>), dim3((unsigned)M), dim3(256), 0, st, x, K, ldx,
                     r, w.xq, w.pm);
  hipLaunchKernelGGL(k_step_exp, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, st, scales, N,
                     K / kGroup, w.en);
  const dim3 grid((unsigned)((N + kNT - 1) / kNT), (unsigned)((M + kMT - 1) / kMT));
  hipLaunchKernelGGL((k_gemm<YDT>), grid, dim3(512), 0, st, w.xq, M, K, w.pm, qw, scales, zeros,
                     w.en, N, y, ldy);
  return hipGetLastError();
}

template <int DT, int YDT>
hipError_t w4a16_dispatch(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint32_t* qw,
                          const uint16_t* scales, const uint8_t* zeros, int64_t N, const float* r,
                          void* y, int64_t ldy, void* ws, hipStream_t st) {
  if (M == 1 && awq::gemv1_supported(K, N))
    return awq::launch_gemv1(x, DT, K, qw, scales, zeros, N, r, y, YDT, st);
  if (use_gemv(M, K)) {
    if (r) return gemv_dispatch<DT, YDT, true>(x, (int)M, K, ldx, qw, scales, zeros, N, r, y, ldy, st);
    return gemv_dispatch<DT, YDT, false>(x, (int)M, K, ldx, qw, scales, zeros, N, r, y, ldy, st);
  }
  if (r) return gemm_dispatch<DT, YDT, true>(x, M, K, ldx, qw, scales, zeros, N, r, y, ldy, ws, st);
  return gemm_dispatch<DT, YDT, false>(x, M, K, ldx, qw, scales, zeros, N, r, y, ldy, ws, st);
}

}  // namespace awqk

namespace awq {

size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || awqk::use_gemv(M, K) || (M == 1 && gemv1_supported(K, N)))
    return 0;
  return awqk::gemm_ws(nullptr, M, N, K).bytes;
}

hipError_t launch_w4a16(const void* x, int xdt, int64_t M, int64_t K, int64_t ldx,
                        const uint32_t* qw, const uint16_t* scales, const uint8_t* zeros,
                        int64_t N, const float* inv_s, void* y, int ydt, int64_t ldy, void* ws,
                        hipStream_t st) {
  using namespace awqk;
  const uint16_t* xp = (const uint16_t*)x;
  if (xdt == DT_F16) {
    if (ydt == DT_F16) return w4a16_dispatch<DT_F16, DT_F16>(xp, M, K, ldx, qw, scales, zeros, N, inv_s, y, ldy, ws, st);
    if (ydt == DT_BF16) return w4a16_dispatch<DT_F16, DT_BF16>(xp, M, K, ldx, qw, scales, zeros, N, inv_s, y, ldy, ws, st);
    return w4a16_dispatch<DT_F16, DT_F32>(xp, M, K, ldx, qw, scales, zeros, N, inv_s, y, ldy, ws, st);
  }
  if (ydt == DT_F16) return w4a16_dispatch<DT_BF16, DT_F16>(xp, M, K, ldx, qw, scales, zeros, N, inv_s, y, ldy, ws, st);
  if (ydt == DT_BF16) return w4a16_dispatch<DT_BF16, DT_BF16>(xp, M, K, ldx, qw, scales, zeros, N, inv_s, y, ldy, ws, st);
  return w4a16_dispatch<DT_BF16, DT_F32>(xp, M, K, ldx, qw, scales, zeros, N, inv_s, y, ldy, ws, st);
}

}  // namespace awq
