// W4A16 product for small batches, 17 <= M <= 64 ("AWQ > Benefits and
// Practical Considerations": unpack the 4-bit integers, apply the group scale
// and zero point and the optional per-channel inverse scale, fused with the
// multiply).  At these batch sizes the product is bound by the packed weight
// stream ("AWQ Math", "Weight-only quantization and where it breaks": decode
// is weight-loading bound), not by the matrix cores.
//
//   1. k_rows_f16 (pre-pass): each token row x r as fp16 with an exact power
//      of two per row, in the order the nibble unpack yields, each
//      128-channel unit's sixteen 8-channel pieces transposed 4 x 4 (x_q [M][K]).
//   2. k_gemm_mid: block (s, b) takes a range of at most T 16-row tiles and
//      the s-th of S slices of the 128-channel units; wave w takes an eighth
//      of the slice's units.  Per unit a lane loads one 128-bit chunk of
//      packed words per tile and, straight from x_q (a few hundred KB, served
//      by the L2 after the first reads), the activation operands of its token
//      in each 16-token group, which serve all T tiles; it runs
//      v_mfma_f32_16x16x32_f16 with the dequantized weights as A and each
//      token group as B, two units of operands in flight.  The eight waves'
//      partial tiles meet in LDS in wave order; with S = 1 the result is
//      scaled back and stored, otherwise fp32 partial sums go to the
//      workspace.
//   3. k_mid_reduce (S > 1): y = sum over slices in slice order, scaled back.
// Layers with more 16-row tiles than compute units run as whole rounds of one
// block per compute unit over nearly equal row ranges (no slices, no third
// launch); smaller ones split over K only when every block reading all of the
// activations would cost more than the extra launch.  The partial sums meet
// in a separate kernel rather than in the last-arriving block: each L2 slice
// of this chip serves its own group of compute units, so making one block's
// writes visible to blocks elsewhere takes a device-scope fence that writes
// the L2 back (measured 8x slower).
#include "awq_device.h"
#include "awq_internal.h"
#include "k_rows_f16.h"

namespace awqk {

constexpr int kMidWaves = 8;                       // waves per block, each 1/8 of the slice's units
constexpr int kMidP = 2;                           // units of operands in flight per wave (4: slower)
constexpr int kMidPad = 17;                        // floats per token row of a partial tile in LDS
constexpr int64_t kMidWholeX = 256 * 1024;         // activation bytes every block of a small layer may read
// Below 17 tokens the single-launch product that stages the whole activation
// in each compute unit's LDS (k_gemm_skinny_st) is faster.
constexpr int64_t kMidMinM = 17;

template <int YDT>
__device__ __forceinline__ void store_ym(void* y, int64_t idx, float v) {
  if constexpr (YDT == DT_F32) reinterpret_cast<float*>(y)[idx] = v;
  else reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)from_f32<YDT>(v);
}

// One packed word -> 8 fp16 operands step 2^e (q - z), in the order
// (0,4 | 2,6 | 1,5 | 3,7): the nibbles are read as fp16 subnormals q 2^-24
// (odd nibbles still 4 bits up: q 2^-20) and one packed fma with the fp16
// constants D' 2^24 (D' 2^20) and -D' z gives D' q - D' z with one rounding.
__device__ __forceinline__ u32x4 mid_dequant(uint32_t w, f16x2 c24, f16x2 c20, f16x2 nzd) {
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

// TG: 16-token groups (1..4); T: 16-row tiles per block (every wave runs all
// of them, so one load of an activation operand serves T tiles); SPLIT: S > 1.
// Block (s, b) takes rows [b N / nb, (b + 1) N / nb) (at most 16 T) and the
// s-th of S slices of the 128-channel units; each wave takes an eighth of the
// slice's units.
// Lane (rl, b4) = (lane % 16, lane / 16) holds, per unit, the 32-channel block
// b4 of weight row rl of each tile (one 128-bit chunk) and of token rl of each
// token group (four 128-bit chunks of x_q, read straight from memory: x_q is a
// few hundred KB, so after the first reads it is served by the L2).
template <int YDT, int TG, int T, bool SPLIT>
__global__ __launch_bounds__(64 * kMidWaves) void k_gemm_mid(
    const uint16_t* __restrict__ xq, const int* __restrict__ pm, int M, int64_t K,
    const uint32_t* __restrict__ qw, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zeros, int64_t N, int64_t nb, int glog, int S,
    float* __restrict__ partial, int* __restrict__ en, void* __restrict__ y, int64_t ldy) {
  constexpr int R = 16 * T;                      // rows a block can hold
  constexpr int TILE = 16 * kMidPad;             // floats of one partial 16 x 16 tile in LDS
  extern __shared__ __attribute__((aligned(16))) float red[];   // [waves][T][TG][16 tokens][kMidPad]
  __shared__ int e_s[R];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rl = lane & 15;                      // A row / B token within a group
  const int b4 = lane >> 4;                      // 32-channel block of the unit
  const int bs = (int)(blockIdx.x % (unsigned)S);
  const int64_t bn = blockIdx.x / (unsigned)S;
  const int64_t n0 = bn * N / nb;                // rows [n0, n1): nb nearly equal ranges
  const int nrows = (int)((bn + 1) * N / nb - n0);   // <= ceil(N / nb) <= R
  const int U = (int)(K >> 7);
  const int u0 = bs * U / S, u1 = (bs + 1) * U / S;            // U <= 1024, S <= U
  const int us = u1 - u0;
  // the wave's eighth of the slice and the unit it starts from both turn with
  // the block, so that the blocks do not all read the same activation columns
  // at once (measured neutral to 1.5 % faster)
  const int ks = (wv + (int)(blockIdx.x % (unsigned)kMidWaves)) % kMidWaves;
  const int w0 = u0 + ks * us / kMidWaves;
  const int nw = u0 + (ks + 1) * us / kMidWaves - w0;          // the wave's units
  const int rot = nw > 0 ? (int)((blockIdx.x / (unsigned)kMidWaves) % (unsigned)nw) : 0;
  const int GW = (int)(K >> glog);               // weight groups per row
  const int csh = glog - 5;                      // 32-code chunk -> weight group
  const uint32_t KW = (uint32_t)(K >> 3);

  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(qw + n0 * KW), (short)0, nrows * (int)KW * 4, kBufferWord3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(scales + n0 * GW), (short)0, nrows * GW * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(zeros + n0 * GW), (short)0, nrows * GW, kBufferWord3);
  // token rows >= M lie past the end: they read as zeros
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)xq, (short)0, (int)((int64_t)M * K * 2), kBufferWord3);

  // ---- 1. the first units' operands
  u32x4 xa[kMidP][TG][4];
  u32x4 wa[kMidP][T];
  uint32_t sr[kMidP][T], zr[kMidP][T];
  auto load_unit = [&](int slot, int j) {      // the wave's j-th unit
    const bool ok = j < nw;                      // wave-uniform
    const int u = w0 + (j + rot < nw ? j + rot : j + rot - nw);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const int row = 16 * t + rl;
      const bool rok = ok && row < nrows;
      const uint32_t gw = (uint32_t)(row * GW + ((4 * u + b4) >> csh));
      wa[slot][t] = __builtin_amdgcn_raw_buffer_load_b128(
          wrs, rok ? (uint32_t)row * KW * 4 + (uint32_t)(4 * u + b4) * 16 : kBufferOob, 0, kBufferNt);
      sr[slot][t] = __builtin_amdgcn_raw_buffer_load_b16(srs, rok ? gw * 2 : kBufferOob, 0, 0);
      zr[slot][t] = __builtin_amdgcn_raw_buffer_load_b8(zrs, rok ? gw : kBufferOob, 0, 0);
    }
#pragma unroll
    for (int g = 0; g < TG; ++g) {
      const uint32_t off = (uint32_t)(16 * g + rl) * (uint32_t)K * 2 + (uint32_t)u * 256 + (uint32_t)b4 * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        xa[slot][g][i] = __builtin_amdgcn_raw_buffer_load_b128(xrs, ok ? off + 64 * i : kBufferOob, 0, 0);
    }
  };
#pragma unroll
  for (int d = 0; d < kMidP; ++d) load_unit(d, d);

  // ---- 2. per-row power of two e (max step 2^e in [2^-10, 2^-9)) from all of
  // the row's steps: the same for every slice, so partial sums share a scale
  const int npc = (GW * 2 + 15) / 16;            // 16-byte pieces of a row's steps
  int e[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int row = 16 * t + rl;
    float mx = 0.0f;
    for (int pc = b4; pc < npc; pc += 4) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(
          srs, row < nrows ? (uint32_t)row * GW * 2 + 16 * pc : kBufferOob, 0, 0);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (pc * 8 + j < GW) mx = fmaxf(mx, f16_to_f32((v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu));
    }
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    e[t] = 0;
    if (mx > 0.0f) {
      int ex;
      frexpf(mx, &ex);
      e[t] = -9 - ex;
    }
    if (wv == 0 && b4 == 0) {
      e_s[row] = e[t];
      if (SPLIT && bs == 0 && row < nrows) en[n0 + row] = e[t];
    }
  }

  // ---- 3. units: dequantize each tile's chunk, multiply every token group
  f32x4 acc[T][TG];
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int g = 0; g < TG; ++g) acc[t][g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int jb = 0; jb < nw; jb += kMidP) {
#pragma unroll
    for (int d = 0; d < kMidP; ++d) {
      const int j = jb + d;
      if (j < nw) {                                             // wave-uniform
#pragma unroll
        for (int t = 0; t < T; ++t) {
          const float D = ldexpf(f16_to_f32(sr[d][t]), e[t]);
          const uint32_t h24 = f32_to_f16_bits(D * 16777216.0f);
          const uint32_t h20 = f32_to_f16_bits(D * 1048576.0f);
          const uint32_t hz = f32_to_f16_bits(-(D * (float)zr[d][t]));
          const f16x2 c24 = as_f16x2(h24 | (h24 << 16));
          const f16x2 c20 = as_f16x2(h20 | (h20 << 16));
          const f16x2 nzd = as_f16x2(hz | (hz << 16));
          u32x4 a[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) a[i] = mid_dequant(wa[d][t][i], c24, c20, nzd);
#pragma unroll
          for (int g = 0; g < TG; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][g] = mfma16h(a[i], xa[d][g][i], acc[t][g]);
        }
      }
      load_unit(d, j + kMidP);
    }
  }

  // ---- 4. the waves' partial tiles meet in LDS, added in wave order.
  // 16 x 16 layout: token = lane % 16, row = 4 (lane / 16) + v.
  float* mine = red + (size_t)wv * T * TG * TILE;
#pragma unroll
  for (int t = 0; t < T; ++t)
#pragma unroll
    for (int g = 0; g < TG; ++g)
#pragma unroll
      for (int v = 0; v < 4; ++v) mine[(t * TG + g) * TILE + rl * kMidPad + 4 * b4 + v] = acc[t][g][v];
  __syncthreads();
  // output j: row j % 16 of tile (j / 256) / TG, token (j / 16) % 16 of group (j / 256) % TG
  for (int j = tid; j < T * TG * 256; j += 64 * kMidWaves) {
    const int orr = j & 15, otok = (j >> 4) & 15, tg = j >> 8;
    const int orow = (tg / TG) * 16 + orr, m = (tg % TG) * 16 + otok;
    if (orow < nrows && m < M) {
      float tot = 0.0f;
#pragma unroll
      for (int w = 0; w < kMidWaves; ++w) tot += red[((size_t)w * T * TG + tg) * TILE + otok * kMidPad + orr];
      const int64_t n = n0 + orow;
      if constexpr (SPLIT) partial[((int64_t)bs * M + m) * N + n] = tot;
      else store_ym<YDT>(y, (int64_t)m * ldy + n, ldexpf(tot, -(pm[m] + e_s[orow])));
    }
  }
}

// y[m][n] = (sum over slices s = 0..S-1 of partial[s][m][n]) 2^-(pm[m] + en[n])
template <int YDT>
__global__ __launch_bounds__(256) void k_mid_reduce(const float* __restrict__ partial, int S, int M,
                                                    int64_t N, const int* __restrict__ pm,
                                                    const int* __restrict__ en, void* __restrict__ y,
                                                    int64_t ldy) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)M * N) return;
  const int64_t m = i / N, n = i - m * N;
  float tot = 0.0f;
  for (int s = 0; s < S; ++s) tot += partial[(int64_t)s * M * N + i];
  store_ym<YDT>(y, m * ldy + n, ldexpf(tot, -(pm[m] + en[n])));
}

struct MidPlan {
  int S = 0;          // K slices
  int tg = 0;         // 16-token groups
  int T = 0;          // 16-row tiles a block can hold
  int64_t nb = 0;     // row blocks
  size_t lds = 0;     // dynamic LDS: the waves' partial tiles
  int64_t blocks = 0;
};

// Row blocks hold at most T tiles (T <= 4 with up to 32 tokens, <= 2 above:
// the operands in flight must fit the registers); one load of an activation
// operand serves all of a block's tiles.  With more tiles than compute units,
// a whole number of rounds of one block per compute unit, the rows split into
// nearly equal ranges, so every compute unit streams the same share of the
// weights.  With fewer: one tile per block while the activations are at most
// kMidWholeX bytes (every block reads all of them), else blocks of T whole
// tiles and the units split into slices, so that each block reads only its
// slice of the activations at the cost of the slices' sum in a second kernel
// (measured: 4096 x 11008 at 32 tokens 28.8 against 32.0 us, 4096 x 4096 at
// 32 tokens 18.6 against 16.6 us).  Slices: the fewest (a power of two) that
// give a block per compute unit while every wave keeps a unit.
inline MidPlan mid_plan(int64_t M, int64_t N, int64_t K) {
  MidPlan p;
  if (M < kMidMinM || M > 64 || K % 128 != 0 || N <= 0) return p;
  const int64_t U = K / 128;
  const int64_t cus = awq::device_cus();
  p.tg = (int)((M + 15) / 16);
  const int64_t tmax = p.tg <= 2 ? 4 : 2;
  const int64_t tiles = (N + 15) / 16;
  if (tiles > cus) {
    const int64_t rounds = (tiles + cus * tmax - 1) / (cus * tmax);
    p.nb = tiles < rounds * cus ? tiles : rounds * cus;
  } else if (M * K * 2 <= kMidWholeX) {
    p.nb = tiles;
  } else {
    p.nb = (tiles + tmax - 1) / tmax;
  }
  p.T = (int)(((N + p.nb - 1) / p.nb + 15) / 16);
  int64_t S = 1;
  while (S * p.nb < cus && S * 2 * kMidWaves <= U) S *= 2;
  p.S = (int)S;
  p.lds = (size_t)kMidWaves * p.T * p.tg * 16 * kMidPad * sizeof(float);
  p.blocks = S * p.nb;
  return p;
}

struct MidWs {
  uint16_t* xq;
  int* pm;
  int* en;
  float* partial;
  size_t bytes;
};

inline MidWs mid_ws(void* ws, int64_t M, int64_t N, int64_t K, int S) {
  MidWs w{};
  char* base = (char*)ws;
  size_t off = 0;
  auto take = [&](size_t b) {
    char* q = base ? base + off : nullptr;
    off += awq::align_up(b, 256);
    return q;
  };
  w.xq = (uint16_t*)take((size_t)M * K * 2);
  w.pm = (int*)take((size_t)M * 4);
  w.en = (int*)take((size_t)N * 4);
  w.partial = S > 1 ? (float*)take((size_t)S * M * N * 4) : nullptr;
  w.bytes = off;
  return w;
}

template <int YDT, int TG, int T>
hipError_t mid_launch_t(const MidWs& w, int64_t M, int64_t K, const uint32_t* qw, const uint16_t* scales,
                        const uint8_t* zeros, int64_t N, int glog, void* y, int64_t ldy, const MidPlan& p,
                        hipStream_t st) {
  if (p.S == 1) {
    hipLaunchKernelGGL((k_gemm_mid<YDT, TG, T, false>), dim3((unsigned)p.blocks), dim3(64 * kMidWaves), p.lds,
                       st, w.xq, w.pm, (int)M, K, qw, scales, zeros, N, p.nb, glog, p.S, w.partial, w.en, y,
                       ldy);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_gemm_mid<YDT, TG, T, true>), dim3((unsigned)p.blocks), dim3(64 * kMidWaves), p.lds,
                     st, w.xq, w.pm, (int)M, K, qw, scales, zeros, N, p.nb, glog, p.S, w.partial, w.en, y,
                     ldy);
  hipLaunchKernelGGL((k_mid_reduce<YDT>), dim3((unsigned)((M * N + 255) / 256)), dim3(256), 0, st,
                     w.partial, p.S, (int)M, N, w.pm, w.en, y, ldy);
  return hipGetLastError();
}

template <int DT, int YDT, bool HAS_R, int TG>
hipError_t mid_launch(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint32_t* qw,
                      const uint16_t* scales, const uint8_t* zeros, int64_t N, int glog, const float* r,
                      void* y, int64_t ldy, const MidPlan& p, void* ws, hipStream_t st) {
  const MidWs w = mid_ws(ws, M, N, K, p.S);
  hipLaunchKernelGGL((k_rows_f16<DT, HAS_R, true, true>), dim3((unsigned)M), dim3(256), 0, st, x, K, ldx, r,
                     w.xq, w.pm);
  switch (p.T) {
    case 1: return mid_launch_t<YDT, TG, 1>(w, M, K, qw, scales, zeros, N, glog, y, ldy, p, st);
    case 2: return mid_launch_t<YDT, TG, 2>(w, M, K, qw, scales, zeros, N, glog, y, ldy, p, st);
    default:
      if constexpr (TG <= 2) {
        if (p.T == 3) return mid_launch_t<YDT, TG, 3>(w, M, K, qw, scales, zeros, N, glog, y, ldy, p, st);
        return mid_launch_t<YDT, TG, 4>(w, M, K, qw, scales, zeros, N, glog, y, ldy, p, st);
      }
      return hipErrorInvalidValue;
  }
}

template <int DT, int YDT, bool HAS_R>
hipError_t mid_dispatch(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint32_t* qw,
                        const uint16_t* scales, const uint8_t* zeros, int64_t N, int glog, const float* r,
                        void* y, int64_t ldy, void* ws, hipStream_t st) {
  const MidPlan p = mid_plan(M, N, K);
  if (p.S == 0) return hipErrorInvalidValue;
  switch (p.tg) {                                // M >= 17: two to four token groups
    case 2: return mid_launch<DT, YDT, HAS_R, 2>(x, M, K, ldx, qw, scales, zeros, N, glog, r, y, ldy, p, ws, st);
    case 3: return mid_launch<DT, YDT, HAS_R, 3>(x, M, K, ldx, qw, scales, zeros, N, glog, r, y, ldy, p, ws, st);
    default: return mid_launch<DT, YDT, HAS_R, 4>(x, M, K, ldx, qw, scales, zeros, N, glog, r, y, ldy, p, ws, st);
  }
}

}  // namespace awqk

namespace awq {

bool mid_supported(int64_t M, int64_t N, int64_t K) { return awqk::mid_plan(M, N, K).S != 0; }

size_t mid_ws_bytes(int64_t M, int64_t N, int64_t K) {
  const awqk::MidPlan p = awqk::mid_plan(M, N, K);
  return p.S ? awqk::mid_ws(nullptr, M, N, K, p.S).bytes : 0;
}

hipError_t launch_mid(const void* x, int xdt, int64_t M, int64_t K, int64_t ldx, const uint32_t* qw,
                      const uint16_t* scales, const uint8_t* zeros, int64_t N, int group,
                      const float* inv_s, void* y, int ydt, int64_t ldy, void* ws, hipStream_t st) {
  using namespace awqk;
  const uint16_t* xp = (const uint16_t*)x;
  const int glog = group == 64 ? 6 : group == 128 ? 7 : group == 256 ? 8 : -1;
  if (glog < 0) return hipErrorInvalidValue;
#define AWQ_MD(XT, YT)                                                                           \
  return inv_s ? mid_dispatch<XT, YT, true>(xp, M, K, ldx, qw, scales, zeros, N, glog, inv_s, y, ldy, ws, st) \
               : mid_dispatch<XT, YT, false>(xp, M, K, ldx, qw, scales, zeros, N, glog, inv_s, y, ldy, ws, st)
  if (xdt == DT_F16) {
    if (ydt == DT_F16) AWQ_MD(DT_F16, DT_F16);
    if (ydt == DT_BF16) AWQ_MD(DT_F16, DT_BF16);
    AWQ_MD(DT_F16, DT_F32);
  }
  if (ydt == DT_F16) AWQ_MD(DT_BF16, DT_F16);
  if (ydt == DT_BF16) AWQ_MD(DT_BF16, DT_BF16);
  AWQ_MD(DT_BF16, DT_F32);
#undef AWQ_MD
}

}  // namespace awq
