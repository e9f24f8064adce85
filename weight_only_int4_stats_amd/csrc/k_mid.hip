// W4A16 product for small batches, 17 <= M <= 64 ("AWQ > Benefits and
// Practical Considerations": unpack the 4-bit integers, apply the group scale
// and zero point and the optional per-channel inverse scale, fused with the
// multiply).  At these batch sizes the product is bound by the packed weight
// stream ("AWQ Math", "Weight-only quantization and where it breaks": decode
// is weight-loading bound), not by the matrix cores.
//
//   1. k_rows_f16 (pre-pass): each token row x r as fp16 with an exact power
//      of two per row, in the order the nibble unpack yields (x_q [M][K]).
//   2. k_gemm_mid: block (s, b) takes 64 weight rows and the s-th of S slices
//      of the 128-channel units.  Its slice of x_q (16 TG token rows, rows
//      past M read as zeros) is copied into LDS by LDS DMA; wave w takes
//      16-row tile w / 4 and a quarter of the slice's units, streams the packed
//      words (one 128-bit chunk per lane per unit, P units in flight) and runs
//      v_mfma_f32_16x16x32_f16 with the dequantized weights as A and each
//      16-token group as B.  The four quarters of a tile meet in LDS in a fixed
//      order; with S = 1 the result is scaled back and stored, otherwise fp32
//      partial sums go to the workspace.
//   3. k_mid_reduce (S > 1): y = sum over slices in slice order, scaled back.
// The split over K keeps each block's activation slice small when N is small
// (a 4096-row layer gives each compute unit only 16 rows, while a 32-token
// activation of 4096 channels is 256 KB), at the cost of S M N fp32 partials
// and a third launch.  The partial sums meet in a separate kernel rather than
// in the last-arriving block: each L2 slice of this chip serves its own group
// of compute units, so making one block's writes visible to blocks elsewhere
// takes a device-scope fence that writes the L2 back (measured 8x slower).
#include "awq_device.h"
#include "awq_internal.h"
#include "k_rows_f16.h"

#include <utility>

namespace awqk {

constexpr int kMidWaves = 16;
constexpr int kMidTiles = 4;                       // 16-row tiles per block (64 rows)
constexpr int kMidKsl = kMidWaves / kMidTiles;     // waves per tile (K quarters)
constexpr int kMidRows = 16 * kMidTiles;
constexpr size_t kMidLdsMax = 128 * 1024;
// Below 17 tokens the single-launch product that stages the whole activation
// in each compute unit's LDS (k_gemm_skinny_cu) is faster.
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

// TG: 16-token groups (1..4); P: units in flight per wave; SPLIT: S > 1.
// pitch: LDS bytes per staged token row (a whole number of KB plus 16, so the
// 16 rows of one 128-bit read pass fall on distinct bank slots).
template <int YDT, int TG, int P, bool SPLIT>
__global__ __launch_bounds__(1024) void k_gemm_mid(const uint16_t* __restrict__ xq,
                                                   const int* __restrict__ pm, int M, int64_t K,
                                                   const uint32_t* __restrict__ qw,
                                                   const uint16_t* __restrict__ scales,
                                                   const uint8_t* __restrict__ zeros, int64_t N,
                                                   int glog, int S, int pitch,
                                                   float* __restrict__ partial, int* __restrict__ en,
                                                   void* __restrict__ y, int64_t ldy) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_mid[];
  __shared__ int e_s[kMidRows];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rl = lane & 15;                      // A row / B token within a group
  const int b = lane >> 4;                       // 32-k block of the 128-channel unit
  const int bs = (int)(blockIdx.x % (unsigned)S);
  const int64_t n0 = (int64_t)(blockIdx.x / (unsigned)S) * kMidRows;
  const int nrows = (int)(N - n0 < kMidRows ? N - n0 : kMidRows);
  const int U = (int)(K >> 7);
  const int u0 = bs * U / S, u1 = (bs + 1) * U / S;            // U <= 1024, S <= U
  const int us = u1 - u0;
  const int tile = wv / kMidKsl, ks = wv % kMidKsl;
  const int w0 = u0 + ks * us / kMidKsl, w1 = u0 + (ks + 1) * us / kMidKsl;
  const int row = tile * 16 + rl;                // this lane's weight row in the block
  const bool rowok = row < nrows;
  const int GW = (int)(K >> glog);               // weight groups per row
  const int csh = glog - 5;                      // 32-code chunk -> weight group
  const uint32_t KW = (uint32_t)(K >> 3);

  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(qw + n0 * KW), (short)0, nrows * (int)KW * 4, kBufferWord3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(scales + n0 * GW), (short)0, nrows * GW * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(zeros + n0 * GW), (short)0, nrows * GW, kBufferWord3);

  // ---- 1. this block's slice of the activations into LDS (rows >= M: 0)
  {
    const i32x4 xrs = rsrc4(xq, (uint32_t)((int64_t)M * K * 2));
    const int per_row = (us * 256 + 1023) / 1024;              // 1 KB copies per token row
    const uint32_t lbase = __builtin_amdgcn_readfirstlane(lds_addr(lds_mid));
    for (int j = wv; j < 16 * TG * per_row; j += kMidWaves) {  // wave-uniform
      const int m = j / per_row, i = j - m * per_row;
      dma16(xrs, lbase + (uint32_t)(m * pitch + i * 1024), (uint32_t)(i * 1024 + lane * 16),
            (uint32_t)((int64_t)m * K * 2 + (int64_t)u0 * 256));
    }
  }
  // ---- 2. the row's steps (for its power of two), then the first P units
  const int npc = (GW * 2 + 15) / 16;            // 16-byte pieces of a row's steps
  auto load_piece = [&](int pc) {
    return __builtin_amdgcn_raw_buffer_load_b128(
        srs, rowok && pc < npc ? (uint32_t)row * GW * 2 + 16 * pc : kBufferOob, 0, 0);
  };
  const u32x4 sp0 = load_piece(b);
  u32x4 wa[P];
  uint32_t sr[P], zr[P];
  auto load_unit = [&](int slot, int u) {
    const bool ok = rowok && u < w1;
    const uint32_t gw = (uint32_t)(row * GW + ((4 * u + b) >> csh));
    wa[slot] = __builtin_amdgcn_raw_buffer_load_b128(
        wrs, ok ? (uint32_t)row * KW * 4 + (uint32_t)(4 * u + b) * 16 : kBufferOob, 0, kBufferNt);
    sr[slot] = __builtin_amdgcn_raw_buffer_load_b16(srs, ok ? gw * 2 : kBufferOob, 0, 0);
    zr[slot] = __builtin_amdgcn_raw_buffer_load_b8(zrs, ok ? gw : kBufferOob, 0, 0);
  };
#pragma unroll
  for (int d = 0; d < P; ++d) load_unit(d, w0 + d);

  // ---- 3. per-row power of two e (max step 2^e in [2^-10, 2^-9)) from all of
  // the row's steps: the same for every slice, so partial sums share a scale
  auto piece_max = [&](const u32x4& v, int pc, float mx) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (pc * 8 + j < GW) mx = fmaxf(mx, f16_to_f32((v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu));
    return mx;
  };
  float mx = piece_max(sp0, b, 0.0f);
  for (int pc = b + 4; pc < npc; pc += 4) mx = piece_max(load_piece(pc), pc, mx);
  {
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  }
  int e = 0;
  if (mx > 0.0f) {
    int ex;
    frexpf(mx, &ex);
    e = -9 - ex;
  }
  if (ks == 0 && b == 0) {
    e_s[row] = e;
    if (SPLIT && bs == 0 && rowok) en[n0 + row] = e;
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));     // the activation copies (and the first units)
  __syncthreads();

  // ---- 4. units: dequantize the lane's chunk, multiply every token group
  f32x4 acc[TG];
#pragma unroll
  for (int g = 0; g < TG; ++g) acc[g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const uint8_t* xrow = lds_mid + rl * pitch + b * 64;          // token rl, k block b
  for (int ub = w0; ub < w1; ub += P) {
#pragma unroll
    for (int d = 0; d < P; ++d) {
      const int u = ub + d;
      if (u < w1) {                                             // wave-uniform
        const float D = ldexpf(f16_to_f32(sr[d]), e);
        const uint32_t h24 = f32_to_f16_bits(D * 16777216.0f);
        const uint32_t h20 = f32_to_f16_bits(D * 1048576.0f);
        const uint32_t hz = f32_to_f16_bits(-(D * (float)zr[d]));
        const f16x2 c24 = as_f16x2(h24 | (h24 << 16));
        const f16x2 c20 = as_f16x2(h20 | (h20 << 16));
        const f16x2 nzd = as_f16x2(hz | (hz << 16));
        u32x4 a[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = mid_dequant(wa[d][i], c24, c20, nzd);
        const uint8_t* xp = xrow + (u - u0) * 256;
#pragma unroll
        for (int g = 0; g < TG; ++g) {
          u32x4 xb[4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            xb[i] = *reinterpret_cast<const u32x4*>(xp + g * 16 * pitch + i * 16);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[g] = mfma16h(a[i], xb[i], acc[g]);
        }
      }
      load_unit(d, u + P);
    }
  }

  // ---- 5. the four K quarters of each tile meet in LDS (the activation
  // area, free once every wave is done with it), in quarter order.
  // 16 x 16 layout: token = lane % 16, row = 4 (lane / 16) + v.
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds_mid);               // [16 waves][TG][16 rows][16 tokens]
#pragma unroll
  for (int g = 0; g < TG; ++g)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[((wv * TG + g) * 16 + 4 * b + v) * 16 + rl] = acc[g][v];
  __syncthreads();
  // thread t: row t % 64 of the block, token t / 64 of each group
  const int orow = tid & 63, otok = tid >> 6;
  const int ot = orow >> 4, orr = orow & 15;
  if (orow < nrows) {
    const int eo = e_s[orow];
#pragma unroll
    for (int g = 0; g < TG; ++g) {
      const int m = g * 16 + otok;
      if (m < M) {
        float tot = 0.0f;
#pragma unroll
        for (int q = 0; q < kMidKsl; ++q) tot += red[(((ot * kMidKsl + q) * TG + g) * 16 + orr) * 16 + otok];
        const int64_t n = n0 + orow;
        if constexpr (SPLIT) partial[((int64_t)bs * M + m) * N + n] = tot;
        else store_ym<YDT>(y, (int64_t)m * ldy + n, ldexpf(tot, -(pm[m] + eo)));
      }
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
  int pitch = 0;      // LDS bytes per staged token row
  size_t lds = 0;
  int64_t blocks = 0;
};

// Slices: the fewest (a power of two) that give about one block per compute
// unit and keep the activation slice within kMidLdsMax.
inline MidPlan mid_plan(int64_t M, int64_t N, int64_t K) {
  MidPlan p;
  if (M < kMidMinM || M > 64 || K % 128 != 0 || N <= 0) return p;
  const int64_t U = K / 128;
  const int64_t nbn = (N + kMidRows - 1) / kMidRows;
  const int64_t cus = awq::device_cus();
  p.tg = (int)((M + 15) / 16);
  auto lds_for = [&](int64_t S) {
    const int64_t us = (U + S - 1) / S;
    const int64_t pitch = (us * 256 + 1023) / 1024 * 1024 + 16;
    return std::pair<int64_t, size_t>(pitch, (size_t)(16 * p.tg) * pitch);
  };
  int64_t S = 1;
  while (S * nbn < cus && S * 2 <= U) S *= 2;
  while (lds_for(S).second > kMidLdsMax && S * 2 <= U) S *= 2;
  const auto pl = lds_for(S);
  if (pl.second > kMidLdsMax) return MidPlan{};
  p.S = (int)S;
  p.pitch = (int)pl.first;
  // the reduction reuses the activation area: 16 waves x TG x 1 KB
  const size_t red = (size_t)kMidWaves * p.tg * 1024;
  p.lds = pl.second > red ? pl.second : red;
  p.blocks = S * nbn;
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

template <int DT, int YDT, bool HAS_R, int TG>
hipError_t mid_launch(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint32_t* qw,
                      const uint16_t* scales, const uint8_t* zeros, int64_t N, int glog, const float* r,
                      void* y, int64_t ldy, const MidPlan& p, void* ws, hipStream_t st) {
  const MidWs w = mid_ws(ws, M, N, K, p.S);
  hipLaunchKernelGGL((k_rows_f16<DT, HAS_R, true>), dim3((unsigned)M), dim3(256), 0, st, x, K, ldx, r,
                     w.xq, w.pm);
  constexpr int P = 4;
  if (p.S == 1) {
    hipLaunchKernelGGL((k_gemm_mid<YDT, TG, P, false>), dim3((unsigned)p.blocks), dim3(1024), p.lds, st,
                       w.xq, w.pm, (int)M, K, qw, scales, zeros, N, glog, p.S, p.pitch, w.partial, w.en,
                       y, ldy);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_gemm_mid<YDT, TG, P, true>), dim3((unsigned)p.blocks), dim3(1024), p.lds, st,
                     w.xq, w.pm, (int)M, K, qw, scales, zeros, N, glog, p.S, p.pitch, w.partial, w.en, y,
                     ldy);
  hipLaunchKernelGGL((k_mid_reduce<YDT>), dim3((unsigned)((M * N + 255) / 256)), dim3(256), 0, st,
                     w.partial, p.S, (int)M, N, w.pm, w.en, y, ldy);
  return hipGetLastError();
}

template <int DT, int YDT, bool HAS_R>
hipError_t mid_dispatch(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint32_t* qw,
                        const uint16_t* scales, const uint8_t* zeros, int64_t N, int glog, const float* r,
                        void* y, int64_t ldy, void* ws, hipStream_t st) {
  const MidPlan p = mid_plan(M, N, K);
  if (p.S == 0) return hipErrorInvalidValue;
  switch (p.tg) {
    case 1: return mid_launch<DT, YDT, HAS_R, 1>(x, M, K, ldx, qw, scales, zeros, N, glog, r, y, ldy, p, ws, st);
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
