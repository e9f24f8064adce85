// Calibration statistic: mean |x_j| over the calibration tokens, per input
// channel ("AWQ Math", section "Saliency is an activation property, not a
// weight property"; "AWQ > Limitations": the saliency metric is the average
// activation magnitude over a calibration set).
//
// The column sums are exact.  Each |x| is taken in fixed point with LSB 2^-24
// (floor(|x| * 2^24), exact for every fp16 value), built from the 16-bit
// pattern with integer operations (the significand shifted by the exponent),
// accumulated per thread and across the block in 64-bit integers, and added
// across blocks with 64-bit integer atomics (exact and order-free).  The finalisation divides once in double
// and rounds once to float, so the result does not depend on the grid.
//
// Layout: X is [T][ldx] row-major.  A thread owns 8 consecutive columns (one
// 128-bit load per row); a wave covers 512 columns of a row, the four waves of
// a block take interleaved rows of the block's row range.
#include "awq_device.h"
#include "awq_internal.h"

namespace awqk {

constexpr int kStatsThreads = 256;
constexpr int kStatsCols = 512;      // columns per block (64 lanes x 8)
constexpr int kStatsUnroll = 16;     // rows per wave per loop trip (loads in flight)

__global__ void k_fill_u64(unsigned long long* p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

// floor(|x| 2^24) of one 16-bit value, as an integer.  fp16: a subnormal is
// m 2^-24 -> m; a normal (1024 + m) 2^(e - 25) -> (1024 + m) 2^(e - 1).  bf16:
// (128 + m) 2^(e - 134) -> (128 + m) 2^(e - 110), shifted right (the floor)
// below 2^24 and 0 for subnormals.  Shifts are capped at 40: values that large
// already break the statistic's range (sum below 2^29).
template <int DT>
__device__ __forceinline__ uint64_t fixed24(uint32_t h) {
  if constexpr (DT == DT_F16) {
    const uint32_t e = (h >> 10) & 0x1Fu, m = h & 0x3FFu;
    return e ? (uint64_t)(1024u | m) << (e - 1) : (uint64_t)m;
  } else {
    const int e = (int)((h >> 7) & 0xFFu);
    const uint32_t m = (h & 0x7Fu) | 0x80u;
    const int sh = e - 110;
    if (e == 0 || sh <= -8) return 0;
    return sh >= 0 ? (uint64_t)m << (sh < 40 ? sh : 40) : (uint64_t)(m >> -sh);
  }
}

template <int DT>
__device__ __forceinline__ void accum_word(uint32_t w, uint64_t& a, uint64_t& b) {
  a += fixed24<DT>(w & 0xFFFFu);
  b += fixed24<DT>(w >> 16);
}

template <int DT>
__global__ __launch_bounds__(kStatsThreads) void k_act_accum(const uint16_t* __restrict__ x,
                                                             int64_t T, int64_t K, int64_t ldx,
                                                             int64_t rows_per_block, int64_t slabs,
                                                             int64_t chunks,
                                                             unsigned long long* __restrict__ acc) {
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  // Block i runs on L2 slice i mod 8; slice x takes chunks x, x + 8, ... with
  // all column slabs of a chunk back to back, so each slice reads whole rows.
  const int64_t bi = blockIdx.x;
  const int64_t xs = bi % 8, slot = bi / 8;
  const int64_t slab = slot % slabs;
  const int64_t chunk = (slot / slabs) * 8 + xs;
  if (chunk >= chunks) return;
  const int64_t col = slab * kStatsCols + lane * 8;
  const int64_t r0 = chunk * rows_per_block;
  const int64_t r1 = min(T, r0 + rows_per_block);
  uint64_t s[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) s[j] = 0;

  if (col < K) {
    const uint16_t* base = x + col;
    int64_t r = r0 + wv;
    // main trips: kStatsUnroll rows per wave, loads issued before use
    for (; r + 4 * (kStatsUnroll - 1) < r1; r += 4 * kStatsUnroll) {
      u32x4 v[kStatsUnroll];
#pragma unroll
      for (int u = 0; u < kStatsUnroll; ++u) v[u] = ldg128(base + (r + 4 * u) * ldx);
#pragma unroll
      for (int u = 0; u < kStatsUnroll; ++u) {
        accum_word<DT>(v[u][0], s[0], s[1]);
        accum_word<DT>(v[u][1], s[2], s[3]);
        accum_word<DT>(v[u][2], s[4], s[5]);
        accum_word<DT>(v[u][3], s[6], s[7]);
      }
    }
    for (; r < r1; r += 4) {
      u32x4 v = ldg128(base + r * ldx);
      accum_word<DT>(v[0], s[0], s[1]);
      accum_word<DT>(v[1], s[2], s[3]);
      accum_word<DT>(v[2], s[4], s[5]);
      accum_word<DT>(v[3], s[6], s[7]);
    }
  }

  __shared__ uint64_t red[4][8][64];
#pragma unroll
  for (int j = 0; j < 8; ++j) red[wv][j][lane] = s[j];
  __syncthreads();
  if (wv == 0 && col < K) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint64_t t = red[0][j][lane] + red[1][j][lane] + red[2][j][lane] + red[3][j][lane];
      if (t != 0) atomicAdd(&acc[col + j], (unsigned long long)t);
    }
  }
}

__global__ void k_act_finalize(const unsigned long long* __restrict__ acc, int64_t K, int64_t T,
                               float* __restrict__ mean_abs) {
  int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j < K) {
    const double sum = (double)acc[j] * 0x1p-24;    // exact: acc < 2^53
    mean_abs[j] = (float)(sum / (double)T);        // one double rounding, one float rounding
  }
}

}  // namespace awqk

namespace awq {

size_t act_stats_ws_bytes(int64_t K) { return align_up((size_t)K * 8, 256); }

hipError_t launch_act_stats(const void* x, int dt, int64_t T, int64_t K, int64_t ldx,
                            float* mean_abs, void* ws, hipStream_t st) {
  using namespace awqk;
  unsigned long long* acc = reinterpret_cast<unsigned long long*>(ws);
  hipLaunchKernelGGL(k_fill_u64, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st, acc, K);
  const int64_t slabs = (K + kStatsCols - 1) / kStatsCols;
  // about 4096 blocks, each row range a multiple of 4 rows x unroll
  int64_t chunks = (4096 + slabs - 1) / slabs;
  const int64_t quantum = 4 * kStatsUnroll;
  const int64_t max_chunks = (T + quantum - 1) / quantum;
  if (chunks > max_chunks) chunks = max_chunks;
  if (chunks > 65535) chunks = 65535;
  if (chunks < 1) chunks = 1;
  int64_t rpb = (T + chunks - 1) / chunks;
  rpb = (rpb + quantum - 1) / quantum * quantum;
  chunks = (T + rpb - 1) / rpb;
  // chunks rounded up to a multiple of 8 slices; blocks past the last chunk exit
  const dim3 grid((unsigned)(slabs * ((chunks + 7) / 8) * 8));
  if (dt == DT_F16)
    hipLaunchKernelGGL(k_act_accum<DT_F16>, grid, dim3(kStatsThreads), 0, st,
                       (const uint16_t*)x, T, K, ldx, rpb, slabs, chunks, acc);
  else
    hipLaunchKernelGGL(k_act_accum<DT_BF16>, grid, dim3(kStatsThreads), 0, st,
                       (const uint16_t*)x, T, K, ldx, rpb, slabs, chunks, acc);
  hipLaunchKernelGGL(k_act_finalize, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st, acc, K,
                     T, mean_abs);
  return hipGetLastError();
}

}  // namespace awq
