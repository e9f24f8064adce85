// Calibration statistic: mean |x_j| over the calibration tokens, per input
// channel ("AWQ Math", section "Saliency is an activation property, not a
// weight property"; "AWQ > Limitations": the saliency metric is the average
// activation magnitude over a calibration set).
//
// The column sums are exact.  Each |x| is taken in fixed point with LSB 2^-24
// (floor(|x| * 2^24), exact for every fp16 value) and summed per thread in
// double: every term and partial sum is an integer number of 2^-24 units below
// 2^53 under the precondition (column sums below 2^29), so the double sums are
// exact and equal to the integer ones.  Integer sums built from the 16-bit
// patterns (the significand shifted by the exponent, 64-bit adds) were the
// slower path: 79 against 35 us on 2048 x 28672 bf16; for fp16 the double
// path needs only a conversion and an add per value.
// Across the block the sums are 64-bit integers; each row range writes its
// column sums to a slot of its own in the workspace (no atomics, nothing to
// clear first), and the finalisation adds a column's slots in 64-bit integers
// (exact and order-free), divides once in double and rounds once to float,
// so the result does not depend on the grid.  The calibration rows are read
// with non-temporal loads: each is read once.
//
// Layout: X is [T][ldx] row-major.  A thread owns 8 consecutive columns (one
// 128-bit load per row); a wave covers 512 columns of a row, the four waves of
// a block take interleaved rows of the block's row range.
#include "awq_device.h"
#include "awq_internal.h"

namespace awqk {

typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));

constexpr int kStatsThreads = 256;
constexpr int kStatsCols = 512;      // columns per block (64 lanes x 8)
constexpr int kStatsUnroll = 16;     // rows per wave per loop trip (loads in flight)


// Per thread, per column, in double, exactly:
//   fp16: sum of |x| (every fp16 value is a multiple of 2^-24 below 2^16, so
//         each partial sum is an integer multiple of 2^-24; times 2^24 it is
//         the integer fixed-point sum, scaled once at the end);
//   bf16: sum of floor(|x| 2^24) (values below 2^-24 floor away).
// Under the precondition (column sums below 2^29) every partial sum is below
// 2^53 units of 2^-24, so the double sums are exact and equal to the integer
// sums of floor(|x| 2^24).
template <int DT>
__device__ __forceinline__ void accum_word(uint32_t w, double& a, double& b) {
  if constexpr (DT == DT_F16) {
    a += (double)f16_to_f32(w & 0x7FFFu);
    b += (double)f16_to_f32((w >> 16) & 0x7FFFu);
  } else {
    a += floor((double)fabsf(bf16_to_f32(w & 0xFFFFu)) * 16777216.0);   // exact: power-of-two scale
    b += floor((double)fabsf(bf16_to_f32(w >> 16)) * 16777216.0);
  }
}

template <int DT>
__global__ __launch_bounds__(kStatsThreads) void k_act_accum(const uint16_t* __restrict__ x,
                                                             int64_t T, int64_t K, int64_t ldx,
                                                             int64_t rows_per_block, int64_t slabs,
                                                             int64_t chunks,
                                                             unsigned long long* __restrict__ part) {
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
  double s[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) s[j] = 0.0;

  if (col < K) {
    const uint16_t* base = x + col;
    int64_t r = r0 + wv;
    // main trips: kStatsUnroll rows per wave, loads issued before use
    for (; r + 4 * (kStatsUnroll - 1) < r1; r += 4 * kStatsUnroll) {
      u32x4 v[kStatsUnroll];
#pragma unroll
      for (int u = 0; u < kStatsUnroll; ++u) v[u] = ldg128_stream(base + (r + 4 * u) * ldx);
#pragma unroll
      for (int u = 0; u < kStatsUnroll; ++u) {
        accum_word<DT>(v[u][0], s[0], s[1]);
        accum_word<DT>(v[u][1], s[2], s[3]);
        accum_word<DT>(v[u][2], s[4], s[5]);
        accum_word<DT>(v[u][3], s[6], s[7]);
      }
    }
    for (; r < r1; r += 4) {
      u32x4 v = ldg128_stream(base + r * ldx);
      accum_word<DT>(v[0], s[0], s[1]);
      accum_word<DT>(v[1], s[2], s[3]);
      accum_word<DT>(v[2], s[4], s[5]);
      accum_word<DT>(v[3], s[6], s[7]);
    }
  }

  __shared__ uint64_t red[4][8][64];
#pragma unroll
  for (int j = 0; j < 8; ++j)    // an integer below 2^53 (the fp16 sums in units of 2^-24)
    red[wv][j][lane] = (uint64_t)(DT == DT_F16 ? s[j] * 16777216.0 : s[j]);
  __syncthreads();
  if (wv == 0 && col < K) {
    // this row range's column sums, one slot per range (no atomics, nothing to clear)
    u64x2 o[4];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      o[j >> 1][j & 1] = red[0][j][lane] + red[1][j][lane] + red[2][j][lane] + red[3][j][lane];
    u64x2* dst = reinterpret_cast<u64x2*>(part + chunk * K + col);
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[i] = o[i];
  }
}

// Column j: the row ranges' integer sums added (exact, any order), then one
// double division and one float rounding.  A block takes 64 columns; its four
// waves take every fourth row range, eight loads in flight per lane.
__global__ __launch_bounds__(256) void k_act_finalize(const unsigned long long* __restrict__ part,
                                                      int64_t chunks, int64_t K, int64_t T,
                                                      float* __restrict__ mean_abs) {
  __shared__ unsigned long long red[4][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t j = (int64_t)blockIdx.x * 64 + lane;
  unsigned long long acc = 0;
  if (j < K) {
    int64_t c = wv;
    for (; c + 4 * 7 < chunks; c += 4 * 8) {
      unsigned long long v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[(c + 4 * u) * K + j];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; c < chunks; c += 4) acc += part[c * K + j];
  }
  red[wv][lane] = acc;
  __syncthreads();
  if (wv == 0 && j < K) {
    acc = red[0][lane] + red[1][lane] + red[2][lane] + red[3][lane];
    const double sum = (double)acc * 0x1p-24;       // exact: acc < 2^53
    mean_abs[j] = (float)(sum / (double)T);         // one double rounding, one float rounding
  }
}

}  // namespace awqk

namespace awq {

// at most ceil(1024 / slabs) row ranges (stats_chunks), each a uint64 per column
size_t act_stats_ws_bytes(int64_t K) {
  const int64_t slabs = (K + awqk::kStatsCols - 1) / awqk::kStatsCols;
  return align_up((size_t)((1024 + slabs - 1) / slabs) * (size_t)K * 8, 256);
}

hipError_t launch_act_stats(const void* x, int dt, int64_t T, int64_t K, int64_t ldx,
                            float* mean_abs, void* ws, hipStream_t st) {
  using namespace awqk;
  unsigned long long* part = reinterpret_cast<unsigned long long*>(ws);
  const int64_t slabs = (K + kStatsCols - 1) / kStatsCols;
  // about 1024 blocks (four per compute unit), each row range a multiple of
  // 4 rows x unroll: longer row ranges mean fewer partial sums per column
  // (4096 blocks measured 125 against 108 us on 65536 x 4096)
  int64_t chunks = (1024 + slabs - 1) / slabs;
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
                       (const uint16_t*)x, T, K, ldx, rpb, slabs, chunks, part);
  else
    hipLaunchKernelGGL(k_act_accum<DT_BF16>, grid, dim3(kStatsThreads), 0, st,
                       (const uint16_t*)x, T, K, ldx, rpb, slabs, chunks, part);
  hipLaunchKernelGGL(k_act_finalize, dim3((unsigned)((K + 63) / 64)), dim3(256), 0, st, part, chunks, K, T,
                     mean_abs);
  return hipGetLastError();
}

}  // namespace awq
