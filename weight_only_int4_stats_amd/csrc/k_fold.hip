// Folding the activation scaling into the operation that produces x ("AWQ
// Math", section "The equivalent transform: scale up W, scale down x": the
// division of x_j by s_j moves backward into the preceding LayerNorm or
// linear, so that the product runs without the per-channel 1/s).
//   axis 1: v[i][j] <- dt(float(v[i][j]) / s[j])
//   axis 0: v[i][j] <- dt(float(v[i][j]) / s[i])
// IEEE binary32 division, round-to-nearest-even to dt.  Elementwise and
// memory bound: consecutive threads take consecutive columns of a row.
#include "awq_device.h"
#include "awq_internal.h"

namespace awqk {

template <int DT>
__device__ __forceinline__ float fold_load(const void* v, int64_t i) {
  if constexpr (DT == DT_F32) return reinterpret_cast<const float*>(v)[i];
  else if constexpr (DT == DT_F16) return f16_to_f32(reinterpret_cast<const uint16_t*>(v)[i]);
  else return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(v)[i] << 16);
}

template <int DT>
__device__ __forceinline__ void fold_store(void* v, int64_t i, float f) {
  if constexpr (DT == DT_F32) reinterpret_cast<float*>(v)[i] = f;
  else reinterpret_cast<uint16_t*>(v)[i] = (uint16_t)from_f32<DT>(f);
}

template <int DT>
__global__ __launch_bounds__(256) void k_fold_scales(void* __restrict__ v, int64_t rows, int64_t cols,
                                                     int64_t ld, const float* __restrict__ s, int axis) {
  const int64_t n = rows * cols;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int64_t i = e / cols, j = e - i * cols;
    const int64_t at = i * ld + j;
    fold_store<DT>(v, at, fold_load<DT>(v, at) / s[axis ? j : i]);
  }
}

}  // namespace awqk

namespace awq {

hipError_t launch_fold_scales(void* v, int dt, int64_t rows, int64_t cols, int64_t ld, const float* s,
                              int axis, hipStream_t st) {
  using namespace awqk;
  const int64_t n = rows * cols;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  const dim3 grid((unsigned)blocks), block(256);
  if (dt == DT_F16) hipLaunchKernelGGL(k_fold_scales<DT_F16>, grid, block, 0, st, v, rows, cols, ld, s, axis);
  else if (dt == DT_BF16) hipLaunchKernelGGL(k_fold_scales<DT_BF16>, grid, block, 0, st, v, rows, cols, ld, s, axis);
  else hipLaunchKernelGGL(k_fold_scales<DT_F32>, grid, block, 0, st, v, rows, cols, ld, s, axis);
  return hipGetLastError();
}

}  // namespace awq
