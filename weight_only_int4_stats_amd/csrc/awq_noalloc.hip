// awq_w4a16_gemm_noalloc: the fused W4A16 product for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops).
// The product's scratch (the activations converted to fp16, their exponents,
// the weight rows' exponents and the dequantization constants) lives in one
// file-scope device array instead of a caller workspace.  Its device address
// is looked up once per device with hipGetSymbolAddress and kept: in host
// code the array's name is only a host-side handle, never a device address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/awq.h"
#include "awq_internal.h"

namespace {

// Every GPU the library runs on holds its own copy until the process ends.
static __device__ __align__(256) unsigned char scratch[AWQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
std::mutex g_lock;

// Device address of this device's scratch, looked up on its first use with
// that device current.
hipError_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_lock);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" awq_status awq_w4a16_gemm_noalloc(const void* x, awq_dtype xdt, int64_t M, int64_t K,
                                             int64_t ldx, const int32_t* qweight,
                                             const uint16_t* scales, const uint8_t* zeros, int64_t N,
                                             int group_size, const float* inv_s, void* y,
                                             awq_dtype ydt, int64_t ldy, void* stream) {
  if (group_size != 64 && group_size != 128 && group_size != 256) return AWQ_ERR_UNSUPPORTED;
  if ((xdt != AWQ_F16 && xdt != AWQ_BF16) || (ydt != AWQ_F16 && ydt != AWQ_BF16 && ydt != AWQ_F32))
    return AWQ_ERR_DTYPE;
  if (M < 0 || N < 0 || K <= 0 || K % group_size != 0 || ldx < K || ldy < N) return AWQ_ERR_SHAPE;
  if (M == 0 || N == 0) return AWQ_OK;
  if (!x || !qweight || !scales || !zeros || !y) return AWQ_ERR_NULL;
  if (K > AWQ_MAX_K) return AWQ_ERR_UNSUPPORTED;
  if (ldx % 8 != 0 || !aligned16(x) || !aligned16(qweight) || (inv_s && !aligned16(inv_s)))
    return AWQ_ERR_ALIGN;
  const size_t need = awq::gemm_ws_bytes(M, N, K, group_size);
  if (need > (size_t)AWQ_NOALLOC_SCRATCH_BYTES) return AWQ_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (need) {
    const hipError_t e = scratch_ptr(&ws);
    if (e != hipSuccess) return AWQ_ERR_HIP;
  }
  const hipError_t e = awq::launch_w4a16(x, (int)xdt, M, K, ldx, (const uint32_t*)qweight, scales,
                                         zeros, N, group_size, inv_s, y, (int)ydt, ldy, ws,
                                         (hipStream_t)stream);
  return e == hipSuccess ? AWQ_OK : AWQ_ERR_HIP;
}
