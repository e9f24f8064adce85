// C ABI of the AWQ hot path: argument validation on the host, then the
// kernel launchers.  Nothing here allocates device memory or keeps state.
#include <hip/hip_runtime.h>

#include "../../include/awq.h"
#include "awq_internal.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned256(const void* p) { return ((uintptr_t)p & 255u) == 0; }
bool is_act_dtype(awq_dtype d) { return d == AWQ_F16 || d == AWQ_BF16; }
bool is_out_dtype(awq_dtype d) { return d == AWQ_F16 || d == AWQ_BF16 || d == AWQ_F32; }

awq_status from_hip(hipError_t e) { return e == hipSuccess ? AWQ_OK : AWQ_ERR_HIP; }

bool group_ok(int g) { return g == 64 || g == 128 || g == 256; }
bool grid_ok(int bits, int symmetric) {
  return (symmetric == 0 && bits >= 2 && bits <= 8) || (symmetric == 1 && bits >= 2 && bits <= 7);
}

}  // namespace

extern "C" {

int awq_abi_version(void) { return 6; }

const char* awq_status_str(awq_status st) {
  switch (st) {
    case AWQ_OK: return "ok";
    case AWQ_ERR_NULL: return "required pointer is NULL";
    case AWQ_ERR_SHAPE: return "invalid shape (sizes, K % group, leading dimension)";
    case AWQ_ERR_DTYPE: return "element type not accepted";
    case AWQ_ERR_ALIGN: return "pointer not 16-byte aligned or leading dimension not a multiple of 8";
    case AWQ_ERR_UNSUPPORTED: return "unsupported parameter (group size, bits, candidate count, K)";
    case AWQ_ERR_WORKSPACE: return "workspace missing or too small";
    case AWQ_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

size_t awq_workspace_bytes(awq_op op, int64_t M, int64_t N, int64_t K, int64_t T, int n_alpha) {
  if (N < 0 || K < 0 || T < 0 || M < 0) return 0;
  switch (op) {
    case AWQ_OP_ACT_STATS: return awq::act_stats_ws_bytes(K);
    case AWQ_OP_SEARCH:  // the larger of the fp16 and bf16 layouts
      return awq::search_ws_bytes((int)AWQ_BF16, N, K, T, n_alpha < 1 ? 1 : n_alpha);
    case AWQ_OP_QUANTIZE: return 0;
    case AWQ_OP_GEMM: return awq::gemm_ws_bytes(M, N, K, 64);   // the smallest group needs the most
  }
  return 0;
}

awq_status awq_act_stats(const void* x, awq_dtype xdt, int64_t T, int64_t K, int64_t ldx,
                         float* mean_abs, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !mean_abs) return AWQ_ERR_NULL;
  if (!is_act_dtype(xdt)) return AWQ_ERR_DTYPE;
  if (T <= 0 || K <= 0 || ldx < K) return AWQ_ERR_SHAPE;
  if (K % 8 != 0 || ldx % 8 != 0 || !aligned16(x)) return AWQ_ERR_ALIGN;
  if (K > AWQ_MAX_K) return AWQ_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < awq::act_stats_ws_bytes(K) || !aligned256(ws)) return AWQ_ERR_WORKSPACE;
  return from_hip(awq::launch_act_stats(x, (int)xdt, T, K, ldx, mean_abs, ws, (hipStream_t)stream));
}

awq_status awq_search_scales_ex(const void* w, awq_dtype dt, int64_t N, int64_t K,
                                const void* x_calib, int64_t T, int64_t ldx,
                                const float* mean_abs, const double* alphas, int n_alpha,
                                int group_size, int bits, int symmetric, const uint8_t* kept,
                                float* s_out, float* inv_s_out, double* loss_out,
                                int32_t* best_idx_out, void* ws, size_t ws_bytes, void* stream) {
  if (!w || !x_calib || !mean_abs || !alphas || !s_out) return AWQ_ERR_NULL;
  if (!is_act_dtype(dt)) return AWQ_ERR_DTYPE;
  if (!group_ok(group_size) || !grid_ok(bits, symmetric)) return AWQ_ERR_UNSUPPORTED;
  if (n_alpha < 1 || n_alpha > AWQ_MAX_ALPHA) return AWQ_ERR_UNSUPPORTED;
  // K also whole 128-channel units: the error contraction runs 4 stages of 32 at a time
  if (N <= 0 || K <= 0 || T <= 0 || ldx < K || K % group_size != 0 || K % 128 != 0)
    return AWQ_ERR_SHAPE;
  if (K > AWQ_MAX_K || N > 0x7FFFFFFF || ldx > AWQ_MAX_LDX_SEARCH) return AWQ_ERR_UNSUPPORTED;
  if (ldx % 8 != 0 || !aligned16(w) || !aligned16(x_calib) || !aligned16(mean_abs) ||
      (kept && !aligned16(kept)))
    return AWQ_ERR_ALIGN;
  if (!ws || ws_bytes < awq::search_ws_bytes((int)dt, N, K, T, n_alpha) || !aligned256(ws))
    return AWQ_ERR_WORKSPACE;
  awq::QuantVariant qv;
  qv.group = group_size;
  qv.bits = bits;
  qv.sym = symmetric != 0;
  return from_hip(awq::launch_search(w, (int)dt, N, K, x_calib, T, ldx, mean_abs, alphas, n_alpha,
                                     qv, kept, s_out, inv_s_out, loss_out, best_idx_out, ws,
                                     (hipStream_t)stream));
}

awq_status awq_search_scales(const void* w, awq_dtype dt, int64_t N, int64_t K,
                             const void* x_calib, int64_t T, int64_t ldx,
                             const float* mean_abs, const double* alphas, int n_alpha,
                             int group_size, float* s_out, float* inv_s_out, double* loss_out,
                             int32_t* best_idx_out, void* ws, size_t ws_bytes, void* stream) {
  return awq_search_scales_ex(w, dt, N, K, x_calib, T, ldx, mean_abs, alphas, n_alpha, group_size,
                              4, 0, nullptr, s_out, inv_s_out, loss_out, best_idx_out, ws, ws_bytes,
                              stream);
}

awq_status awq_salient_channels(const float* mean_abs, int64_t K, int64_t n_keep, uint8_t* kept,
                                void* stream) {
  if (K <= 0 || n_keep < 0 || n_keep > K) return AWQ_ERR_SHAPE;
  if (!mean_abs || !kept) return AWQ_ERR_NULL;
  if (K > AWQ_MAX_K) return AWQ_ERR_UNSUPPORTED;
  if (((uintptr_t)mean_abs & 3u) != 0) return AWQ_ERR_ALIGN;
  return from_hip(awq::launch_salient_channels(mean_abs, K, n_keep, kept, (hipStream_t)stream));
}

awq_status awq_quantize_pack(const void* w, awq_dtype dt, int64_t N, int64_t K, const float* s,
                             int group_size, int32_t* qweight, uint16_t* scales, uint8_t* zeros,
                             float* scales_f32_dbg, void* stream) {
  if (!group_ok(group_size)) return AWQ_ERR_UNSUPPORTED;
  if (!is_act_dtype(dt)) return AWQ_ERR_DTYPE;
  if (N < 0 || K <= 0 || K % group_size != 0) return AWQ_ERR_SHAPE;
  if (N == 0) return AWQ_OK;
  if (!w || !qweight || !scales || !zeros) return AWQ_ERR_NULL;
  if (K > AWQ_MAX_K) return AWQ_ERR_UNSUPPORTED;
  if (!aligned16(w) || !aligned16(qweight) || (s && !aligned16(s))) return AWQ_ERR_ALIGN;
  return from_hip(awq::launch_quantize_pack(w, (int)dt, N, K, s, group_size, (uint32_t*)qweight, scales,
                                            zeros, scales_f32_dbg, (hipStream_t)stream));
}

awq_status awq_quantize_codes(const void* w, awq_dtype dt, int64_t N, int64_t K, const float* s,
                              int group_size, int bits, int symmetric, uint8_t* codes,
                              uint16_t* scales, uint8_t* zeros, void* stream) {
  if (!group_ok(group_size) || !grid_ok(bits, symmetric)) return AWQ_ERR_UNSUPPORTED;
  if (!is_act_dtype(dt)) return AWQ_ERR_DTYPE;
  if (N < 0 || K <= 0 || K % group_size != 0) return AWQ_ERR_SHAPE;
  if (N == 0) return AWQ_OK;
  if (!w || !codes || !scales || !zeros) return AWQ_ERR_NULL;
  if (K > AWQ_MAX_K) return AWQ_ERR_UNSUPPORTED;
  if (!aligned16(w) || !aligned16(codes) || (s && !aligned16(s))) return AWQ_ERR_ALIGN;
  awq::QuantVariant qv;
  qv.group = group_size;
  qv.bits = bits;
  qv.sym = symmetric != 0;
  return from_hip(awq::launch_quantize_codes(w, (int)dt, N, K, s, qv, codes, scales, zeros,
                                             (hipStream_t)stream));
}

awq_status awq_w4a16_gemm(const void* x, awq_dtype xdt, int64_t M, int64_t K, int64_t ldx,
                          const int32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                          int64_t N, int group_size, const float* inv_s, void* y, awq_dtype ydt,
                          int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  if (!group_ok(group_size)) return AWQ_ERR_UNSUPPORTED;
  if (!is_act_dtype(xdt) || !is_out_dtype(ydt)) return AWQ_ERR_DTYPE;
  if (M < 0 || N < 0 || K <= 0 || K % group_size != 0 || ldx < K || ldy < N) return AWQ_ERR_SHAPE;
  if (M == 0 || N == 0) return AWQ_OK;
  if (!x || !qweight || !scales || !zeros || !y) return AWQ_ERR_NULL;
  if (K > AWQ_MAX_K) return AWQ_ERR_UNSUPPORTED;
  if (ldx % 8 != 0 || !aligned16(x) || !aligned16(qweight) || (inv_s && !aligned16(inv_s)))
    return AWQ_ERR_ALIGN;
  const size_t need = awq::gemm_ws_bytes(M, N, K, group_size);
  if (need && (!ws || ws_bytes < need || !aligned256(ws))) return AWQ_ERR_WORKSPACE;
  return from_hip(awq::launch_w4a16(x, (int)xdt, M, K, ldx, (const uint32_t*)qweight, scales,
                                    zeros, N, group_size, inv_s, y, (int)ydt, ldy, ws,
                                    (hipStream_t)stream));
}

awq_status awq_fold_scales(void* v, awq_dtype dt, int64_t rows, int64_t cols, int64_t ld, const float* s,
                           int axis, void* stream) {
  if (dt != AWQ_F16 && dt != AWQ_BF16 && dt != AWQ_F32) return AWQ_ERR_DTYPE;
  if (rows < 0 || cols < 0 || ld < cols || (axis != 0 && axis != 1)) return AWQ_ERR_SHAPE;
  if (rows == 0 || cols == 0) return AWQ_OK;
  if (!v || !s) return AWQ_ERR_NULL;
  const uintptr_t el = dt == AWQ_F32 ? 4u : 2u;
  if (((uintptr_t)v & (el - 1)) != 0 || ((uintptr_t)s & 3u) != 0) return AWQ_ERR_ALIGN;
  return from_hip(awq::launch_fold_scales(v, (int)dt, rows, cols, ld, s, axis, (hipStream_t)stream));
}

}  // extern "C"

extern "C" awq_status awq_read_stream(const void* p, int64_t bytes, int blocks, int unroll,
                                      uint32_t* block_xor, void* stream) {
  if (!p || !block_xor) return AWQ_ERR_NULL;
  if (bytes <= 0 || bytes % 1024 != 0 || blocks < 1 || blocks > 65535) return AWQ_ERR_SHAPE;
  if (unroll != 1 && unroll != 2 && unroll != 4 && unroll != 8) return AWQ_ERR_UNSUPPORTED;
  if (!aligned16(p)) return AWQ_ERR_ALIGN;
  return from_hip(awq::launch_read_stream(p, bytes, blocks, unroll, block_xor, (hipStream_t)stream));
}
