// Host-side launchers of the gfx950 kernels (one translation unit each).
// Every launcher enqueues on `st` and returns hipGetLastError() of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace awq {

// Quantizer variant: input channels per group (64, 128, 256), bits per code,
// and the grid (asymmetric with a zero point, or symmetric max|w| / 2^(N-1)).
struct QuantVariant {
  int group = 128;
  int bits = 4;
  bool sym = false;
};

// ---- calibration statistic (mean |x|) -------------------------------------
size_t act_stats_ws_bytes(int64_t K);
hipError_t launch_act_stats(const void* x, int dt, int64_t T, int64_t K, int64_t ldx,
                            float* mean_abs, void* ws, hipStream_t st);

// ---- quantize + pack --------------------------------------------------------
hipError_t launch_quantize_pack(const void* w, int dt, int64_t N, int64_t K, const float* s, int group,
                                uint32_t* qw, uint16_t* scales, uint8_t* zeros, float* dbg,
                                hipStream_t st);
hipError_t launch_quantize_codes(const void* w, int dt, int64_t N, int64_t K, const float* s,
                                 QuantVariant qv, uint8_t* codes, uint16_t* scales, uint8_t* zeros,
                                 hipStream_t st);

// ---- scale search -----------------------------------------------------------
size_t search_ws_bytes(int dt, int64_t N, int64_t K, int64_t T, int n_alpha);
hipError_t launch_search(const void* w, int dt, int64_t N, int64_t K, const void* x, int64_t T,
                         int64_t ldx, const float* mean_abs, const double* alphas, int n_alpha,
                         QuantVariant qv, const uint8_t* kept, float* s_out, float* inv_s_out,
                         double* loss_out, int32_t* best_out, void* ws, hipStream_t st);

// ---- mixed-precision baseline: the n most salient channels (k_salient.hip) ---
hipError_t launch_salient_channels(const float* mean_abs, int64_t K, int64_t n_keep, uint8_t* kept,
                                   hipStream_t st);

// Gram form of the search loss (k_gram.hip): Xt [K][Tp] 16-bit, fp32 partial
// tiles of G (gram_partial_floats), G [K][K] fp64, P [K][2 Kp] fp16 (Kp = K
// rounded up to 256; per 256-wide block the high then the low parts of each
// row of G scaled by 2^-sk[k]).
int64_t gram_tokens_padded(int64_t T);
int64_t gram_loss_tiles(int64_t N, int64_t K);
int64_t gram_partial_floats(int64_t T, int64_t K);
hipError_t launch_gram_prepare(const void* x, int dt, int64_t T, int64_t K, int64_t ldx,
                               uint16_t* Xt, float* Gp, double* G, uint16_t* P, int* sk,
                               hipStream_t st);
hipError_t launch_gram_loss(const uint16_t* E, int64_t N, int64_t K, const int* pexp,
                            const uint16_t* P, const int* sk, double* partial, int nc,
                            hipStream_t st);

// ---- folding 1/s into the producer of x (k_fold.hip) ---------------------------
hipError_t launch_fold_scales(void* v, int dt, int64_t rows, int64_t cols, int64_t ld, const float* s,
                              int axis, hipStream_t st);

// ---- W4A16 product ----------------------------------------------------------
// group: input channels per step / zero point (64, 128 or 256)
bool gemv1_supported(int64_t K, int64_t N);   // batch-1 GEMV kernels cover this shape
hipError_t launch_gemv1(const void* x, int xdt, int64_t K, const uint32_t* qw,
                        const uint16_t* scales, const uint8_t* zeros, int64_t N, int group,
                        const float* r, void* y, int ydt, hipStream_t st);
size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K, int group);
hipError_t launch_w4a16(const void* x, int xdt, int64_t M, int64_t K, int64_t ldx,
                        const uint32_t* qw, const uint16_t* scales, const uint8_t* zeros,
                        int64_t N, int group, const float* inv_s, void* y, int ydt, int64_t ldy,
                        void* ws, hipStream_t st);

// 2 <= M <= 64 (k_mid.hip): the memory-bound small-batch product
bool mid_supported(int64_t M, int64_t N, int64_t K);
size_t mid_ws_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_mid(const void* x, int xdt, int64_t M, int64_t K, int64_t ldx, const uint32_t* qw,
                      const uint16_t* scales, const uint8_t* zeros, int64_t N, int group,
                      const float* inv_s, void* y, int ydt, int64_t ldy, void* ws, hipStream_t st);

// 2 <= M <= 16 (k_skinny.hip): one block per compute unit with the
// activations, steps and zero points staged in LDS; blocks (0: shape not
// covered) and launch.  No workspace.
int skinny_st_blocks(int64_t M, int64_t N, int64_t K, int group);
hipError_t launch_skinny_st(const void* x, int xdt, int64_t M, int64_t K, int64_t ldx,
                            const uint32_t* qw, const uint16_t* scales, const uint8_t* zeros,
                            int64_t N, int group, const float* inv_s, void* y, int ydt, int64_t ldy,
                            hipStream_t st);
// Layers whose rows exceed one launch's steps and zero points: the kernel on
// row chunks, one launch each (chunks: 1 = one launch, 0 = not covered).
int skinny_st_chunks(int64_t M, int64_t N, int64_t K, int group);
hipError_t launch_skinny_st_chunked(const void* x, int xdt, int64_t M, int64_t K, int64_t ldx,
                                    const uint32_t* qw, const uint16_t* scales, const uint8_t* zeros,
                                    int64_t N, int group, const float* inv_s, void* y, int ydt, int64_t ldy,
                                    hipStream_t st);

// ---- plain streaming read (k_stream.hip): bytes a multiple of 1024, blocks
// of 1024 threads, unroll 1, 2, 4 or 8 units in flight per wave
hipError_t launch_read_stream(const void* p, int64_t bytes, int blocks, int unroll, uint32_t* block_xor,
                              hipStream_t st);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Compute units of the current device (cached per device).
int device_cus();

}  // namespace awq
