/*
 * awq.h -- C ABI of the AWQ W4A16 hot path for AMD Instinct MI355X (gfx950).
 *
 * The method is activation-aware weight quantization as described in
 *   "AWQ Math" (aicassindra.com transformer-math series),
 *   "AWQ > Benefits and Practical Considerations" and "AWQ > Limitations"
 *   (mbrenndoerfer.com),
 *   "AWQ vs. GPTQ: Understanding Weight Quantization Principles".
 *
 * Four calls make up the path:
 *   awq_act_stats      per-input-channel mean |x_j| over calibration tokens
 *   awq_search_scales  s_j = (mean|x_j|)^alpha, alpha chosen on a grid by the
 *                      layer-output MSE of Q(W diag(s)) diag(s)^-1 x
 *                      (awq_search_scales_ex: the same under the quantizer's
 *                      variants and with channels kept in 16-bit)
 *   awq_quantize_pack  group-wise asymmetric 4-bit round-to-nearest of
 *                      W diag(s): codes packed 8 per int32, one fp16 step and
 *                      one uint8 zero point per group (of 64, 128 or 256)
 *   awq_w4a16_gemm     y = x (dequant W)^T fused: unpack, apply the group step
 *                      and zero point, optionally the per-channel 1/s
 * and two helpers:
 *   awq_fold_scales    divides the producer of x (a LayerNorm's gain and bias,
 *                      a preceding linear's rows) by s, which moves the
 *                      per-channel 1/s out of the product
 *   awq_quantize_codes the quantizer's variants (N bits, asymmetric or
 *                      symmetric grid), one unpacked code per byte; the search
 *                      scores the same variants
 * and, for the mixed-precision baseline that AWQ replaces (the salient
 * channels kept in 16-bit, the rest quantized), a channel selector whose mask
 * the search accepts:
 *   awq_salient_channels  the n channels with the largest mean |x_j|
 * Linears that read the same input (q, k and v; gate and up) are searched
 * together by passing their row-concatenated W to awq_search_scales: they then
 * share s, and one fold serves them all.
 *
 * Conventions shared by every call
 * --------------------------------
 *  Shapes.  W is [N][K] row-major (N = output channels C_out, K = input
 *    channels C_in); activations are [rows][ldx] row-major with K used
 *    columns.  A quantization group is 64, 128 (the usual choice) or 256
 *    consecutive input channels of one row, and K must be a multiple of it.
 *  Memory.  Every array argument is a DEVICE pointer on the current HIP device,
 *    allocated and owned by the caller; the library allocates nothing and keeps
 *    no state between calls.  Scratch memory is the caller's workspace `ws` of
 *    at least awq_workspace_bytes(...) bytes, 256-byte aligned.
 *  Alignment.  Activations, weights and packed codes must be 16-byte aligned
 *    and leading dimensions multiples of 8 elements (128-bit loads).
 *  Execution.  Every call validates its arguments on the host, then enqueues
 *    kernels on `stream` (a hipStream_t; NULL is the null stream) and returns
 *    without waiting.  Asynchronous device faults surface at the caller's
 *    synchronisation.  Calls are re-entrant; two calls that share a workspace
 *    must be ordered on one stream.
 *  Errors.  On any status other than AWQ_OK nothing was enqueued and the
 *    outputs are untouched (AWQ_ERR_HIP: a launch failed part way).
 *  Determinism.  The same inputs give bit-identical outputs on every run: no
 *    floating-point atomics, fixed reduction orders.
 *  Numerical domain.  Inputs are finite.  Calibration column sums satisfy
 *    sum_t |x_tj| < 2^29 (fixed-point range of the statistic).  The step of
 *    every group of W diag(s) before rounding (its range over 2^N - 1, or
 *    max|w| over 2^(N-1) for the symmetric grid) is below 65504 (the step is
 *    stored in fp16).
 *    Outside this domain results are unspecified.
 */
#ifndef AWQ_H
#define AWQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum awq_status {
  AWQ_OK = 0,
  AWQ_ERR_NULL = 1,         /* a required pointer is NULL                          */
  AWQ_ERR_SHAPE = 2,        /* K % group != 0, a size < 0 (or 0 where > 0 needed), ld < K */
  AWQ_ERR_DTYPE = 3,        /* element type not accepted by this call               */
  AWQ_ERR_ALIGN = 4,        /* pointer not 16-byte aligned or ld % 8 != 0            */
  AWQ_ERR_UNSUPPORTED = 5,  /* group size, bits, n_alpha outside [1, 64], K too big */
  AWQ_ERR_WORKSPACE = 6,    /* ws NULL or smaller than awq_workspace_bytes(...)      */
  AWQ_ERR_HIP = 7           /* a HIP launch failed                                   */
} awq_status;

typedef enum awq_dtype {
  AWQ_F16 = 0,   /* IEEE binary16                       */
  AWQ_BF16 = 1,  /* bfloat16                            */
  AWQ_F32 = 2    /* IEEE binary32 (outputs only)        */
} awq_dtype;

typedef enum awq_op {
  AWQ_OP_ACT_STATS = 0,
  AWQ_OP_SEARCH = 1,
  AWQ_OP_QUANTIZE = 2,
  AWQ_OP_GEMM = 3
} awq_op;

#define AWQ_GROUP 128           /* the usual group size; 64 and 256 are accepted too */
#define AWQ_MAX_ALPHA 64
#define AWQ_MAX_K 131072
/* Largest calibration row stride (elements) of awq_search_scales: 256 rows of
 * it must span less than 2^31 bytes (the error product addresses a tile of
 * tokens with 32-bit offsets). */
#define AWQ_MAX_LDX_SEARCH 4194304

/* Version of this interface (incremented on any signature change). */
int awq_abi_version(void);

/* Human-readable name of a status value (static storage). */
const char* awq_status_str(awq_status st);

/* Workspace bytes a call needs for the given sizes (0 if it needs none), for
 * every group size.  Arguments that an op does not use are ignored. */
size_t awq_workspace_bytes(awq_op op, int64_t M, int64_t N, int64_t K, int64_t T, int n_alpha);

/*
 * Calibration statistic: mean_abs[j] = average over t of |x[t][j]|.
 * "AWQ Math", section "Saliency is an activation property, not a weight
 * property" (input channels ranked by average |x_j| over a calibration set);
 * "AWQ > Limitations" (the saliency metric is the average activation
 * magnitude).
 *
 * The sum is exact: each |x| is taken in fixed point with LSB 2^-24 (exact for
 * fp16; bf16 magnitudes below 2^-17 are truncated to that LSB), summed in
 * integers, converted once to double, multiplied by 2^-24, divided by T in
 * double and rounded to float.
 *
 *   x         [T][ldx] fp16 or bf16 (xdt), K columns used
 *   T         calibration tokens, > 0
 *   K         input channels, > 0, multiple of 8
 *   ldx       row stride in elements, >= K, multiple of 8
 *   mean_abs  [K] float, written
 *   ws        >= awq_workspace_bytes(AWQ_OP_ACT_STATS, 0, 0, K, T, 0)
 */
awq_status awq_act_stats(const void* x, awq_dtype xdt, int64_t T, int64_t K, int64_t ldx,
                         float* mean_abs, void* ws, size_t ws_bytes, void* stream);

/*
 * Scale search.  "AWQ Math", section "Searching the scale -- no backprop
 * required": s_j = (s_X,j)^alpha with s_X,j = mean |x_j|, alpha on a small grid
 * in [0, 1], and the alpha that minimises the mean squared error between the
 * layer output W x and Q(W diag(s)) diag(s)^-1 x over the calibration tokens
 * wins.  Q is the quantizer of awq_quantize_pack (4-bit asymmetric grid, fp16
 * step as stored); with alpha = 0 (s = 1) the loss is that of plain
 * round-to-nearest.
 *
 *   candidate i: s_ij = float( pow( max(double(mean_abs[j]), 2^-14), alphas[i] ) )
 *   loss_i      = (1 / (T N)) sum_t sum_n ( ((W - W_hat_i) x_t)_n )^2
 *   best        = lowest i with the minimal loss (NaN losses are skipped)
 *
 *   w           [N][K] fp16 or bf16 (dt), contiguous
 *   x_calib     [T][ldx] same dtype as w; ldx <= AWQ_MAX_LDX_SEARCH
 *   mean_abs    [K] float (output of awq_act_stats)
 *   alphas      [n_alpha] double, device memory
 *   n_alpha     1..AWQ_MAX_ALPHA
 *   group_size  64, 128 or 256; K a multiple of it and of 128
 *   s_out       [K] float: s of the best candidate
 *   inv_s_out   [K] float: 1.0f / s (IEEE division); may be NULL
 *   loss_out    [n_alpha] double; may be NULL
 *   best_idx_out  int32; may be NULL; -1 if every loss is NaN
 *   ws          >= awq_workspace_bytes(AWQ_OP_SEARCH, 0, N, K, T, n_alpha)
 * The error products run on fp16/bf16 matrix cores with fp32 accumulation;
 * the per-row error is scaled by an exact power of two before rounding to
 * fp16 so that it stays in the normal range.  Two equivalent forms of the
 * loss: the direct one contracts E_i with the tokens (2 T N K operations per
 * candidate); the Gram one uses sum_t ||E_i x_t||^2 = sum_n e_n^T (X^T X) e_n,
 * forms G = X^T X once (its tiles on and above the diagonal; Tp = T rounded
 * up to 256; fp32 per chunk of at most 8192 tokens, fp64 across chunks in
 * chunk order) and carries each row of G as two fp16
 * parts (22 significant bits); with G symmetric, a candidate contracts only
 * over the 256 x 256 blocks of G on and below the diagonal (off-diagonal
 * blocks counted twice), 2 N 256^2 g (g + 1) operations for g = ceil(K / 256),
 * about 2 N K^2.  The Gram form is taken when K <= 32768, Tp < 2^23 (its
 * token rows are addressed with 32-bit offsets) and its total is under half
 * of the direct one's.
 * Linears that read the same input may be searched together by passing their
 * row-concatenated W.
 */
awq_status awq_search_scales(const void* w, awq_dtype dt, int64_t N, int64_t K,
                             const void* x_calib, int64_t T, int64_t ldx,
                             const float* mean_abs, const double* alphas, int n_alpha,
                             int group_size, float* s_out, float* inv_s_out, double* loss_out,
                             int32_t* best_idx_out, void* ws, size_t ws_bytes, void* stream);

/*
 * The scale search of awq_search_scales under the quantizer's variants and
 * with channels kept out of the quantization.  "AWQ Math", sections
 * "Weight-only quantization and where it breaks" (N-bit weights; the
 * symmetric step max|w| / 2^(N-1)) and "Shapes, granularity, and complexity"
 * (groups with their own step and zero point); for kept channels, "AWQ vs.
 * GPTQ: Understanding Weight Quantization Principles" (the salient weights
 * kept in higher precision).  Same arguments and workspace as
 * awq_search_scales, plus:
 *   bits, symmetric  the grid, as for awq_quantize_codes (4 and 0: the grid
 *               of awq_quantize_pack, which awq_search_scales scores)
 *   kept        [K] uint8 or NULL, 16-byte aligned: channels with kept[k] != 0
 *               stay in 16-bit (W_hat = W there) and are left out of their
 *               groups' ranges; with alphas = {0} the loss is that of the
 *               mixed-precision baseline (see awq_salient_channels)
 * bits = 4, symmetric = 0, kept = NULL is exactly awq_search_scales.
 */
awq_status awq_search_scales_ex(const void* w, awq_dtype dt, int64_t N, int64_t K,
                                const void* x_calib, int64_t T, int64_t ldx,
                                const float* mean_abs, const double* alphas, int n_alpha,
                                int group_size, int bits, int symmetric, const uint8_t* kept,
                                float* s_out, float* inv_s_out, double* loss_out,
                                int32_t* best_idx_out, void* ws, size_t ws_bytes, void* stream);

/*
 * The salient channels of the mixed-precision baseline that AWQ replaces.
 * "AWQ vs. GPTQ: Understanding Weight Quantization Principles", sections on
 * the central insight (a weight's importance follows the magnitude of the
 * activations it meets; protecting about 1 % of the salient weights greatly
 * reduces the degradation) and on per-channel scaling (keeping them in higher
 * precision works but makes the layer mixed-precision); "AWQ Math", section
 * "Weight-only quantization and where it breaks" (keep the important weights
 * in FP16 and quantize the rest).
 *   kept[j] = 1 if rank_j < n_keep else 0,
 *   rank_j  = #{i : m_i > m_j} + #{i < j : m_i = m_j}   (ties: lower index first)
 *
 *   mean_abs  [K] float (output of awq_act_stats), finite
 *   K         > 0;  n_keep  0..K
 *   kept      [K] uint8, written
 * O(K^2) comparisons; not part of the quantization path.
 */
awq_status awq_salient_channels(const float* mean_abs, int64_t K, int64_t n_keep, uint8_t* kept,
                                void* stream);

/*
 * Group-wise asymmetric 4-bit round-to-nearest of W' = W diag(s).
 * "AWQ Math", sections "Weight-only quantization and where it breaks"
 * (Q(w) = step * round(w / step)) and "Shapes, granularity, and complexity"
 * (groups of commonly 128 input channels, each with its own step and zero
 * point); "AWQ > Benefits and Practical Considerations" (one scale and one
 * zero point per 128 weights).  Per group of g = group_size (64, 128 or 256)
 * consecutive k of one row n:
 *   w'  = float(w) * s_k                      (s == NULL: s = 1, plain RTN)
 *   lo  = min(0, min w'),  hi = max(0, max w')
 *   d   = (hi - lo) / 15                      (float, IEEE division)
 *   step = smallest fp16 >= max(d, 2^-24);   D = float(step)
 *   z   = clamp(rint(-lo / D), 0, 15)
 *   q_k = clamp(rint(w'_k / D) + z, 0, 15)    (rint: round half to even)
 *
 *   w         [N][K] fp16 or bf16 (dt), contiguous
 *   s         [K] float or NULL
 *   qweight   [N][K/8] int32: code of k = 8c + j in bits [4j, 4j+4) of word c
 *   scales    [N][K/g] fp16 bit patterns (step)
 *   zeros     [N][K/g] uint8 (z)
 *   scales_f32_dbg [N][K/g] float (d, before rounding); may be NULL
 * N == 0 is a no-op.
 */
awq_status awq_quantize_pack(const void* w, awq_dtype dt, int64_t N, int64_t K, const float* s,
                             int group_size, int32_t* qweight, uint16_t* scales, uint8_t* zeros,
                             float* scales_f32_dbg, void* stream);

/*
 * The quantizer's variants, one code per byte: N = bits, asymmetric or
 * symmetric grid, groups of g = group_size.  "AWQ Math", section
 * "Weight-only quantization and where it breaks" (N-bit weights; the
 * symmetric step max|w| / 2^(N-1), Q(w) = step * round(w / step)) and
 * "Shapes, granularity, and complexity" (groups, each with its own step and
 * zero point); "CPU-SLM implications and common pitfalls" (larger groups
 * widen the step).  Per group, with w' = float(w) * s_k (s == NULL: s = 1):
 *   asymmetric (symmetric == 0), bits 2..8:
 *     d = (max(0, max w') - min(0, min w')) / (2^N - 1)        (IEEE division)
 *     z = clamp(rint(-min(0, min w') / D), 0, 2^N - 1),  C = 2^N - 1
 *   symmetric (symmetric == 1), bits 2..7:
 *     d = max|w'| / 2^(N-1)                                     (exact)
 *     z = 2^(N-1),  C = 2^N: codes -2^(N-1) .. 2^(N-1) are stored shifted up by
 *     z, 2^N + 1 levels as the formula gives (so not packable into N bits)
 *   both: step = smallest fp16 >= max(d, 2^-24), D = float(step),
 *     q_k = clamp(rint(w'_k / D) + z, 0, C); the grid value is D (q_k - z).
 * bits 4 and symmetric 0 give the codes awq_quantize_pack packs (same g).
 *
 *   w        [N][K] fp16 or bf16 (dt), contiguous
 *   s        [K] float or NULL
 *   codes    [N][K] uint8, 16-byte aligned
 *   scales   [N][K/g] fp16 bit patterns (step)
 *   zeros    [N][K/g] uint8 (z)
 * N == 0 is a no-op.
 */
awq_status awq_quantize_codes(const void* w, awq_dtype dt, int64_t N, int64_t K, const float* s,
                              int group_size, int bits, int symmetric, uint8_t* codes,
                              uint16_t* scales, uint8_t* zeros, void* stream);

/*
 * Fused W4A16 product.  "AWQ > Benefits and Practical Considerations": the
 * dequantization unpacks 4-bit integers, applies the group scale and zero
 * point and optionally the per-channel inverse scale (when it is not folded
 * into the preceding layer), fused with the matrix multiply so that the fp16
 * weight matrix is never materialised.
 *   y[m][n] = sum_k step[n][k/g] * (q[n][k] - z[n][k/g]) * x[m][k] * r[k]
 * with r = inv_s (or 1 when inv_s == NULL) and g = group_size (64, 128 or
 * 256, as quantized).
 *
 *   x        [M][ldx] fp16 or bf16 (xdt)
 *   qweight, scales, zeros  as written by awq_quantize_pack
 *   inv_s    [K] float or NULL
 *   y        [M][ldy] of ydt (F16, BF16 or F32)
 *   ws       >= awq_workspace_bytes(AWQ_OP_GEMM, M, N, K, 0, 0)
 * M == 1 runs the batch-1 GEMV (fp32 accumulation of exact int4 x fp16
 * products of x r); larger M runs matrix-core products on fp16 operands: x r
 * scaled by exact powers of two (per token and 128 channels for M <= 16 when
 * K is a multiple of 128, per token otherwise) and the dequantized weights
 * step (q - z) rounded once to fp16.  M == 0 or N == 0 is a no-op.
 */
awq_status awq_w4a16_gemm(const void* x, awq_dtype xdt, int64_t M, int64_t K, int64_t ldx,
                          const int32_t* qweight, const uint16_t* scales, const uint8_t* zeros,
                          int64_t N, int group_size, const float* inv_s, void* y, awq_dtype ydt,
                          int64_t ldy, void* ws, size_t ws_bytes, void* stream);

/*
 * The fused W4A16 product of awq_w4a16_gemm for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, results and kernels as
 * awq_w4a16_gemm, without the workspace: the product's scratch (for M > 16 the
 * activations converted to fp16 and the dequantization constants, at most
 * awq_workspace_bytes(AWQ_OP_GEMM, M, N, K, 0, 0) bytes) lives in one
 * library-held device array of AWQ_NOALLOC_SCRATCH_BYTES per GPU, reserved
 * when the library's code is loaded on that GPU and held until the process
 * ends.  Its address is looked up on the first call on each device.  Nothing
 * is allocated per call.
 *   Sizes whose scratch exceeds AWQ_NOALLOC_SCRATCH_BYTES -> AWQ_ERR_UNSUPPORTED
 *   (the prefill shape 2048 x 28672 -> 8192 with groups of 128 fits; with
 *   groups of 64 it does not).
 * Every call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (different streams, or host threads, without ordering) race and give
 * undefined results.  The kernels write every scratch byte they read within
 * the same call, so nothing has to start at zero.
 */
#define AWQ_NOALLOC_SCRATCH_BYTES (128u << 20)
awq_status awq_w4a16_gemm_noalloc(const void* x, awq_dtype xdt, int64_t M, int64_t K, int64_t ldx,
                                  const int32_t* qweight, const uint16_t* scales,
                                  const uint8_t* zeros, int64_t N, int group_size,
                                  const float* inv_s, void* y, awq_dtype ydt, int64_t ldy,
                                  void* stream);

/*
 * Folds the activation scaling into the operation that produces x, so that
 * the product runs with inv_s == NULL.  "AWQ Math", section "The equivalent
 * transform: scale up W, scale down x": the division of x_j by s_j can be
 * moved backward into the previous layer, for example the preceding LayerNorm
 * or linear; "AWQ > Benefits and Practical Considerations": the product applies
 * the inverse scale only when it is not already fused into the preceding layer.
 * In place, on v [rows][ld] (cols used):
 *   axis 1: v[i][j] <- v[i][j] / s[j]   s has cols entries: a LayerNorm's gain
 *           and bias, a preceding linear's bias (1 x K rows)
 *   axis 0: v[i][j] <- v[i][j] / s[i]   s has rows entries: a preceding
 *           linear's weight [K][C_in], whose row i produces x_i
 * Each value becomes dt(float(v) / s) with IEEE binary32 division and
 * round-to-nearest-even to dt.
 *
 *   v       device, dt F16, BF16 or F32, aligned to its element size
 *   rows, cols  >= 0 (an empty array is a no-op); ld >= cols
 *   s       device float, finite and nonzero
 *   axis    0 or 1
 */
awq_status awq_fold_scales(void* v, awq_dtype dt, int64_t rows, int64_t cols, int64_t ld, const float* s,
                           int axis, void* stream);

/* Diagnostic: a plain streaming read of `bytes` of device memory, the rate the
 * W4A16 products are measured against at their own sizes.  "AWQ Math",
 * section "Weight-only quantization and where it breaks": at decode batch
 * sizes the product is bound by moving the weights, so its ceiling is the rate
 * at which this chip reads the same number of bytes, not the HBM peak alone.
 * One launch of `blocks` blocks of 1024 threads; each wave reads `unroll`
 * whole 1 KB units per step (64 lanes x 16 B, non-temporal loads), striding
 * over the buffer, and each block writes the XOR of every 32-bit word it read
 * to block_xor[block] (the XOR over all blocks is the XOR of the buffer).
 *
 *   p          device, 16-byte aligned, `bytes` readable
 *   bytes      > 0, a multiple of 1024
 *   blocks     1 .. 65535
 *   unroll     1, 2, 4 or 8
 *   block_xor  device uint32 [blocks], written
 * Errors: NULL pointer -> AWQ_ERR_NULL; bytes or blocks out of range ->
 * AWQ_ERR_SHAPE; unroll -> AWQ_ERR_UNSUPPORTED; p misaligned -> AWQ_ERR_ALIGN.
 */
awq_status awq_read_stream(const void* p, int64_t bytes, int blocks, int unroll, uint32_t* block_xor,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AWQ_H */
