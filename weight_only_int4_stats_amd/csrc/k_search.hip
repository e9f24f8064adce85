// Scale search ("AWQ Math", section "Searching the scale -- no backprop
// required"): candidates s_j = (s_X,j)^alpha on a grid of alpha, each scored
// by the mean squared error between W x and Q(W diag(s)) diag(s)^-1 x over
// the calibration tokens; the lowest-error candidate wins.
//
// Per candidate i the loss is
//     L_i = (1 / (T N)) sum_t sum_n ( (E_i x_t)_n )^2,   E_i = W - W_hat_i,
// and its cost is the dense contraction E_i X^T (2 T N K flops), which runs on
// the matrix cores.  Three steps per candidate:
//   1. k_err_gen    one block per row: the row's groups are quantized exactly
//                   as awq_quantize_pack (the 4-bit asymmetric grid) or
//                   awq_quantize_codes (any grid) do, E = W - D (q - z) r in
//                   float with r = fp32(1 / s) (diag(s)^-1, computed once per
//                   candidate and channel);
//                   the row's max|E| fixes p (so the row fits fp16's normal
//                   range), then E * 2^p is written as fp16 into the
//                   workspace, with p per row (the errors stay in registers
//                   in between for K <= 8192, else they are computed twice).
//   2. k_err_contract  256x256 tiles of C = X E'^T with fp16 MFMA (fp32
//                   accumulation); the epilogue squares and sums the tile,
//                   undoes the powers of two in double, and writes one double
//                   per tile.  bf16 calibration tokens are first rounded to
//                   fp16 with their own power-of-two scale (exact unless a
//                   value falls 2^24 below its token's largest).
//   3. k_sum_partials  fixed-order double sum of the tile partials -> L_i.
// Each step runs for a batch of candidates per launch (blockIdx.y, or the
// block of k_sum_partials, is the candidate's slot in the workspace): small
// layers score all candidates in three launches.
// Finally k_select picks the lowest index among the minimal finite losses and
// writes s, 1/s, the losses and the index.  Every sum has a fixed order, so
// the result is bit-reproducible.
#include "awq_device.h"
#include "awq_internal.h"
#include "k_contract.h"
#include "k_rows_f16.h"

#include <algorithm>

namespace awqk {

// ---------------------------------------------------------------------------
// candidate scales: S[i][j] = float(pow(max(double(m_j), 2^-14), alpha_i))
// ---------------------------------------------------------------------------
__global__ void k_cand_scales(const float* __restrict__ m, const double* __restrict__ alphas,
                              int n_alpha, int64_t K, float* __restrict__ S, float* __restrict__ IS) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)n_alpha * K) return;
  const int64_t i = idx / K;
  const int64_t j = idx - i * K;
  const double b = fmax((double)m[j], 0x1p-14);
  const float sv = (float)pow(b, alphas[i]);
  S[idx] = sv;
  IS[idx] = 1.0f / sv;                           // IEEE division, once per candidate and channel
}

// ---------------------------------------------------------------------------
// error generation
// ---------------------------------------------------------------------------
// Grids of the error generator: the 4-bit asymmetric one with compile-time
// constants, any asymmetric one, any symmetric one.
enum { kGridQ4 = 0, kGridAsym = 1, kGridSym = 2 };

// KEPT: channels with kept[k] != 0 stay in 16-bit (the mixed-precision
// baseline): they are left out of the group's min / max and have no error.
template <int DT, int GL, int GR, bool KEPT>
__device__ __forceinline__ void err_word(const uint16_t* __restrict__ wrow,
                                         const float* __restrict__ s, const float* __restrict__ is,
                                         const uint8_t* __restrict__ kept, int64_t k0, QSpec q,
                                         float e[8]) {
  const u32x4 raw = ldg128(wrow + k0);
  uint2 kb = {0u, 0u};
  if constexpr (KEPT) kb = *reinterpret_cast<const uint2*>(kept + k0);
  auto is_kept = [&](int j) {
    return KEPT && (((j < 4 ? kb.x : kb.y) >> (8 * (j & 3))) & 0xFFu) != 0u;
  };
  const f32x4 s0 = *reinterpret_cast<const f32x4*>(s + k0);
  const f32x4 s1 = *reinterpret_cast<const f32x4*>(s + k0 + 4);
  const f32x4 r0 = *reinterpret_cast<const f32x4*>(is + k0);
  const f32x4 r1 = *reinterpret_cast<const f32x4*>(is + k0 + 4);
  float w[8], sv[8], rv[8], wp[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    w[2 * j] = lo_f32<DT>(raw[j]);
    w[2 * j + 1] = hi_f32<DT>(raw[j]);
    sv[j] = s0[j];
    sv[4 + j] = s1[j];
    rv[j] = r0[j];
    rv[4 + j] = r1[j];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) wp[j] = w[j] * sv[j];
  float mn = is_kept(0) ? INFINITY : wp[0], mx = is_kept(0) ? -INFINITY : wp[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) {
    mn = fminf(mn, is_kept(j) ? INFINITY : wp[j]);
    mx = fmaxf(mx, is_kept(j) ? -INFINITY : wp[j]);
  }
  seg_minmax<GL>(mn, mx);
  const GroupGrid g = group_grid<GR == kGridSym>(mn, mx, GR == kGridQ4 ? kQ4 : q);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float c = quant_code(wp[j], g);
    const float grid = g.D * (c - g.z);            // exact: fp16 step x small integer
    e[j] = is_kept(j) ? 0.0f : w[j] - grid * rv[j];  // times fp32(1 / s): diag(s)^-1
  }
}

constexpr int kErrKeep = 4;   // packed words per thread kept in registers (K <= 8192)

// GL: threads per quantization group (group / 8); q: the grid, GR its kind;
// KEPT: a mask of channels kept in 16-bit.
template <int DT, int GL, int GR, bool KEPT>
__global__ __launch_bounds__(256) void k_err_gen(const uint16_t* __restrict__ W, int64_t N,
                                                 int64_t K, const float* __restrict__ s,
                                                 const float* __restrict__ is, QSpec q,
                                                 const uint8_t* __restrict__ kept,
                                                 uint16_t* __restrict__ E, int* __restrict__ pexp) {
  // candidate slot blockIdx.y of a batched launch: its scales and error rows
  const int64_t cy = blockIdx.y;
  s += cy * K;
  is += cy * K;
  E += cy * N * K;
  pexp += cy * N;
  const int64_t n = blockIdx.x;
  const uint16_t* wrow = W + n * K;
  const int64_t wpr = K >> 3;
  uint16_t* erow = E + n * K;
  __shared__ float wmax[4];
  __shared__ int sp;
  auto row_exp = [&](float emax) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) emax = fmaxf(emax, __shfl_xor(emax, off));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = emax;
    __syncthreads();
    if (threadIdx.x == 0) {
      const float m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
      int p = 0;
      if (m > 0.0f) {
        int ex;
        frexpf(m, &ex);          // m < 2^ex
        p = 14 - ex;             // m * 2^p < 2^14, well inside fp16's finite range
      }
      sp = p;
      pexp[n] = p;
    }
    __syncthreads();
    return sp;
  };
  auto store = [&](int64_t c, const float e[8], int p) {
    u32x4 out;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      out[j] = f32_to_f16_bits(ldexpf(e[2 * j], p)) | (f32_to_f16_bits(ldexpf(e[2 * j + 1], p)) << 16);
    *reinterpret_cast<u32x4*>(erow + c * 8) = out;
  };
  float emax = 0.0f;
  if (wpr <= 256 * kErrKeep) {
    // the row's errors stay in registers between the maximum and the store
    // (whole GL-lane segments are in or out: wpr is a multiple of GL)
    float e[kErrKeep][8];
#pragma unroll
    for (int i = 0; i < kErrKeep; ++i) {
      const int64_t c = threadIdx.x + 256 * i;
      if (c < wpr) {
        err_word<DT, GL, GR, KEPT>(wrow, s, is, kept, c * 8, q, e[i]);
#pragma unroll
        for (int j = 0; j < 8; ++j) emax = fmaxf(emax, fabsf(e[i][j]));
      }
    }
    const int p = row_exp(emax);
#pragma unroll
    for (int i = 0; i < kErrKeep; ++i) {
      const int64_t c = threadIdx.x + 256 * i;
      if (c < wpr) store(c, e[i], p);
    }
    return;
  }
  // pass 1: largest |E| of the row (whole GL-lane segments are in or out)
  for (int64_t c0 = 0; c0 < wpr; c0 += 256) {
    const int64_t c = c0 + threadIdx.x;
    float e[8];
    if (c < wpr) {
      err_word<DT, GL, GR, KEPT>(wrow, s, is, kept, c * 8, q, e);
#pragma unroll
      for (int j = 0; j < 8; ++j) emax = fmaxf(emax, fabsf(e[j]));
    }
  }
  const int p = row_exp(emax);
  // pass 2: the same arithmetic again, scaled by 2^p and rounded to fp16
  for (int64_t c0 = 0; c0 < wpr; c0 += 256) {
    const int64_t c = c0 + threadIdx.x;
    if (c < wpr) {
      float e[8];
      err_word<DT, GL, GR, KEPT>(wrow, s, is, kept, c * 8, q, e);
      store(c, e, p);
    }
  }
}

// ---------------------------------------------------------------------------
// contraction C = X E'^T, sum of squares per tile
// ---------------------------------------------------------------------------
// C = X E'^T on 256 x 256 tiles (tokens x error rows; the shared contraction
// core), the squares of each tile summed in the epilogue.
// Tile order: block i runs on L2 slice i mod 8 and slice x takes the x-th
// eighth of the tiles in band order (bands of 8 error-row tiles; inside a band
// token tiles, then the band's row tiles), so the 32 blocks a slice runs at
// once share 4 token tiles and 8 error-row tiles through its L2.
constexpr int kCBand = 8;                // error-row tiles per band
constexpr int kCXcds = 8;                // L2 slices (block i -> slice i mod 8)

inline int64_t contract_blocks(int64_t T, int64_t N) {
  const int64_t tiles = ((T + kCT - 1) / kCT) * ((N + kCT - 1) / kCT);
  return kCXcds * ((tiles + kCXcds - 1) / kCXcds);
}

// px: per-token power of two of the fp16 tokens (NULL: tokens unscaled).
// partial[ty * gx + tx] = sum of squares of tile (token tile ty, row tile tx).
__global__ __launch_bounds__(256) void k_err_contract(const uint16_t* __restrict__ X, int64_t T,
                                                      int64_t ldx, const int* __restrict__ px,
                                                      const uint16_t* __restrict__ E, int64_t N,
                                                      int64_t K, const int* __restrict__ pexp,
                                                      double* __restrict__ partial) {
  // four LDS arrays, the loop unrolled by four: each stage is a known array
  __shared__ __attribute__((aligned(16))) uint8_t lds0[kCStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[kCStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds2[kCStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds3[kCStage];
  __shared__ double wsum[kCWaves];

  // ---- tile of this block (candidate slot blockIdx.y of a batched launch)
  const int64_t gx = (N + kCT - 1) / kCT, gy = (T + kCT - 1) / kCT, tiles = gx * gy;
  E += (int64_t)blockIdx.y * N * K;
  pexp += (int64_t)blockIdx.y * N;
  partial += (int64_t)blockIdx.y * tiles;
  const int64_t per = (tiles + kCXcds - 1) / kCXcds;
  const int64_t slot = blockIdx.x / kCXcds;
  const int64_t o = (int64_t)(blockIdx.x % kCXcds) * per + slot;
  if (slot >= per || o >= tiles) return;
  const int64_t band = o / (gy * kCBand);
  const int64_t rb = o - band * gy * kCBand;
  const int64_t bw = gx - band * kCBand < kCBand ? gx - band * kCBand : kCBand;
  const int64_t ty = rb / bw;
  const int64_t tx = band * kCBand + (rb - ty * bw);
  const int64_t t0 = ty * kCT;   // tokens (MFMA rows)
  const int64_t n0 = tx * kCT;   // rows of E (MFMA columns)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 1, wn = wv & 1;
  const int64_t rows = T - t0 < kCT ? T - t0 : kCT;
  const int64_t cols = N - n0 < kCT ? N - n0 : kCT;
  // rows past T / N fall outside the descriptors and arrive as zeros
  ContractSrc cs;
  cs.ars = rsrc4(X + t0 * ldx, (uint32_t)((rows - 1) * ldx * 2 + K * 2));
  cs.a_ld = (uint32_t)(ldx * 2);
  cs.brs = rsrc4(E + n0 * K, (uint32_t)(cols * K * 2));
  cs.b_ld = (uint32_t)(K * 2);
  cs.k0 = 0;
  cs.a_dup_sh = 0;
  cs.S = K / kCBK;

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;
  contract_tile<false>(cs, lds0, lds1, lds2, lds3, acc);

  // epilogue.  Lane value v of block (mb, nb) belongs to E row
  // n = n0 + wn 128 + nb 32 + lane % 32 and token
  // t = t0 + wm 128 + mb 32 + 8 (v / 4) + 4 (lane / 32) + v % 4.  Tokens past T
  // were copied as zeros, so their products are 0 and need no mask (the token
  // scale index is clamped); columns past N are skipped.
  // the power of two of each E row this lane's results belong to
  int pe[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int64_t n = n0 + wn * 128 + nb * 32 + (lane & 31);
    pe[nb] = pexp[n < N ? n : N - 1];
  }
  double tot = 0.0;
  if (px == nullptr) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      float q[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int v = 0; v < 16; ++v) q[v & 3] = fmaf(acc[mb][nb][v], acc[mb][nb][v], q[v & 3]);
      const double ssq = ((double)q[0] + (double)q[1]) + ((double)q[2] + (double)q[3]);
      if (n0 + wn * 128 + nb * 32 + (lane & 31) < N) tot += ldexp(ssq, -2 * pe[nb]);
    }
  } else {
    double ssq[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      int ps[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t t = t0 + wm * 128 + mb * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        ps[v] = px[t < T ? t : T - 1];
      }
#pragma unroll
      for (int v = 0; v < 16; ++v)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const double c = (double)acc[mb][nb][v];
          ssq[nb] += ldexp(c * c, -2 * ps[v]);
        }
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
      if (n0 + wn * 128 + nb * 32 + (lane & 31) < N) tot += ldexp(ssq[nb], -2 * pe[nb]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off);
  if (lane == 0) wsum[wv] = tot;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int w = 0; w < kCWaves; ++w) t += wsum[w];
    partial[ty * gx + tx] = t;
  }
}

// Fixed-order sum of n doubles by one block of 256 threads -> out[0] = sum / denom.
__global__ __launch_bounds__(256) void k_sum_partials(const double* __restrict__ part, int64_t n,
                                                      double denom, double* __restrict__ out) {
  // block b: the b-th of a batch of partial sets, n apart
  part += (int64_t)blockIdx.x * n;
  out += blockIdx.x;
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 256) s += part[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = red[0] / denom;
}

__device__ __forceinline__ int argmin_finite(const double* L, int n) {
  int best = -1;
  double bv = 0.0;
  for (int i = 0; i < n; ++i) {
    const double v = L[i];
    if (v != v) continue;             // NaN is never chosen
    if (best < 0 || v < bv) {
      best = i;
      bv = v;
    }
  }
  return best;
}

__global__ void k_select(const double* __restrict__ L, int n_alpha, const float* __restrict__ S,
                         int64_t K, float* __restrict__ s_out, float* __restrict__ inv_out,
                         double* __restrict__ loss_out, int32_t* __restrict__ best_out) {
  const int best = argmin_finite(L, n_alpha);
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j == 0) {
    if (best_out) best_out[0] = best;
    if (loss_out)
      for (int i = 0; i < n_alpha; ++i) loss_out[i] = L[i];
  }
  if (best < 0 || j >= K) return;
  const float s = S[(int64_t)best * K + j];
  s_out[j] = s;
  if (inv_out) inv_out[j] = 1.0f / s;
}

}  // namespace awqk

namespace awq {

namespace {

// Candidates whose Gram-form losses one launch computes (error rows of each
// kept in the workspace): the uneven tiles of the triangle then fill the
// compute units better.
constexpr int kGramBatch = 4;

// Direct form: candidates per launch, as many as fit their error rows in this
// many bytes of workspace (small layers, where each candidate alone would be a
// launch of a few blocks: the 512 x 512 layer scores all 20 in one launch).
constexpr int64_t kDirectBatchBytes = int64_t(64) << 20;

// The Gram form (G = X^T X once, then per candidate a contraction with G
// carried as two fp16 parts, over the blocks on and below the diagonal only)
// replaces the T-long contraction when it costs well under half as many
// matrix-core operations and G (K^2 doubles, 6.6 GB at K = 28672, the widest
// Llama-70B input) stays within a few GB: K <= 32768.
// The Gram build addresses 256 token rows of the transposed tokens with
// 32-bit buffer offsets, so Tp stays below 2^23; longer calibration sets take
// the direct form.
bool search_uses_gram(int64_t N, int64_t K, int64_t T, int n_alpha) {
  if (K > 32768 || gram_tokens_padded(T) >= (int64_t(1) << 23)) return false;
  const double Tp = (double)gram_tokens_padded(T);
  const double g = (double)((K + awqk::kCT - 1) / awqk::kCT);
  const double direct = (double)n_alpha * 2.0 * (double)T * (double)N * (double)K;
  const double cand = 2.0 * (double)N * awqk::kCT * awqk::kCT * g * (g + 1.0);
  const double gram = 2.0 * Tp * (double)K * (double)K + (double)n_alpha * cand;
  return gram < 0.5 * direct;
}

struct SearchWs {
  float* S;
  float* IS;        // fp32(1 / S)
  int* pexp;
  uint16_t* E;
  double* partial;
  double* losses;
  uint16_t* Xh;     // bf16 tokens rounded to fp16 (direct form, bf16 input only)
  int* px;
  uint16_t* Xt;     // Gram form: tokens transposed
  float* Gp;        // Gram form: fp32 partial tiles of G per token chunk
  double* G;
  uint16_t* P;
  int* sk;
  bool gram;
  int nc;           // Gram form: candidates scored per loss launch
  size_t bytes;
};

SearchWs carve(void* ws, int dt, int64_t N, int64_t K, int64_t T, int n_alpha) {
  SearchWs w{};
  size_t off = 0;
  char* base = (char*)ws;
  auto take = [&](size_t b) {
    char* p = base ? base + off : nullptr;
    off += align_up(b, 256);
    return p;
  };
  w.gram = search_uses_gram(N, K, T, n_alpha);
  const int direct_nc = (int)std::max<int64_t>(1, std::min<int64_t>(n_alpha, kDirectBatchBytes / (N * K * 2)));
  w.nc = w.gram ? (n_alpha < kGramBatch ? n_alpha : kGramBatch) : direct_nc;
  w.S = (float*)take((size_t)n_alpha * K * 4);
  w.IS = (float*)take((size_t)n_alpha * K * 4);
  w.pexp = (int*)take((size_t)w.nc * N * 4);
  w.E = (uint16_t*)take((size_t)w.nc * N * K * 2);
  w.losses = (double*)take((size_t)n_alpha * 8);
  if (w.gram) {
    const int64_t Tp = gram_tokens_padded(T);
    w.partial = (double*)take((size_t)w.nc * gram_loss_tiles(N, K) * 8);
    w.Xt = (uint16_t*)take((size_t)K * Tp * 2);
    w.Gp = (float*)take((size_t)gram_partial_floats(T, K) * 4);
    w.G = (double*)take((size_t)K * K * 8);
    w.P = (uint16_t*)take((size_t)K * ((K + awqk::kCT - 1) / awqk::kCT * awqk::kCT) * 4);
    w.sk = (int*)take((size_t)K * 4);
  } else {
    const int64_t gx = (N + awqk::kCT - 1) / awqk::kCT;
    const int64_t gy = (T + awqk::kCT - 1) / awqk::kCT;
    w.partial = (double*)take((size_t)w.nc * gx * gy * 8);
    if (dt == awqk::DT_BF16) {
      w.Xh = (uint16_t*)take((size_t)T * K * 2);
      w.px = (int*)take((size_t)T * 4);
    }
  }
  w.bytes = off;
  return w;
}
}  // namespace

size_t search_ws_bytes(int dt, int64_t N, int64_t K, int64_t T, int n_alpha) {
  return carve(nullptr, dt, N, K, T, n_alpha).bytes;
}

hipError_t launch_search(const void* w, int dt, int64_t N, int64_t K, const void* x, int64_t T,
                         int64_t ldx, const float* mean_abs, const double* alphas, int n_alpha,
                         QuantVariant qv, const uint8_t* kept, float* s_out, float* inv_s_out,
                         double* loss_out, int32_t* best_out, void* ws, hipStream_t st) {
  using namespace awqk;
  const SearchWs sw = carve(ws, dt, N, K, T, n_alpha);
  const int64_t nS = (int64_t)n_alpha * K;
  hipLaunchKernelGGL(k_cand_scales, dim3((unsigned)((nS + 255) / 256)), dim3(256), 0, st, mean_abs,
                     alphas, n_alpha, K, sw.S, sw.IS);
  const double tn = (double)T * (double)N;
  // error rows of candidates cand .. cand + nb - 1 into slots 0 .. nb - 1 of
  // the workspace, one launch (blockIdx.y = slot)
  const QSpec q = qspec(qv.bits, qv.sym);
  auto err_gen = [&](int cand, int nb) {
    const float* s_i = sw.S + (int64_t)cand * K;
    const float* is_i = sw.IS + (int64_t)cand * K;
    uint16_t* E = sw.E;
    int* pe = sw.pexp;
    const uint16_t* W = (const uint16_t*)w;
    const dim3 grid((unsigned)N, (unsigned)nb);
#define AWQ_EG3(GL, GR, KP)                                                                         \
  if (dt == DT_F16)                                                                                 \
    hipLaunchKernelGGL((k_err_gen<DT_F16, GL, GR, KP>), grid, dim3(256), 0, st, W, N, K, s_i, is_i, q, kept, E, pe); \
  else                                                                                              \
    hipLaunchKernelGGL((k_err_gen<DT_BF16, GL, GR, KP>), grid, dim3(256), 0, st, W, N, K, s_i, is_i, q, kept, E, pe)
#define AWQ_EG2(GL, GR) \
  if (kept) { AWQ_EG3(GL, GR, true); } else { AWQ_EG3(GL, GR, false); }
#define AWQ_EG(GL)                                                                                  \
  if (q.sym) { AWQ_EG2(GL, kGridSym); }                                                             \
  else if (qv.bits == 4) { AWQ_EG2(GL, kGridQ4); }                                                  \
  else { AWQ_EG2(GL, kGridAsym); }
    if (qv.group == 64) { AWQ_EG(8); }
    else if (qv.group == 256) { AWQ_EG(32); }
    else { AWQ_EG(16); }
#undef AWQ_EG3
#undef AWQ_EG2
#undef AWQ_EG
  };
  if (qv.group != 64 && qv.group != 128 && qv.group != 256) return hipErrorInvalidValue;
  if (sw.gram) {
    const hipError_t e = launch_gram_prepare(x, dt, T, K, ldx, sw.Xt, sw.Gp, sw.G, sw.P, sw.sk, st);
    if (e != hipSuccess) return e;
    const int64_t nt = gram_loss_tiles(N, K);
    for (int i0 = 0; i0 < n_alpha; i0 += sw.nc) {
      const int nc = n_alpha - i0 < sw.nc ? n_alpha - i0 : sw.nc;
      err_gen(i0, nc);
      const hipError_t el = launch_gram_loss(sw.E, N, K, sw.pexp, sw.P, sw.sk, sw.partial, nc, st);
      if (el != hipSuccess) return el;
      hipLaunchKernelGGL(k_sum_partials, dim3((unsigned)nc), dim3(256), 0, st, sw.partial, nt, tn, sw.losses + i0);
    }
  } else {
    const uint16_t* Xop = (const uint16_t*)x;
    int64_t ldop = ldx;
    const int* px = nullptr;
    if (dt == DT_BF16) {
      hipLaunchKernelGGL((k_rows_f16<DT_BF16, false, false>), dim3((unsigned)T), dim3(256), 0, st,
                         (const uint16_t*)x, K, ldx, (const float*)nullptr, sw.Xh, sw.px);
      Xop = sw.Xh;
      ldop = K;
      px = sw.px;
    }
    const int64_t gx = (N + kCT - 1) / kCT;
    const int64_t gy = (T + kCT - 1) / kCT;
    for (int i0 = 0; i0 < n_alpha; i0 += sw.nc) {
      const int nc = n_alpha - i0 < sw.nc ? n_alpha - i0 : sw.nc;
      err_gen(i0, nc);
      hipLaunchKernelGGL(k_err_contract, dim3((unsigned)contract_blocks(T, N), (unsigned)nc), dim3(256), 0, st,
                         Xop, T, ldop, px, sw.E, N, K, sw.pexp, sw.partial);
      hipLaunchKernelGGL(k_sum_partials, dim3((unsigned)nc), dim3(256), 0, st, sw.partial, gx * gy, tn,
                         sw.losses + i0);
    }
  }
  hipLaunchKernelGGL(k_select, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st, sw.losses,
                     n_alpha, sw.S, K, s_out, inv_s_out, loss_out, best_out);
  return hipGetLastError();
}

}  // namespace awq
