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
//                   as awq_quantize_pack does, E = W - D (q - z) / s in float;
//                   a first pass finds max|E| of the row, a second writes
//                   E * 2^p (p chosen so the row fits fp16's normal range) as
//                   fp16 into the workspace, with p per row.
//   2. k_err_contract  128x128 tiles of C = X E'^T with fp16 MFMA (fp32
//                   accumulation); the epilogue squares and sums the tile,
//                   undoes the powers of two in double, and writes one double
//                   per tile.  bf16 calibration tokens are first rounded to
//                   fp16 with their own power-of-two scale (exact unless a
//                   value falls 2^24 below its token's largest).
//   3. k_sum_partials  fixed-order double sum of the tile partials -> L_i.
// Finally k_select picks the lowest index among the minimal finite losses and
// writes s, 1/s, the losses and the index.  Every sum has a fixed order, so
// the result is bit-reproducible.
#include "awq_device.h"
#include "awq_internal.h"
#include "k_rows_f16.h"

namespace awqk {

// ---------------------------------------------------------------------------
// candidate scales: S[i][j] = float(pow(max(double(m_j), 2^-14), alpha_i))
// ---------------------------------------------------------------------------
__global__ void k_cand_scales(const float* __restrict__ m, const double* __restrict__ alphas,
                              int n_alpha, int64_t K, float* __restrict__ S) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)n_alpha * K) return;
  const int64_t i = idx / K;
  const int64_t j = idx - i * K;
  const double b = fmax((double)m[j], 0x1p-14);
  S[idx] = (float)pow(b, alphas[i]);
}

// ---------------------------------------------------------------------------
// error generation
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ void err_word(const uint16_t* __restrict__ wrow,
                                         const float* __restrict__ s, int64_t k0, float e[8]) {
  const u32x4 raw = ldg128(wrow + k0);
  const f32x4 s0 = *reinterpret_cast<const f32x4*>(s + k0);
  const f32x4 s1 = *reinterpret_cast<const f32x4*>(s + k0 + 4);
  float w[8], sv[8], wp[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    w[2 * j] = lo_f32<DT>(raw[j]);
    w[2 * j + 1] = hi_f32<DT>(raw[j]);
    sv[j] = s0[j];
    sv[4 + j] = s1[j];
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) wp[j] = w[j] * sv[j];
  float mn = wp[0], mx = wp[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) {
    mn = fminf(mn, wp[j]);
    mx = fmaxf(mx, wp[j]);
  }
  seg16_minmax(mn, mx);
  const GroupGrid g = group_grid(mn, mx);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float q = quant_code(wp[j], g);
    const float grid = g.D * (q - g.z);            // exact: fp16 step x 4-bit integer
    e[j] = w[j] - grid / sv[j];
  }
}

template <int DT>
__global__ __launch_bounds__(256) void k_err_gen(const uint16_t* __restrict__ W, int64_t N,
                                                 int64_t K, const float* __restrict__ s,
                                                 uint16_t* __restrict__ E, int* __restrict__ pexp) {
  const int64_t n = blockIdx.x;
  const uint16_t* wrow = W + n * K;
  const int64_t wpr = K >> 3;
  float emax = 0.0f;
  // pass 1: largest |E| of the row (whole 16-lane segments are in or out)
  for (int64_t c0 = 0; c0 < wpr; c0 += 256) {
    const int64_t c = c0 + threadIdx.x;
    float e[8];
    if (c < wpr) {
      err_word<DT>(wrow, s, c * 8, e);
#pragma unroll
      for (int j = 0; j < 8; ++j) emax = fmaxf(emax, fabsf(e[j]));
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) emax = fmaxf(emax, __shfl_xor(emax, off));
  __shared__ float wmax[4];
  __shared__ int sp;
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
  const int p = sp;
  // pass 2: the same arithmetic again, scaled by 2^p and rounded to DT
  uint16_t* erow = E + n * K;
  for (int64_t c0 = 0; c0 < wpr; c0 += 256) {
    const int64_t c = c0 + threadIdx.x;
    if (c < wpr) {
      float e[8];
      err_word<DT>(wrow, s, c * 8, e);
      u32x4 out;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        out[j] = f32_to_f16_bits(ldexpf(e[2 * j], p)) | (f32_to_f16_bits(ldexpf(e[2 * j + 1], p)) << 16);
      *reinterpret_cast<u32x4*>(erow + c * 8) = out;
    }
  }
}

// ---------------------------------------------------------------------------
// contraction C = X E'^T, sum of squares per tile
// ---------------------------------------------------------------------------
constexpr int kCT = 256;        // tile edge (tokens and rows)
constexpr int kCBK = 64;        // k per LDS stage
constexpr int kCLd = kCBK + 8;  // LDS row stride in 16-bit elements (padding vs bank conflicts)

__device__ __forceinline__ f32x16 mfma32h(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// 256 tokens x 256 error rows per block of 8 waves (2 along tokens x 4 along
// rows; each wave 128 x 64 = 4 x 2 blocks of 32 x 32), 64 k per LDS stage, two
// stages so the next stage's loads overlap the current matrix-core work.
// px: per-token power of two of the fp16 tokens (NULL: tokens unscaled).
__global__ __launch_bounds__(512) void k_err_contract(const uint16_t* __restrict__ X, int64_t T,
                                                      int64_t ldx, const int* __restrict__ px,
                                                      const uint16_t* __restrict__ E, int64_t N,
                                                      int64_t K, const int* __restrict__ pexp,
                                                      double* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kCT * kCLd];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kCT * kCLd];
  __shared__ double wsum[8];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv >> 2, wn = wv & 3;
  const int64_t n0 = (int64_t)blockIdx.x * kCT;   // rows of E (MFMA columns)
  const int64_t t0 = (int64_t)blockIdx.y * kCT;   // tokens (MFMA rows)
  const int64_t S = K / kCBK;

  // per-thread sources: rows past T / N read row 0 and are excluded in the epilogue
  const uint16_t* asrc[4];
  const uint16_t* bsrc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 512 * i;
    const int64_t t = t0 + (c >> 3), n = n0 + (c >> 3);
    asrc[i] = X + (t < T ? t : 0) * ldx + (c & 7) * 8;
    bsrc[i] = E + (n < N ? n : 0) * K + (c & 7) * 8;
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

  u32x4 ra[4], rb[4];
  auto gload = [&](int64_t s) {
    const int64_t k0 = s * kCBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = ldg128(asrc[i] + k0);
      rb[i] = ldg128(bsrc[i] + k0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + 512 * i;
      const int off = (c >> 3) * kCLd + (c & 7) * 8;
      *reinterpret_cast<u32x4*>(&As[buf][off]) = ra[i];
      *reinterpret_cast<u32x4*>(&Bs[buf][off]) = rb[i];
    }
  };

  gload(0);
  lstore(0);
  __syncthreads();
  for (int64_t s = 0; s < S; ++s) {
    const int buf = (int)(s & 1);
    if (s + 1 < S) gload(s + 1);
#pragma unroll
    for (int ks = 0; ks < kCBK / 16; ++ks) {
      const int kk = ks * 16 + 8 * (lane >> 5);
      u32x4 a[4], b[2];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        a[mb] = *reinterpret_cast<const u32x4*>(&As[buf][(wm * 128 + mb * 32 + (lane & 31)) * kCLd + kk]);
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        b[nb] = *reinterpret_cast<const u32x4*>(&Bs[buf][(wn * 64 + nb * 32 + (lane & 31)) * kCLd + kk]);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32h(a[mb], b[nb], acc[mb][nb]);
    }
    if (s + 1 < S) lstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: every value a lane holds for block nb belongs to E row n;
  // token row of value v in block mb: 8 (v / 4) + 4 (lane / 32) + v % 4
  double tot = 0.0;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int64_t n = n0 + wn * 64 + nb * 32 + (lane & 31);
    if (n >= N) continue;
    double ssq = 0.0;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      float part = 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t t = t0 + wm * 128 + mb * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (t < T) {
          const float c = acc[mb][nb][v];
          if (px == nullptr) part += c * c;
          else ssq += ldexp((double)c * (double)c, -2 * px[t]);
        }
      }
      ssq += (double)part;
    }
    tot += ldexp(ssq, -2 * pexp[n]);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) tot += __shfl_xor(tot, off);
  if (lane == 0) wsum[wv] = tot;
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int w = 0; w < 8; ++w) t += wsum[w];
    partial[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = t;
  }
}

// Fixed-order sum of n doubles by one block of 256 threads -> out[0] = sum / denom.
__global__ __launch_bounds__(256) void k_sum_partials(const double* __restrict__ part, int64_t n,
                                                      double denom, double* __restrict__ out) {
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
struct SearchWs {
  float* S;
  int* pexp;
  uint16_t* E;
  double* partial;
  double* losses;
  uint16_t* Xh;     // bf16 tokens rounded to fp16 (bf16 input only)
  int* px;
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
  const int64_t gx = (N + awqk::kCT - 1) / awqk::kCT;
  const int64_t gy = (T + awqk::kCT - 1) / awqk::kCT;
  w.S = (float*)take((size_t)n_alpha * K * 4);
  w.pexp = (int*)take((size_t)N * 4);
  w.E = (uint16_t*)take((size_t)N * K * 2);
  w.partial = (double*)take((size_t)gx * gy * 8);
  w.losses = (double*)take((size_t)n_alpha * 8);
  if (dt == awqk::DT_BF16) {
    w.Xh = (uint16_t*)take((size_t)T * K * 2);
    w.px = (int*)take((size_t)T * 4);
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
                         float* s_out, float* inv_s_out, double* loss_out, int32_t* best_out,
                         void* ws, hipStream_t st) {
  using namespace awqk;
  const SearchWs sw = carve(ws, dt, N, K, T, n_alpha);
  const int64_t nS = (int64_t)n_alpha * K;
  hipLaunchKernelGGL(k_cand_scales, dim3((unsigned)((nS + 255) / 256)), dim3(256), 0, st, mean_abs,
                     alphas, n_alpha, K, sw.S);
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
  const double tn = (double)T * (double)N;
  for (int i = 0; i < n_alpha; ++i) {
    const float* s_i = sw.S + (int64_t)i * K;
    if (dt == DT_F16)
      hipLaunchKernelGGL(k_err_gen<DT_F16>, dim3((unsigned)N), dim3(256), 0, st,
                         (const uint16_t*)w, N, K, s_i, sw.E, sw.pexp);
    else
      hipLaunchKernelGGL(k_err_gen<DT_BF16>, dim3((unsigned)N), dim3(256), 0, st,
                         (const uint16_t*)w, N, K, s_i, sw.E, sw.pexp);
    hipLaunchKernelGGL(k_err_contract, dim3((unsigned)gx, (unsigned)gy), dim3(512), 0, st, Xop, T,
                       ldop, px, sw.E, N, K, sw.pexp, sw.partial);
    hipLaunchKernelGGL(k_sum_partials, dim3(1), dim3(256), 0, st, sw.partial, gx * gy, tn,
                       sw.losses + i);
  }
  hipLaunchKernelGGL(k_select, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st, sw.losses,
                     n_alpha, sw.S, K, s_out, inv_s_out, loss_out, best_out);
  return hipGetLastError();
}

}  // namespace awq
