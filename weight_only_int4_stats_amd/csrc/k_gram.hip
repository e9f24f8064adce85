// Gram form of the scale search's loss ("AWQ Math", section "Searching the
// scale -- no backprop required": each candidate is scored by the output error
// over the calibration tokens).  With E_i = W - W_hat_i and G = X^T X (K x K),
//     sum_t || E_i x_t ||^2 = sum_n e_n^T G e_n,
// so G is formed once and a candidate then costs a contraction of length 2K
// per (row, channel) instead of one of length T per (token, row); the search
// uses this form when the calibration set is much longer than a row.
//   1. k_transpose16  X [T][ldx] -> Xt [K][Tp] (tokens along rows, zero padded
//                     to Tp, a multiple of 256; the 16-bit values are copied)
//   2. k_gram         G (fp64) += Xt[:, chunk] Xt[:, chunk]^T on the matrix
//                     cores (shared contraction core): fp32 within a chunk of
//                     kGramChunk tokens, fp64 across chunks in a fixed order
//                     (one launch per chunk)
//   3. k_gram_split   per row k of G a power of two 2^s_k with
//                     max_j |G_kj| 2^-s_k in [2^14, 2^15), and
//                     P[k][j] = fp16(G_kj 2^-s_k), P[k][K + j] = fp16(G_kj 2^-s_k - P[k][j])
//                     (22 significant bits of each row relative to its largest entry)
//   4. k_gram_loss    per candidate: C = [E' E'] P^T (contraction over 2K, so
//                     C_nk = sum_j E'_nj G_kj 2^-s_k to 22 bits), E' = E 2^p_n as
//                     stored by the error generator; the epilogue adds
//                     E'_nk C_nk 2^(s_k - 2 p_n) over the tile in fp64 -> one
//                     partial per tile (summed in a fixed order afterwards).
#include "awq_device.h"
#include "awq_internal.h"
#include "k_contract.h"

namespace awqk {

constexpr int64_t kGramChunk = 8192;     // tokens per fp32 accumulation chunk

// 64 tokens x 64 channels per block of 256 threads; tokens past T are zeros.
__global__ __launch_bounds__(256) void k_transpose16(const uint16_t* __restrict__ X, int64_t T,
                                                     int64_t K, int64_t ldx,
                                                     uint16_t* __restrict__ Xt, int64_t Tp) {
  __shared__ uint16_t tile[64][72];
  const int64_t t0 = (int64_t)blockIdx.x * 64, k0 = (int64_t)blockIdx.y * 64;
  const int tid = threadIdx.x;
  {
    const int r = tid >> 2, c = (tid & 3) * 16;
    const int64_t t = t0 + r;
    u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
    if (t < T) {
      v0 = ldg128(X + t * ldx + k0 + c);
      v1 = ldg128(X + t * ldx + k0 + c + 8);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tile[r][c + 2 * j] = (uint16_t)(v0[j] & 0xFFFFu);
      tile[r][c + 2 * j + 1] = (uint16_t)(v0[j] >> 16);
      tile[r][c + 8 + 2 * j] = (uint16_t)(v1[j] & 0xFFFFu);
      tile[r][c + 8 + 2 * j + 1] = (uint16_t)(v1[j] >> 16);
    }
  }
  __syncthreads();
  {
    const int c = tid >> 2, r = (tid & 3) * 16;      // channel c, tokens r .. r + 15
    u32x4 o0, o1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o0[j] = (uint32_t)tile[r + 2 * j][c] | ((uint32_t)tile[r + 2 * j + 1][c] << 16);
      o1[j] = (uint32_t)tile[r + 8 + 2 * j][c] | ((uint32_t)tile[r + 8 + 2 * j + 1][c] << 16);
    }
    uint16_t* dst = Xt + (k0 + c) * Tp + t0 + r;
    *reinterpret_cast<u32x4*>(dst) = o0;
    *reinterpret_cast<u32x4*>(dst + 8) = o1;
  }
}

// One 256 x 256 tile of G per block (row tile gy = blockIdx / gx, column tile
// blockIdx % gx), tokens [c0, c0 + len) of Xt; G tile = (first ? 0 : G) + chunk.
template <int DT>
__global__ __launch_bounds__(256) void k_gram(const uint16_t* __restrict__ Xt, int64_t K, int64_t Tp,
                                              int64_t c0, int64_t len, int first,
                                              double* __restrict__ G) {
  __shared__ __attribute__((aligned(16))) uint8_t lds0[kCStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[kCStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds2[kCStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds3[kCStage];
  const int64_t gx = (K + kCT - 1) / kCT;
  const int64_t tj = blockIdx.x / gx, tk = blockIdx.x - tj * gx;
  const int64_t j0 = tj * kCT, k0 = tk * kCT;
  const int64_t rj = K - j0 < kCT ? K - j0 : kCT;
  const int64_t rk = K - k0 < kCT ? K - k0 : kCT;
  ContractSrc cs;
  cs.ars = rsrc4(Xt + j0 * Tp, (uint32_t)(rj * Tp * 2));
  cs.a_ld = (uint32_t)(Tp * 2);
  cs.brs = rsrc4(Xt + k0 * Tp, (uint32_t)(rk * Tp * 2));
  cs.b_ld = (uint32_t)(Tp * 2);
  cs.k0 = (uint32_t)(c0 * 2);
  cs.a_wrap = 0;
  cs.S = len / kCBK;
  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;
  contract_tile<DT == DT_BF16>(cs, lds0, lds1, lds2, lds3, acc);

  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int wm = wv >> 1, wn = wv & 1;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int64_t k = k0 + wn * 128 + nb * 32 + (lane & 31);
    if (k >= K) continue;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t j = j0 + wm * 128 + mb * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (j < K) {
          double* g = G + j * K + k;
          *g = (first ? 0.0 : *g) + (double)acc[mb][nb][v];
        }
      }
  }
}

// One block per row k of G.
__global__ __launch_bounds__(256) void k_gram_split(const double* __restrict__ G, int64_t K,
                                                    uint16_t* __restrict__ P, int* __restrict__ sk) {
  const int64_t k = blockIdx.x;
  const double* row = G + k * K;
  double mx = 0.0;
  for (int64_t j = threadIdx.x; j < K; j += 256) mx = fmax(mx, fabs(row[j]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmax(mx, __shfl_xor(mx, off));
  __shared__ double wmax[4];
  __shared__ int s_sh;
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double m = fmax(fmax(wmax[0], wmax[1]), fmax(wmax[2], wmax[3]));
    int s = 0;
    if (m > 0.0) {
      int ex;
      frexp(m, &ex);           // m < 2^ex
      s = ex - 15;             // m 2^-s in [2^14, 2^15)
    }
    s_sh = s;
    sk[k] = s;
  }
  __syncthreads();
  const int s = s_sh;
  uint16_t* prow = P + k * 2 * K;
  for (int64_t j = threadIdx.x; j < K; j += 256) {
    const double g = ldexp(row[j], -s);
    const uint32_t hi = f32_to_f16_bits((float)g);
    const double rest = g - (double)f16_to_f32(hi);
    prow[j] = (uint16_t)hi;
    prow[K + j] = (uint16_t)f32_to_f16_bits((float)rest);
  }
}

// Tile order as the direct contraction: L2 slice i mod 8 takes the x-th eighth
// of the tiles in band order (bands of 8 column tiles of k).
constexpr int kGBand = 8;
constexpr int kGXcds = 8;

inline int64_t gram_loss_blocks(int64_t N, int64_t K) {
  const int64_t tiles = ((N + kCT - 1) / kCT) * ((K + kCT - 1) / kCT);
  return kGXcds * ((tiles + kGXcds - 1) / kGXcds);
}

// partial[ty * gx + tx] for tile (row tile ty of E, column tile tx of k).
__global__ __launch_bounds__(256) void k_gram_loss(const uint16_t* __restrict__ E, int64_t N, int64_t K,
                                                   const int* __restrict__ pexp,
                                                   const uint16_t* __restrict__ P,
                                                   const int* __restrict__ sk,
                                                   double* __restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint8_t lds0[kCStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[kCStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds2[kCStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds3[kCStage];
  __shared__ double wsum[kCWaves];

  const int64_t gx = (K + kCT - 1) / kCT, gy = (N + kCT - 1) / kCT, tiles = gx * gy;
  const int64_t per = (tiles + kGXcds - 1) / kGXcds;
  const int64_t slot = blockIdx.x / kGXcds;
  const int64_t o = (int64_t)(blockIdx.x % kGXcds) * per + slot;
  if (slot >= per || o >= tiles) return;
  const int64_t band = o / (gy * kGBand);
  const int64_t rb = o - band * gy * kGBand;
  const int64_t bw = gx - band * kGBand < kGBand ? gx - band * kGBand : kGBand;
  const int64_t ty = rb / bw;
  const int64_t tx = band * kGBand + (rb - ty * bw);
  const int64_t n0 = ty * kCT;   // rows of E (MFMA A rows)
  const int64_t k0 = tx * kCT;   // rows of P (MFMA B rows) = output channels

  const int64_t rn = N - n0 < kCT ? N - n0 : kCT;
  const int64_t rk = K - k0 < kCT ? K - k0 : kCT;
  ContractSrc cs;
  cs.ars = rsrc4(E + n0 * K, (uint32_t)(rn * K * 2));
  cs.a_ld = (uint32_t)(K * 2);
  cs.brs = rsrc4(P + k0 * 2 * K, (uint32_t)(rk * K * 4));
  cs.b_ld = (uint32_t)(K * 4);
  cs.k0 = 0;
  cs.a_wrap = (uint32_t)(K * 2);
  cs.S = 2 * K / kCBK;
  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;
  contract_tile<false>(cs, lds0, lds1, lds2, lds3, acc);

  // epilogue: lane value v of block (mb, nb): channel k = k0 + wn 128 + nb 32 + lane % 32,
  // row n = n0 + wm 128 + mb 32 + 8 (v / 4) + 4 (lane / 32) + v % 4
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  double tot = 0.0;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    int pn[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int64_t n = n0 + wm * 128 + mb * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      pn[v] = pexp[n < N ? n : N - 1];
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int64_t k = k0 + wn * 128 + nb * 32 + (lane & 31);
      if (k >= K) continue;
      const int s = sk[k];
      double part = 0.0;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t n = n0 + wm * 128 + mb * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (n < N) {
          const double e = (double)f16_to_f32(E[n * K + k]);
          part += ldexp(e * (double)acc[mb][nb][v], -2 * pn[v]);
        }
      }
      tot += ldexp(part, s);
    }
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

}  // namespace awqk

namespace awq {

int64_t gram_tokens_padded(int64_t T) { return (T + 255) / 256 * 256; }

int64_t gram_loss_tiles(int64_t N, int64_t K) {
  return ((N + awqk::kCT - 1) / awqk::kCT) * ((K + awqk::kCT - 1) / awqk::kCT);
}

hipError_t launch_gram_prepare(const void* x, int dt, int64_t T, int64_t K, int64_t ldx,
                               uint16_t* Xt, double* G, uint16_t* P, int* sk, hipStream_t st) {
  using namespace awqk;
  const int64_t Tp = gram_tokens_padded(T);
  hipLaunchKernelGGL(k_transpose16, dim3((unsigned)(Tp / 64), (unsigned)(K / 64)), dim3(256), 0, st,
                     (const uint16_t*)x, T, K, ldx, Xt, Tp);
  const int64_t g = (K + kCT - 1) / kCT;
  for (int64_t c0 = 0; c0 < Tp; c0 += kGramChunk) {
    const int64_t len = Tp - c0 < kGramChunk ? Tp - c0 : kGramChunk;
    if (dt == DT_BF16)
      hipLaunchKernelGGL(k_gram<DT_BF16>, dim3((unsigned)(g * g)), dim3(256), 0, st, Xt, K, Tp, c0, len,
                         (int)(c0 == 0), G);
    else
      hipLaunchKernelGGL(k_gram<DT_F16>, dim3((unsigned)(g * g)), dim3(256), 0, st, Xt, K, Tp, c0, len,
                         (int)(c0 == 0), G);
  }
  hipLaunchKernelGGL(k_gram_split, dim3((unsigned)K), dim3(256), 0, st, G, K, P, sk);
  return hipGetLastError();
}

hipError_t launch_gram_loss(const uint16_t* E, int64_t N, int64_t K, const int* pexp,
                            const uint16_t* P, const int* sk, double* partial, hipStream_t st) {
  using namespace awqk;
  hipLaunchKernelGGL(k_gram_loss, dim3((unsigned)gram_loss_blocks(N, K)), dim3(256), 0, st, E, N, K,
                     pexp, P, sk, partial);
  return hipGetLastError();
}

}  // namespace awq
