// Gram form of the scale search's loss ("AWQ Math", section "Searching the
// scale -- no backprop required": each candidate is scored by the output error
// over the calibration tokens).  With E_i = W - W_hat_i and G = X^T X (K x K),
//     sum_t || E_i x_t ||^2 = sum_n e_n^T G e_n,
// so G is formed once and a candidate then costs a contraction of length 2K
// per (row, channel) instead of one of length T per (token, row); the search
// uses this form when the calibration set is much longer than a row.
//   1. k_transpose16  X [T][ldx] -> Xt [K][Tp] (tokens along rows, zero padded
//                     to Tp, a multiple of 256; the 16-bit values are copied)
//   2. k_gram         one item per (tile of G on or above the diagonal, chunk
//                     of at most kGramChunk tokens): Xt[:, chunk] Xt[:, chunk]^T
//                     on the matrix cores (shared contraction core) in fp32,
//                     written as an fp32 partial tile; the chunk length is
//                     chosen so that the items fill kGramCUs compute units
//                     evenly.  k_gram_reduce adds a tile's chunks in fp64 in
//                     chunk order and writes it and its mirror image into G
//                     (chunks are taken in groups whose partials fit
//                     kGramPartialMax; later groups add to G in the same order).
//   3. k_gram_split   per row k of G a power of two 2^s_k with
//                     max_j |G_kj| 2^-s_k in [2^14, 2^15), and the fp16 pair
//                     hi = fp16(g), lo = fp16(g - hi) of g = G_kj 2^-s_k (22
//                     significant bits of each row relative to its largest
//                     entry), halved when j and k fall in the same 256-wide
//                     block.  Row k of P holds, per 256-wide block b of j,
//                     the 256 hi values then the 256 lo values (zeros past K).
//   4. k_gram_loss    per candidate, with the symmetry of G:
//                        e^T G e = sum_J sum_{I <= J} w_IJ e_I^T G_IJ e_J,
//                     w = 1 off the diagonal blocks counted once each way
//                     (doubling the sum, halving the diagonal blocks).  Output
//                     tile (row tile of E', channel block J) contracts over
//                     the blocks I <= J only: C_nk = sum_{j in blocks <= J}
//                     E'_nj P'_kj (hi and lo, A's block read twice), about half
//                     the work of the full product.  E' = E 2^p_n as stored by
//                     the error generator; the epilogue adds
//                     E'_nk C_nk 2^(s_k + 1 - 2 p_n) over the tile in fp64 ->
//                     one partial per tile (summed in a fixed order afterwards).
#include "awq_device.h"
#include "awq_internal.h"
#include "k_contract.h"

namespace awqk {

constexpr int64_t kGramChunk = 8192;     // most tokens per fp32 accumulation chunk
constexpr int64_t kGramCUs = 256;        // compute units the chunking is planned for
constexpr int64_t kGramPartialMax = int64_t(1) << 30;   // bytes of fp32 partial tiles per launch
constexpr int64_t kGramTile = (int64_t)kCT * kCT;   // floats per partial tile

// Tile u (0 .. g (g + 1) / 2 - 1) of G on or above the diagonal, row-major
// over the upper triangle: (tj, tk) with tj <= tk.
__device__ __forceinline__ void gram_upper_tile(int64_t u, int64_t g, int64_t& tj, int64_t& tk) {
  int64_t r = 0, len = g;
  while (u >= len) {
    u -= len;
    ++r;
    --len;
  }
  tj = r;
  tk = r + u;
}

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

// Item b: chunk cfirst + c of len tokens (c = b / nup; the last chunk may be
// shorter), upper tile u = b mod nup.  The fp32 tile goes to Gp[(c nup + u)] in the
// register order of the contraction core (value i of thread t at i 256 + t),
// which k_gram_reduce reads back with the same order.
template <int DT>
__global__ __launch_bounds__(256) void k_gram(const uint16_t* __restrict__ Xt, int64_t K, int64_t Tp,
                                              int64_t len, int64_t cfirst, float* __restrict__ Gp) {
  __shared__ __attribute__((aligned(16))) uint8_t lds0[kCStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[kCStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds2[kCStage];
  __shared__ __attribute__((aligned(16))) uint8_t lds3[kCStage];
  const int64_t g = (K + kCT - 1) / kCT, nup = g * (g + 1) / 2;
  const int64_t c = blockIdx.x / nup, u = blockIdx.x - c * nup;
  int64_t tj, tk;
  gram_upper_tile(u, g, tj, tk);
  const int64_t j0 = tj * kCT, k0 = tk * kCT;
  const int64_t rj = K - j0 < kCT ? K - j0 : kCT;
  const int64_t rk = K - k0 < kCT ? K - k0 : kCT;
  const int64_t t0 = (cfirst + c) * len;
  ContractSrc cs;
  cs.ars = rsrc4(Xt + j0 * Tp, (uint32_t)(rj * Tp * 2));
  cs.a_ld = (uint32_t)(Tp * 2);
  cs.brs = rsrc4(Xt + k0 * Tp, (uint32_t)(rk * Tp * 2));
  cs.b_ld = (uint32_t)(Tp * 2);
  cs.k0 = (uint32_t)(t0 * 2);
  cs.a_dup_sh = 0;
  cs.S = (Tp - t0 < len ? Tp - t0 : len) / kCBK;
  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;
  contract_tile<DT == DT_BF16>(cs, lds0, lds1, lds2, lds3, acc);
  float* out = Gp + (c * nup + u) * kGramTile + threadIdx.x;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) out[((mb * 4 + nb) * 16 + v) * 256] = acc[mb][nb][v];
}

// Block (u, q): upper tile u, 32 x 32 sub-block q = 4 mb + nb of every
// wave's quarter.  G_jk = (first ? 0 : G_jk) + the fp32 partials of the
// group's nch chunks, added in fp64 in chunk order; an off-diagonal tile also
// fills its mirror G_kj.
__global__ __launch_bounds__(256) void k_gram_reduce(const float* __restrict__ Gp, int64_t K,
                                                     int64_t nch, int first, double* __restrict__ G) {
  const int64_t g = (K + kCT - 1) / kCT, nup = g * (g + 1) / 2;
  const int64_t u = blockIdx.x >> 4;
  const int q = blockIdx.x & 15, mb = q >> 2, nb = q & 3;
  int64_t tj, tk;
  gram_upper_tile(u, g, tj, tk);
  const int lane = threadIdx.x & 63;
  const int wv = threadIdx.x >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int64_t k = tk * kCT + wn * 128 + nb * 32 + (lane & 31);
  const int64_t jb = tj * kCT + wm * 128 + mb * 32 + 4 * (lane >> 5);
  const float* in = Gp + u * kGramTile + q * 16 * 256 + threadIdx.x;
  double sum[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t j = jb + 8 * (v >> 2) + (v & 3);
    sum[v] = first || j >= K || k >= K ? 0.0 : G[j * K + k];
  }
  for (int64_t c = 0; c < nch; ++c) {
    const float* pc = in + c * nup * kGramTile;
#pragma unroll
    for (int v = 0; v < 16; ++v) sum[v] += (double)pc[v * 256];
  }
  if (k >= K) return;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int64_t j = jb + 8 * (v >> 2) + (v & 3);
    if (j < K) {
      G[j * K + k] = sum[v];
      if (tj != tk) G[k * K + j] = sum[v];
    }
  }
}

// One block per row k of G; Kp = K rounded up to a multiple of 256.
__global__ __launch_bounds__(256) void k_gram_split(const double* __restrict__ G, int64_t K,
                                                    int64_t Kp, uint16_t* __restrict__ P,
                                                    int* __restrict__ sk) {
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
  const int64_t kb = k / kCT;
  uint16_t* prow = P + k * 2 * Kp;
  for (int64_t j = threadIdx.x; j < Kp; j += 256) {
    const int64_t b = j / kCT, c = j - b * kCT;
    // exact: a power-of-two scaling (halving for the diagonal block)
    const double g = j < K ? ldexp(row[j], -s - (b == kb ? 1 : 0)) : 0.0;
    const uint32_t hi = f32_to_f16_bits((float)g);
    const double rest = g - (double)f16_to_f32(hi);
    prow[b * 2 * kCT + c] = (uint16_t)hi;
    prow[b * 2 * kCT + kCT + c] = (uint16_t)f32_to_f16_bits((float)rest);
  }
}

// nc candidates per launch (error rows of candidate c at E + c N K, row
// exponents at pexp + c N, tile partials at partial + c gx gy), so that the
// uneven tiles of the triangle fill the compute units.  Tiles longest first:
// block o takes channel block J = gx - 1 - o / (nc gy), then candidate and
// row tile (consecutive blocks share J's rows of P).
inline int64_t gram_loss_blocks(int64_t N, int64_t K, int nc) {
  return ((N + kCT - 1) / kCT) * ((K + kCT - 1) / kCT) * nc;
}

// partial[c gx gy + ty gx + tx] for tile (row tile ty of E, column tile tx of k)
// of candidate c.
__global__ __launch_bounds__(256) void k_gram_loss(const uint16_t* __restrict__ E, int64_t N, int64_t K,
                                                   const int* __restrict__ pexp,
                                                   const uint16_t* __restrict__ P,
                                                   const int* __restrict__ sk,
                                                   double* __restrict__ partial, int nc) {
  // one array for the four stages, so that the epilogue can use 66.5 KB of it at once
  __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kCStage];
  __shared__ __attribute__((aligned(16))) int sks[kCT];
  __shared__ double wsum[kCWaves];

  const int64_t gx = (K + kCT - 1) / kCT, gy = (N + kCT - 1) / kCT;
  const int64_t o = blockIdx.x;
  const int64_t tx = gx - 1 - o / (nc * gy);
  const int64_t rest = o - (gx - 1 - tx) * nc * gy;
  const int64_t cand = rest / gy;
  const int64_t ty = rest - cand * gy;
  const int64_t Kp = gx * kCT;
  E += cand * N * K;
  pexp += cand * N;
  partial += cand * gx * gy;
  const int64_t n0 = ty * kCT;   // rows of E (MFMA A rows)
  const int64_t k0 = tx * kCT;   // rows of P (MFMA B rows) = output channels

  const int64_t rn = N - n0 < kCT ? N - n0 : kCT;
  const int64_t rk = K - k0 < kCT ? K - k0 : kCT;
  ContractSrc cs;
  cs.ars = rsrc4(E + n0 * K, (uint32_t)(rn * K * 2));
  cs.a_ld = (uint32_t)(K * 2);
  cs.brs = rsrc4(P + k0 * 2 * Kp, (uint32_t)(rk * Kp * 4));
  cs.b_ld = (uint32_t)(Kp * 4);
  cs.k0 = 0;
  cs.a_dup_sh = 9;                       // 256 fp16 of E serve a hi and a lo block
  cs.S = (tx + 1) * 2 * kCT / kCBK;      // blocks 0..J, hi and lo
  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;
  contract_tile<false>(cs, lds, lds + kCStage, lds + 2 * kCStage, lds + 3 * kCStage, acc);

  // Epilogue: the tile's sum of E'_nk C_nk 2^(s_k + 1 - 2 p_n) in double (the + 1
  // undoes the halved diagonal blocks).  Lane value v of accumulator block
  // (mb, nb) is tile row wm 128 + mb 32 + 8 (v / 4) + 4 (lane / 32) + v % 4,
  // column wn 128 + nb 32 + lane % 32.  Pass mb writes the 64 tile rows
  // mb 32 + 0..31 and 128 + mb 32 + 0..31 to LDS as fp32 rows of kEpiLd floats;
  // thread t then takes pass row t % 64 and the 64 columns 64 (t / 64) + 0..63,
  // its error values read 16 bytes at a time (past the ends: 0).
  constexpr int kEpiLd = 260;    // a 16-lane read pass (16 rows) covers all 64 banks
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  float* ct = reinterpret_cast<float*>(lds);
  for (int t = tid; t < kCT; t += 256) sks[t] = k0 + t < K ? sk[k0 + t] : 0;
  const uint64_t ea = (uint64_t)(uintptr_t)(E + n0 * K);
  const uint32_t ea_lo = __builtin_amdgcn_readfirstlane((uint32_t)ea);
  const uint32_t ea_hi = __builtin_amdgcn_readfirstlane((uint32_t)(ea >> 32));
  const __amdgpu_buffer_rsrc_t ers = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(((uint64_t)ea_hi << 32) | ea_lo), (short)0,
      __builtin_amdgcn_readfirstlane((int)(rn * K * 2)), kBufferWord3);
  const int q = tid & 63, cg = tid >> 6;
  double tot = 0.0;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    __syncthreads();             // every wave done with the stages / the previous pass
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        ct[r * kEpiLd + wn * 128 + nb * 32 + (lane & 31)] = acc[mb][nb][v];
      }
    __syncthreads();
    const int nl = (q >> 5) * 128 + mb * 32 + (q & 31);   // tile row of pass row q
    const int64_t n = n0 + nl;
    const int pn = pexp[n < N ? n : N - 1];
    u32x4 e8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = cg * 64 + 8 * j;
      const bool ok = nl < rn && k0 + c < K;               // K is a multiple of 8
      e8[j] = __builtin_amdgcn_raw_buffer_load_b128(
          ers, ok ? (uint32_t)(((int64_t)nl * K + k0 + c) * 2) : kBufferOob, 0, 0);
    }
    double part = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = cg * 64 + 8 * j;
      const f32x4 c0 = *reinterpret_cast<const f32x4*>(ct + q * kEpiLd + c);
      const f32x4 c1 = *reinterpret_cast<const f32x4*>(ct + q * kEpiLd + c + 4);
      const i32x4 s0 = *reinterpret_cast<const i32x4*>(sks + c);
      const i32x4 s1 = *reinterpret_cast<const i32x4*>(sks + c + 4);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float cv = i < 4 ? c0[i] : c1[i - 4];
        const int sc = i < 4 ? s0[i] : s1[i - 4];
        const double e = (double)f16_to_f32((e8[j][i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
        part += ldexp(e * (double)cv, sc);
      }
    }
    tot += ldexp(part, 1 - 2 * pn);
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

// Chunk plan of the Gram build: the chunk length (a multiple of 128 tokens, at
// most kGramChunk) whose items, upper tiles x chunks, take the fewest
// rounds x length on kGramCUs compute units; chunks go in groups of cg per
// launch so that a group's partial tiles fit kGramPartialMax.
struct GramPlan {
  int64_t len, nch, cg, nup;
};

GramPlan gram_plan(int64_t T, int64_t K) {
  using namespace awqk;
  const int64_t Tp = gram_tokens_padded(T);
  const int64_t g = (K + kCT - 1) / kCT, nup = g * (g + 1) / 2;
  const int64_t tile_bytes = kGramTile * 4;
  int64_t cg_max = kGramPartialMax / (nup * tile_bytes);
  if (cg_max < 1) cg_max = 1;
  const int64_t n0 = (Tp + kGramChunk - 1) / kGramChunk;
  GramPlan best{0, 0, 0, nup};
  int64_t best_cost = 0;
  for (int64_t n = n0; n <= 2 * n0; ++n) {
    const int64_t len = ((Tp + n - 1) / n + 127) / 128 * 128;
    const int64_t nch = (Tp + len - 1) / len;
    const int64_t cg = nch < cg_max ? nch : cg_max;
    int64_t rounds = 0;
    for (int64_t c = 0; c < nch; c += cg) {
      const int64_t m = nch - c < cg ? nch - c : cg;
      rounds += (nup * m + kGramCUs - 1) / kGramCUs;
    }
    const int64_t cost = rounds * (len + 128);     // + per-item fill and store
    if (best.nch == 0 || cost < best_cost) {
      best = GramPlan{len, nch, cg, nup};
      best_cost = cost;
    }
  }
  return best;
}

int64_t gram_partial_floats(int64_t T, int64_t K) {
  const GramPlan pl = gram_plan(T, K);
  return pl.nup * pl.cg * awqk::kGramTile;
}

hipError_t launch_gram_prepare(const void* x, int dt, int64_t T, int64_t K, int64_t ldx,
                               uint16_t* Xt, float* Gp, double* G, uint16_t* P, int* sk,
                               hipStream_t st) {
  using namespace awqk;
  const int64_t Tp = gram_tokens_padded(T);
  hipLaunchKernelGGL(k_transpose16, dim3((unsigned)(Tp / 64), (unsigned)(K / 64)), dim3(256), 0, st,
                     (const uint16_t*)x, T, K, ldx, Xt, Tp);
  const int64_t g = (K + kCT - 1) / kCT;
  const GramPlan pl = gram_plan(T, K);
  for (int64_t c = 0; c < pl.nch; c += pl.cg) {
    const int64_t m = pl.nch - c < pl.cg ? pl.nch - c : pl.cg;
    const dim3 grid((unsigned)(pl.nup * m));
    if (dt == DT_BF16)
      hipLaunchKernelGGL(k_gram<DT_BF16>, grid, dim3(256), 0, st, Xt, K, Tp, pl.len, c, Gp);
    else
      hipLaunchKernelGGL(k_gram<DT_F16>, grid, dim3(256), 0, st, Xt, K, Tp, pl.len, c, Gp);
    hipLaunchKernelGGL(k_gram_reduce, dim3((unsigned)(pl.nup * 16)), dim3(256), 0, st, Gp, K, m, (int)(c == 0), G);
  }
  hipLaunchKernelGGL(k_gram_split, dim3((unsigned)K), dim3(256), 0, st, G, K, g * kCT, P, sk);
  return hipGetLastError();
}

hipError_t launch_gram_loss(const uint16_t* E, int64_t N, int64_t K, const int* pexp,
                            const uint16_t* P, const int* sk, double* partial, int nc,
                            hipStream_t st) {
  using namespace awqk;
  hipLaunchKernelGGL(k_gram_loss, dim3((unsigned)gram_loss_blocks(N, K, nc)), dim3(256), 0, st, E, N, K,
                     pexp, P, sk, partial, nc);
  return hipGetLastError();
}

}  // namespace awq
