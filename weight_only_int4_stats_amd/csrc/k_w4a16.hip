// Fused W4A16 product ("AWQ > Benefits and Practical Considerations": the
// dequantization unpacks 4-bit integers, applies a group scale and zero point
// and optionally the per-channel inverse scale, fused with the matrix
// multiply so the fp16 weight matrix is never materialised).
//
//   y[m][n] = sum_k step[n][g(k)] * (q[n][k] - z[n][g(k)]) * x[m][k] * r[k]
//
// Kernels (the batch-1 GEMV kernels live in their own source):
//
// * k_gemm_skinny_cu (M <= 16, activations fit in LDS): one block of 16 waves
//   per compute unit stages x * r as fp16 once and runs
//   v_mfma_f32_16x16x32_f16 with 16 weight rows as A and the tokens as B.
// * k_gemm_skinny (M <= 16 otherwise): the same MFMA mapping, one block per
//   16 weight rows, activations from a pre-pass.
// * k_gemm (M > 16): fp16 matrix-core GEMM on 256x256 output tiles.  A
//   pre-pass rounds each activation row x * r, scaled by an exact power of
//   two, to fp16 (exact for bf16 input without 1/s) in the order the nibble
//   unpack produces; the same launch picks a power of two per weight row so
//   that step * 15 stays inside fp16.  Each lane dequantizes its packed word
//   to step * (q - z) rounded once to fp16 and feeds v_mfma_f32_16x16x32_f16;
//   the epilogue undoes both powers of two exactly.
#include "awq_device.h"
#include "awq_internal.h"
#include "k_rows_f16.h"

namespace awqk {

template <int YDT>
__device__ __forceinline__ void store_y(void* y, int64_t idx, float v) {
  if constexpr (YDT == DT_F32) reinterpret_cast<float*>(y)[idx] = v;
  else reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)from_f32<YDT>(v);
}

// ===========================================================================
// matrix-core GEMM
// ===========================================================================

// Per weight row n: e_n with max_g step[n][g] 2^e_n in [2^-10, 2^-9),
// so that D' = step 2^e_n times 2^24 is a finite fp16 and D' (q - z) a normal
// fp16; then, for every group g, the fp16 constants of the packed-fma
// dequantization, group-major so a block's columns are contiguous:
//   ctab[g][n] = (fp16(D' 2^24) | fp16(D' 2^20) << 16, fp16(-D' z) twice).
constexpr int kConstRows = 16;   // weight rows per block of the constants pre-pass
__device__ __forceinline__ void gemm_consts_block(int64_t bid, const uint16_t* __restrict__ scales,
                                                  const uint8_t* __restrict__ zeros, int64_t N,
                                                  int64_t G, int* __restrict__ en,
                                                  uint32_t* __restrict__ ctab) {
  // 16 rows per block of 256 threads, 16 consecutive lanes per row: lane p
  // of a row takes its groups [p G / 16, (p + 1) G / 16), first for the row's
  // largest step (combined over the 16 lanes with shuffles), then for the
  // constants.  Every block is one short round of loads and stores, so the
  // pass keeps up with the activation rows beside it.
  const int tid = threadIdx.x;
  const int rl = tid >> 4, p = tid & 15;
  const int64_t n = bid * kConstRows + rl;
  const bool ok = n < N;
  const int64_t g0 = p * G / 16, g1 = (p + 1) * G / 16;
  const uint16_t* sr = scales + (ok ? n : 0) * G;
  const uint8_t* zr = zeros + (ok ? n : 0) * G;
  float mx = 0.0f;
  if (ok)
    for (int64_t g = g0; g < g1; ++g) mx = fmaxf(mx, f16_to_f32(sr[g]));
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  int e = 0;
  if (mx > 0.0f) {
    int ex;
    frexpf(mx, &ex);          // mx < 2^ex
    e = -9 - ex;              // mx 2^e in [2^-10, 2^-9)
  }
  if (!ok) return;
  if (p == 0) en[n] = e;
  for (int64_t g = g0; g < g1; ++g) {
    const float D = ldexpf(f16_to_f32(sr[g]), e);   // exact: power-of-two scaling
    const uint32_t h24 = f32_to_f16_bits(D * 16777216.0f);
    const uint32_t h20 = f32_to_f16_bits(D * 1048576.0f);
    const uint32_t hz = f32_to_f16_bits(-(D * (float)zr[g]));
    *reinterpret_cast<uint2*>(ctab + (g * N + n) * 2) = make_uint2(h24 | (h20 << 16), hz | (hz << 16));
  }
}


// One packed word (codes of k = 8c + j in bits 4j..4j+3) -> 8 fp16 operands
// D' (q - z), k order (0,4 | 2,6 | 1,5 | 3,7).  The masked nibbles are read
// as fp16 subnormals q 2^-24 (nibbles 1/3/5/7 still 4 bits up: q 2^-20); one
// packed fma with the fp16 constants D' 2^24 (or D' 2^20) and -D' z gives
// D' q - D' z with one rounding.  Shift, 4 ands and 4 fmas per word.
__device__ __forceinline__ u32x4 dequant_word_f16(uint32_t w, f16x2 c24, f16x2 c20, f16x2 nzd) {
  const uint32_t w8 = w >> 8;
  u32x4 out;
  out[0] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(
      __builtin_bit_cast(f16x2, w & 0x000F000Fu), c24, nzd));
  out[1] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(
      __builtin_bit_cast(f16x2, w8 & 0x000F000Fu), c24, nzd));
  out[2] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(
      __builtin_bit_cast(f16x2, w & 0x00F000F0u), c20, nzd));
  out[3] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(
      __builtin_bit_cast(f16x2, w8 & 0x00F000F0u), c20, nzd));
  return out;
}

// The same from the constant table's two words: cx = D' 2^24 | D' 2^20 << 16
// and nzd = -D' z twice (the broadcasts of cx's halves fold into the packed
// fma's operand selection).
__device__ __forceinline__ u32x4 dequant_word_f16(uint32_t w, uint32_t cx, uint32_t nzd) {
  const f16x2 c = as_f16x2(cx);
  return dequant_word_f16(w, __builtin_shufflevector(c, c, 0, 0), __builtin_shufflevector(c, c, 1, 1),
                          as_f16x2(nzd));
}
// 256 x 256 output tile per block of 8 waves (2 along m x 4 along n, each wave
// 128 x 64 = 8 x 4 blocks of 16 x 16: the 16 x 16 x 32 product moves half the
// accumulator data per flop of the 32 x 32 x 16 one and runs at a higher clock
// under the chip's power limit; 256 x 128 tiles, 128 x 32 per wave, fill a
// last round of tiles), 64 k per stage, three LDS stages
// filled by LDS DMA (buffer_load ... lds) two stages ahead of the matrix-core
// work:
//   A  256 rows x 64 k of fp16 activations, row r's 16-byte chunk c stored at
//      chunk c ^ a_swz(r)
//   B  256 columns x 8 packed words; per 32 columns the first 16 bytes of
//      each column, then the last 16
//   C  256 columns of dequantization constants (8 bytes each)
// Operand k order: in k32 step st, lane group h (lanes 16 h .. 16 h + 15) holds
// packed word 2 h + st of its column (8 k), so that its two words are one
// 8-byte LDS read per stage, and reads A chunk 2 h + st to match.
// All three are plain (temporal) copies: a packed column's 128-byte line
// serves four consecutive stages, and the activation and weight stages are
// shared by the blocks that run on one L2 slice at the same time.  Tiles are
// ordered for the chip's eight L2 slices: block i runs on slice i mod 8, and
// slice x takes the x-th eighth of the tiles in a grouped order (4 m-tiles,
// m fastest, then n), so its ~32 concurrent blocks cover about 4 x 8 tiles.
// The GEMM's two pre-passes in one launch (they are independent): the first
// ceil(N / 16) blocks build the constants, the other M convert one activation
// row each.
// KEEP: activation chunks per thread held in registers (16: rows up to 32768).
template <int DT, bool HAS_R, int KEEP>
__global__ __launch_bounds__(256) void k_gemm_prep(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                   int64_t ldx, const float* __restrict__ r,
                                                   uint16_t* __restrict__ xq, int* __restrict__ pm,
                                                   const uint16_t* __restrict__ scales,
                                                   const uint8_t* __restrict__ zeros, int64_t N, int64_t G,
                                                   int* __restrict__ en, uint32_t* __restrict__ ctab) {
  const int64_t nc = (N + kConstRows - 1) / kConstRows;
  if ((int64_t)blockIdx.x < nc) gemm_consts_block(blockIdx.x, scales, zeros, N, G, en, ctab);
  else rows_f16_block<DT, HAS_R, true, KEEP>((int64_t)blockIdx.x - nc, x, K, ldx, r, xq, pm);
}

// Position of an A row's 16-byte chunks in LDS: chunk c of row r at
// c ^ a_swz(r) = c ^ ((r / 2) mod 8): the 16 rows one 16-lane group reads
// land on 16 different 16-byte slots of a 256-byte span.  The bank-conflict
// counter shows that a 128-bit read is served 8 lanes per 128 bytes, so this
// layout is 2-way conflicted within each 8-lane group; (r ^ (r / 8)) mod 8
// removes the conflicts (counter at 0.6 % of the LDS busy cycles, from 44 %)
// but measured 0.3-1 % slower on the 70B prefill shapes (the LDS is not what
// limits this loop), so the layout stays.
__device__ __forceinline__ int a_swz(int r) { return (r >> 1) & 7; }

constexpr int kMT = 256;                // tile rows (m)
constexpr int kBK = 64;                 // k per stage
constexpr int kXcds = 8;                // L2 slices (block i -> slice i mod 8)
constexpr int kAStage = kMT * kBK * 2;  // 32 KB

// A tile of 256 rows x 64 NB columns: each of the 8 waves takes 128 rows x
// 16 NB columns (NB = 4: 256-wide tiles; NB = 2: 128-wide tiles, same k loop)
template <int NB>
struct GemmTile {
  static constexpr int NT = 64 * NB;             // tile columns
  static constexpr int BStage = NT * 8 * 4;      // packed words
  static constexpr int CStage = NT * 8;          // dequantization constants
  static constexpr int Stage = kAStage + BStage + CStage;
  static constexpr int BWaves = NT / 32;         // waves copying packed columns (32 each)
  static constexpr int CWaves = NT / 128;        // waves copying constants (128 columns each)
};
constexpr int kStageMax = GemmTile<4>::Stage;

// How the columns are cut: [0, nsplit) in 256-wide tiles, [nsplit, N) in
// 128-wide ones.  A compute unit holds one block, so the launch runs in rounds
// of one tile per unit; a 128-wide tile takes about half as long as a 256-wide
// one.  The cut is chosen to minimise the estimated rounds, so that a last
// round that would be partly empty (896 tiles of the 2048 x 28672 product on
// 256 units: 3.5 rounds) is spread over twice as many half-width tiles.
struct GemmPlan {
  int64_t nsplit, wide_tiles, narrow_tiles, wide_blocks, blocks;
};

inline GemmPlan gemm_plan(int64_t M, int64_t N) {
  const int64_t cus = awq::device_cus() > 0 ? awq::device_cus() : 256;
  const int64_t mt = (M + kMT - 1) / kMT, ntw = (N + 255) / 256;
  auto rounds = [&](int64_t t) { return (double)((t + cus - 1) / cus); };
  GemmPlan best{};
  double best_cost = 1e300;
  for (int64_t a = ntw; a >= 0; --a) {
    const int64_t ns = a * 256 < N ? a * 256 : N;
    const int64_t tw = mt * a, th = mt * ((N - ns + 127) / 128);
    const double cost = rounds(tw) + 0.55 * rounds(th) + (tw > 0 && th > 0 ? 0.02 : 0.0);
    if (cost < best_cost) {
      best_cost = cost;
      best.nsplit = ns;
      best.wide_tiles = tw;
      best.narrow_tiles = th;
    }
  }
  best.wide_blocks = kXcds * ((best.wide_tiles + kXcds - 1) / kXcds);
  best.blocks = best.wide_blocks + kXcds * ((best.narrow_tiles + kXcds - 1) / kXcds);
  return best;
}

// One output tile of width 64 NB over the columns [nb, ne): tile t of that
// region in grouped order.
template <int YDT, int NB>
__device__ __forceinline__ void gemm_tile(uint8_t* __restrict__ lds0, uint8_t* __restrict__ lds1,
                                          uint8_t* __restrict__ lds2, int64_t t,
                                          const uint16_t* __restrict__ xq, int64_t M, int64_t K,
                                          const int* __restrict__ pm, const uint32_t* __restrict__ qw,
                                          const uint32_t* __restrict__ ctab, const int* __restrict__ en,
                                          int64_t N, int64_t nb, int64_t ne, void* __restrict__ y,
                                          int64_t ldy, int glog, int vec_ok) {
  using Tl = GemmTile<NB>;
  constexpr int NT = Tl::NT;
  const int64_t ntile = (ne - nb + NT - 1) / NT, mtile = (M + kMT - 1) / kMT;
  // tile t in grouped order: 4 m-tiles at a time, m fastest, so the ~32
  // blocks a slice runs at once cover about 4 x 8 tiles and share both
  // operands in its L2
  const int64_t g = t / (4 * ntile);
  const int64_t rr = t - g * 4 * ntile;
  const int64_t gm = mtile - g * 4 < 4 ? mtile - g * 4 : 4;
  const int64_t mt = g * 4 + rr % gm;
  const int64_t m0 = mt * kMT;
  const int64_t n0 = nb + (rr / gm) * NT;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv >> 2, wn = wv & 3;
  const int64_t G = K >> glog;                 // groups of 2^glog >= kBK channels per row
  const int64_t S = K / kBK;
  const int rows = (int)(M - m0 < kMT ? M - m0 : kMT);
  const int cols = (int)(ne - n0 < NT ? ne - n0 : NT);
  const i32x4 ars = rsrc4(xq + m0 * K, (uint32_t)(rows * K * 2));
  const i32x4 brs = rsrc4(qw + n0 * (K >> 3), (uint32_t)(cols * (K >> 1)));
  const i32x4 crs = rsrc4(ctab + n0 * 2, (uint32_t)(((G - 1) * N + cols) * 8));
  // copies per stage issued by this wave: 4 A, 1 B (waves < BWaves), 1 C (waves < CWaves)
  const int nops = 4 + (wv < Tl::BWaves ? 1 : 0) + (wv < Tl::CWaves ? 1 : 0);

  // A copy j (0..31) fills LDS bytes [1024 j, 1024 j + 1024) = rows 8 j .. 8 j + 7;
  // wave w issues j = 4 w + u.  Lane i: row r = 8 j + i / 8 at LDS chunk i % 8,
  // which holds global chunk (i % 8) ^ a_swz(r).
  uint32_t aoff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 8 * (4 * wv + u) + (lane >> 3);
    aoff[u] = (uint32_t)(r * K * 2 + (((lane & 7) ^ a_swz(r)) * 16));
  }
  // B: wave w copies columns 32 w .. 32 w + 31; lane i takes half i / 32 of
  // column 32 w + i % 32
  const uint32_t boff = (uint32_t)((32 * wv + (lane & 31)) * (K >> 1) + (lane >> 5) * 16);
  // C: wave w copies columns 128 w .. 128 w + 127 (two columns per lane)
  const uint32_t coff = (uint32_t)((wv * 128 + lane * 2) * 8);

  // copy u of stage s into the stage array at base: u 0..3 the wave's A rows,
  // 4 its B columns and constants
  auto copy = [&](int64_t s, const uint8_t* base, int u) {
    const uint32_t k0 = (uint32_t)(s * kBK);
    const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_addr(base));
    if (u < 4) {
      dma16(ars, lb + (4 * wv + u) * 1024, aoff[u], k0 * 2);
    } else {
      if (wv < Tl::BWaves) dma16(brs, lb + kAStage + wv * 1024, boff, k0 >> 1);
      if (wv < Tl::CWaves)
        dma16(crs, lb + kAStage + Tl::BStage + wv * 1024, coff, (uint32_t)((k0 >> glog) * N * 8));
    }
  };
  auto issue = [&](int64_t s, const uint8_t* base) {
#pragma unroll
    for (int u = 0; u < 5; ++u) copy(s, base, u);
  };
  // wait until only the copies of the newest stage are in flight (and, with
  // lgkm, every LDS access of the wave has completed)
  auto wait_stage = [&](bool lgkm) {
    if (lgkm) {
      if (nops == 6) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(6));
      else if (nops == 5) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(5));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(4));
    } else {
      if (nops == 6) __builtin_amdgcn_s_waitcnt(waitcnt_vm(6));
      else if (nops == 5) __builtin_amdgcn_s_waitcnt(waitcnt_vm(5));
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(4));
    }
  };

  f32x4 acc[8][NB];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[a][b][v] = 0.0f;

  // 16 x 16 x 32 products.  Operand k order: lane group h = lane / 16 holds
  // packed words 2 h (step 0) and 2 h + 1 (step 1) of its column, one 8-byte
  // LDS read per stage, and A chunk 2 h + st to match.  Sub-step q = 2 st + hh
  // multiplies the row blocks 4 hh .. 4 hh + 3 with the NB column blocks; the
  // next sub-step's four A fragments are read meanwhile.
  struct Raw { uint2 c[NB]; uint2 w[NB]; };
  auto load_raw = [&](const uint8_t* base, Raw& w) {
    const int h = lane >> 4;
#pragma unroll
    for (int nbk = 0; nbk < NB; ++nbk) {
      const int col = wn * 16 * NB + nbk * 16 + (lane & 15);
      w.c[nbk] = *reinterpret_cast<const uint2*>(base + kAStage + Tl::BStage + col * 8);
      w.w[nbk] = *reinterpret_cast<const uint2*>(base + kAStage + (col >> 5) * 1024 + (h >> 1) * 512 +
                                                 (col & 31) * 16 + (h & 1) * 8);
    }
  };
  auto load_a = [&](const uint8_t* base, int q, u32x4 (&a)[4]) {
    const int st = q >> 1, hh = q & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 128 + (hh * 4 + i) * 16 + (lane & 15);
      a[i] = *reinterpret_cast<const u32x4*>(base + r * 128 + (((2 * (lane >> 4) + st) ^ a_swz(r)) * 16));
    }
  };

  Raw R;                // a stage's packed words and constants, straight from LDS
  u32x4 aE[4], aO[4];   // fragments of even and odd sub-steps
  u32x4 bq[NB];         // dequantized column blocks of the current k32 step
  issue(0, lds0);
  issue(1, lds1);
  wait_stage(false);
  lds_barrier();
  load_a(lds0, 0, aE);
  load_raw(lds0, R);
#pragma unroll
  for (int nbk = 0; nbk < NB; ++nbk) bq[nbk] = dequant_word_f16(R.w[nbk].x, R.c[nbk].x, R.c[nbk].y);

  // One stage (64 k) in four sub-steps q = 2 st + hh.  The operands of k32
  // step 0 are ready when the stage starts.  In sub-step 1 each column block's
  // operands are replaced by step 1's as soon as its last product has been
  // issued, and in sub-step 3 by the next stage's step 0 (its words and
  // constants read right after the barrier), so the dequantization runs
  // between the matrix products, three vector instructions after each from
  // the fourth on, instead of ahead of them.
  auto stage = [&](int64_t s, const uint8_t* cur, const uint8_t* nxt, const uint8_t* nxt2) {
    const bool cp = s + 2 < S;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (cp) {
        copy(s + 2, nxt2, q);
        if (q == 3) copy(s + 2, nxt2, 4);
      }
      if (q < 3) {
        load_a(cur, q + 1, (q & 1) ? aE : aO);
      } else {
        if (cp) wait_stage(true);
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
        lds_barrier();
        load_a(nxt, 0, aE);
        load_raw(nxt, R);
      }
      __builtin_amdgcn_sched_barrier(0);
      const u32x4 (&a)[4] = (q & 1) ? aO : aE;
      const int hh = q & 1;
#pragma unroll
      for (int nbk = 0; nbk < NB; ++nbk) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[hh * 4 + i][nbk] = mfma16h(a[i], bq[nbk], acc[hh * 4 + i][nbk]);
        if (q & 1) bq[nbk] = dequant_word_f16(q == 1 ? R.w[nbk].y : R.w[nbk].x, R.c[nbk].x, R.c[nbk].y);
      }
      if (q & 1) {
#pragma unroll
        for (int i = 0; i < 4 * NB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one matrix product
          if (i >= 3) __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // three vector instructions
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  for (int64_t s = 0; s < S; s += 3) {
    stage(s, lds0, lds1, lds2);
    if (s + 1 < S) stage(s + 1, lds1, lds2, lds0);
    if (s + 2 < S) stage(s + 2, lds2, lds0, lds1);
  }

  // 16x16 accumulator layout: column = lane % 16, row = 4 (lane / 16) + v.
  // Each wave stages its 128 x 16 NB outputs through a private LDS area, 32
  // rows at a time, and stores whole row pieces with 16-byte stores; the row
  // pitch is padded by 16 bytes so that the writes of the four lane groups
  // (rows 4 apart) fall on different banks.  Unaligned outputs, and columns
  // of a ragged last tile, are stored one by one.
  constexpr int kWc = 16 * NB;                            // columns per wave
  constexpr int kEs = YDT == DT_F32 ? 4 : 2;              // output bytes
  constexpr int kRowB = kWc * kEs;                        // bytes of a row piece
  constexpr int kLd = kRowB + 16;                         // padded LDS pitch
  constexpr int kLpr = kRowB / 16;                        // lanes per row
  constexpr int kRpi = 64 / kLpr;                         // rows per read pass
  static_assert(4 * 32 * kLd <= Tl::Stage, "four waves' staging in one stage array");
  static_assert(32 % kRpi == 0, "read passes cover the 32 staged rows");
  int en_l[NB];
#pragma unroll
  for (int nbk = 0; nbk < NB; ++nbk) {
    const int64_t n = n0 + wn * kWc + nbk * 16 + (lane & 15);
    en_l[nbk] = n < ne ? en[n] : 0;
  }
  if (!vec_ok) {
#pragma unroll
    for (int nbk = 0; nbk < NB; ++nbk) {
      const int64_t n = n0 + wn * kWc + nbk * 16 + (lane & 15);
      if (n >= ne) continue;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int64_t m = m0 + wm * 128 + mb * 16 + 4 * (lane >> 4) + v;
          if (m < M) store_y<YDT>(y, m * ldy + n, ldexpf(acc[mb][nbk][v], -(pm[m] + en_l[nbk])));
        }
    }
    return;
  }
  __syncthreads();                                        // every wave done with the stages
  uint8_t* stg = (wv < 4 ? lds0 : lds1) + (wv & 3) * 32 * kLd;
#pragma unroll
  for (int hp = 0; hp < 4; ++hp) {                        // rows wm 128 + hp 32 + 0..31
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int mb = 2 * hp + h;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = h * 16 + 4 * (lane >> 4) + v;       // staging row
        const int64_t m = m0 + wm * 128 + mb * 16 + 4 * (lane >> 4) + v;
        const int pmm = m < M ? pm[m] : 0;
#pragma unroll
        for (int nbk = 0; nbk < NB; ++nbk) {
          const float o = ldexpf(acc[mb][nbk][v], -(pmm + en_l[nbk]));
          uint8_t* dst = stg + r * kLd + (nbk * 16 + (lane & 15)) * kEs;
          if constexpr (YDT == DT_F32) *reinterpret_cast<float*>(dst) = o;
          else *reinterpret_cast<uint16_t*>(dst) = (uint16_t)from_f32<YDT>(o);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);                   // lgkmcnt(0): the wave's writes landed
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 32 / kRpi; ++i) {
      const int r = i * kRpi + lane / kLpr;
      const int cb = (lane % kLpr) * 16;                  // byte offset in the row piece
      const u32x4 val = *reinterpret_cast<const u32x4*>(stg + r * kLd + cb);
      const int64_t m = m0 + wm * 128 + hp * 32 + r;
      const int64_t n = n0 + wn * kWc + cb / kEs;
      if (m < M) {
        uint8_t* out = reinterpret_cast<uint8_t*>(y) + (m * ldy + n) * kEs;
        if (n + 16 / kEs <= ne) {
          *reinterpret_cast<u32x4*>(out) = val;
        } else {
#pragma unroll
          for (int j = 0; j < 16 / kEs; ++j)
            if (n + j < ne) {
              if constexpr (YDT == DT_F32) reinterpret_cast<uint32_t*>(out)[j] = val[j];
              else reinterpret_cast<uint16_t*>(out)[j] = (uint16_t)(val[j >> 1] >> (16 * (j & 1)));
            }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// The whole product in one launch: blocks [0, wide_blocks) take the 256-wide
// tiles of columns [0, nsplit), the rest the 128-wide tiles of [nsplit, N).
// Within each part, block i runs on L2 slice i mod 8, and slice x takes the
// x-th eighth of that part's tiles.
template <int YDT>
__global__ __launch_bounds__(512) void k_gemm(const uint16_t* __restrict__ xq, int64_t M, int64_t K,
                                             const int* __restrict__ pm,
                                             const uint32_t* __restrict__ qw,
                                             const uint32_t* __restrict__ ctab,
                                             const int* __restrict__ en, int64_t N,
                                             void* __restrict__ y, int64_t ldy, int glog, int vec_ok,
                                             int64_t nsplit, int64_t wide_tiles, int64_t wide_blocks,
                                             int64_t narrow_tiles) {
  // three LDS arrays, the loop unrolled by three: each stage is a known array
  __shared__ __attribute__((aligned(16))) uint8_t lds0[kStageMax];
  __shared__ __attribute__((aligned(16))) uint8_t lds1[kStageMax];
  __shared__ __attribute__((aligned(16))) uint8_t lds2[kStageMax];
  const int64_t b = blockIdx.x;
  if (b < wide_blocks) {
    const int64_t per = (wide_tiles + kXcds - 1) / kXcds, slot = b / kXcds;
    const int64_t t = (b % kXcds) * per + slot;
    if (slot >= per || t >= wide_tiles) return;
    gemm_tile<YDT, 4>(lds0, lds1, lds2, t, xq, M, K, pm, qw, ctab, en, N, 0, nsplit, y, ldy, glog, vec_ok);
  } else {
    const int64_t bn = b - wide_blocks;
    const int64_t per = (narrow_tiles + kXcds - 1) / kXcds, slot = bn / kXcds;
    const int64_t t = (bn % kXcds) * per + slot;
    if (slot >= per || t >= narrow_tiles) return;
    gemm_tile<YDT, 2>(lds0, lds1, lds2, t, xq, M, K, pm, qw, ctab, en, N, nsplit, N, y, ldy, glog, vec_ok);
  }
}

// ===========================================================================
// skinny matrix-core product (2 <= M <= 16)
// ===========================================================================
// One block of 4 waves per 16 output channels; wave w takes a quarter of the
// groups.  v_mfma_f32_16x16x32_f16 with the weights as A (16 channels x 32 k)
// and the activations as B (32 k x 16 tokens, tokens >= M read as 0).  Lane
// (row l % 16, block b = l / 16) loads chunk 4 g + b of its row (one 128-bit
// load per group) and feeds word i of it to the MFMA of step i; the B lane
// (token l % 16, block b) loads the matching 8 fp16 activations of chunk
// 4 g + b.  A unit g of 128 input channels is four such steps; a lane's chunk
// lies in one weight group (a unit holds one group of 128, half of one of 256
// or two of 64), whose step and zero point turn into the lane's packed-fma
// constants.  The per-row power of two e_n (as in the
// GEMM) is found from the row's steps in a prologue; the four waves' 16 x 16
// partial tiles are added in LDS in a fixed order.
constexpr int kSkW = 4;                 // waves per block (K quarters)
constexpr int kSkP = 2;                 // groups in flight per wave
constexpr int64_t kSkMaxM = 16;         // tokens per B tile


template <int YDT, int P>
__global__ __launch_bounds__(256) void k_gemm_skinny(const uint16_t* __restrict__ xq, int M, int64_t K,
                                                     const int* __restrict__ pm,
                                                     const uint32_t* __restrict__ qw,
                                                     const uint16_t* __restrict__ scales,
                                                     const uint8_t* __restrict__ zeros, int64_t N,
                                                     void* __restrict__ y, int64_t ldy, int glog) {
  __shared__ float red[kSkW][16 * 16];
  __shared__ float rmax[kSkW][16];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rl = lane & 15;                      // A row / B token
  const int b = lane >> 4;                       // k block
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int nrows = (int)(N - n0 < 16 ? N - n0 : 16);
  const int G = (int)(K >> 7);                   // 128-channel units (4 MFMA steps each)
  const int GW = (int)(K >> glog);               // weight groups per row
  const int csh = glog - 5;                      // 32-code chunk -> weight group
  const int g0 = (int)((int64_t)wv * G / kSkW), g1 = (int)((int64_t)(wv + 1) * G / kSkW);
  const uint32_t KW = (uint32_t)(K >> 3);
  const bool rowok = rl < nrows;

  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(qw + n0 * KW), (short)0, nrows * (int)KW * 4, kBufferWord3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(scales + n0 * GW), (short)0, nrows * GW * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(zeros + n0 * GW), (short)0, nrows * GW, kBufferWord3);
  const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)xq, (short)0, M * (int)K * 2, kBufferWord3);

  // ---- slot loads for group g (rows / tokens out of range read 0)
  // first piece of the row's steps for the power of two (issued before the
  // group loads: vector memory returns in order)
  const int npc = (GW * 2 + 15) / 16;            // 16-byte pieces of a row's steps
  const uint32_t srow = (uint32_t)rl * (uint32_t)GW * 2;
  const u32x4 sp0 = __builtin_amdgcn_raw_buffer_load_b128(srs, rowok && b < npc ? srow + 16 * b : kBufferOob, 0, 0);

  u32x4 wa[P], xb[P][4];
  uint32_t sr[P], zr[P];
  // the lane's chunk 4 g + b lies in weight group (4 g + b) >> csh
  auto load_group = [&](int slot, int g) {
    const bool ok = g < g1;
    const uint32_t woff = (uint32_t)rl * KW * 4 + (uint32_t)(4 * g + b) * 16;
    const uint32_t gw = (uint32_t)(rl * GW + ((4 * g + b) >> csh));
    wa[slot] = __builtin_amdgcn_raw_buffer_load_b128(wrs, ok && rowok ? woff : kBufferOob, 0, kBufferNt);
    sr[slot] = __builtin_amdgcn_raw_buffer_load_b16(srs, ok && rowok ? gw * 2 : kBufferOob, 0, 0);
    zr[slot] = __builtin_amdgcn_raw_buffer_load_b8(zrs, ok && rowok ? gw : kBufferOob, 0, 0);
    const uint32_t xoff = ((uint32_t)rl * (uint32_t)K + (uint32_t)(128 * g + 32 * b)) * 2;
    const bool xok = ok && rl < M;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      xb[slot][i] = __builtin_amdgcn_raw_buffer_load_b128(xrs, xok ? xoff + 16 * i : kBufferOob, 0, 0);
  };
#pragma unroll
  for (int d = 0; d < P; ++d) load_group(d, g0 + d);
  __builtin_amdgcn_sched_barrier(0);

  // ---- per-row power of two from the row's largest step (all groups; a
  // piece past the row's end may hold the next row's steps or read 0)
  auto piece_max = [&](const u32x4& v, int pc, float m) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (pc * 8 + j < GW) m = fmaxf(m, f16_to_f32((v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu));
    return m;
  };
  float mx = piece_max(sp0, b, 0.0f);
  for (int pc = b + 4; pc < npc; pc += 4)
    mx = piece_max(__builtin_amdgcn_raw_buffer_load_b128(srs, rowok ? srow + 16 * pc : kBufferOob, 0, 0), pc, mx);
  {
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  }
  int e = 0;
  if (mx > 0.0f) {
    int ex;
    frexpf(mx, &ex);
    e = -9 - ex;                                 // max step 2^e in [2^-10, 2^-9)
  }

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int gb = g0; gb < g1; gb += P) {
#pragma unroll
    for (int d = 0; d < P; ++d) {
      if (gb + d >= g1) break;                   // wave-uniform
      const float D = ldexpf(f16_to_f32(sr[d]), e);
      const uint32_t h24 = f32_to_f16_bits(D * 16777216.0f);
      const uint32_t h20 = f32_to_f16_bits(D * 1048576.0f);
      const uint32_t hz = f32_to_f16_bits(-(D * (float)zr[d]));
      const f16x2 c24 = as_f16x2(h24 | (h24 << 16));
      const f16x2 c20 = as_f16x2(h20 | (h20 << 16));
      const f16x2 nzd = as_f16x2(hz | (hz << 16));
#pragma unroll
      for (int i = 0; i < 4; ++i) acc = mfma16h(dequant_word_f16(wa[d][i], c24, c20, nzd), xb[d][i], acc);
    }
    if (gb + P >= g1) break;                     // wave-uniform
#pragma unroll
    for (int d = 0; d < P; ++d) load_group(d, gb + P + d);
  }

  // ---- add the four K quarters; 16 x 16 layout: token = lane % 16, row = 4 (lane / 16) + v
#pragma unroll
  for (int v = 0; v < 4; ++v) red[wv][(4 * b + v) * 16 + rl] = acc[v];
  if (b == 0) rmax[wv][rl] = (float)e;
  __syncthreads();
  const int t = threadIdx.x;                     // one (row, token) per thread
  const int row = t >> 4, tok = t & 15;
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < kSkW; ++w) tot += red[w][t];
  if (row < nrows && tok < M)
    store_y<YDT>(y, (int64_t)tok * ldy + n0 + row, ldexpf(tot, -(pm[tok] + (int)rmax[0][row])));
}

struct GemmWs {
  uint16_t* xq;
  int* pm;
  int* en;
  uint32_t* ctab;
  size_t bytes;
};

inline GemmWs gemm_ws(void* ws, int64_t M, int64_t N, int64_t K, int group) {
  GemmWs w{};
  char* base = (char*)ws;
  size_t off = 0;
  auto take = [&](size_t b) {
    char* p = base ? base + off : nullptr;
    off += awq::align_up(b, 256);
    return p;
  };
  w.xq = (uint16_t*)take((size_t)M * K * 2);
  w.pm = (int*)take((size_t)M * 4);
  w.en = (int*)take((size_t)N * 4);
  w.ctab = (uint32_t*)take((size_t)N * (K / group) * 8);
  w.bytes = off;
  return w;
}

template <int DT, int YDT, bool HAS_R>
hipError_t gemm_dispatch(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint32_t* qw,
                         const uint16_t* scales, const uint8_t* zeros, int64_t N, int glog,
                         const float* r, void* y, int64_t ldy, void* ws, hipStream_t st) {
  const GemmWs w = gemm_ws(ws, M, N, K, 1 << glog);
  const dim3 pgrid((unsigned)(M + (N + kConstRows - 1) / kConstRows));
  if (K > 256 * 8 * kRowsKeep)
    hipLaunchKernelGGL((k_gemm_prep<DT, HAS_R, 2 * kRowsKeep>), pgrid, dim3(256), 0, st, x, M, K, ldx, r,
                       w.xq, w.pm, scales, zeros, N, K >> glog, w.en, w.ctab);
  else
    hipLaunchKernelGGL((k_gemm_prep<DT, HAS_R, kRowsKeep>), pgrid, dim3(256), 0, st, x, M, K, ldx, r,
                       w.xq, w.pm, scales, zeros, N, K >> glog, w.en, w.ctab);
  // 16-byte output stores need a 16-byte aligned y and row pitch
  const int es = YDT == DT_F32 ? 4 : 2;
  const int vec_ok = ((uintptr_t)y % 16 == 0) && ((ldy * es) % 16 == 0);
  const GemmPlan pl = gemm_plan(M, N);
  hipLaunchKernelGGL((k_gemm<YDT>), dim3((unsigned)pl.blocks), dim3(512), 0, st, w.xq, M, K, w.pm,
                     qw, w.ctab, w.en, N, y, ldy, glog, vec_ok, pl.nsplit, pl.wide_tiles, pl.wide_blocks,
                     pl.narrow_tiles);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Skinny product, one block of 16 waves per compute unit (2 <= M <= 16, the
// M x K activations in LDS).  The block converts x * r to fp16 once, with an
// exact power of two per (token, 128-channel unit) from the unit's largest
// |x r| (so every unit sits in fp16's normal range) and the eight elements of
// every packed word in the unpack order.  Block b owns output rows
// [b N / B, (b + 1) N / B), cut into 16-row tiles; with t tiles each tile's
// units are split into S = 16 / t slices and wave w takes the items
// (tile, slice) w, w + 16, ...  Per unit a lane loads one 128-bit chunk of
// its row plus the step and zero point of the chunk's weight group, reads the
// matching activations from LDS, runs the unit's four MFMAs into a fresh
// 16 x 16 tile and adds it with the unit's activation scale 2^-p.  Slices of
// a tile are added in LDS in a fixed order.
// ---------------------------------------------------------------------------
constexpr int kScWaves = 16;
constexpr size_t kScRedBytes = (size_t)kScWaves * 256 * 4;      // per-item 16 x 16 partial tiles
constexpr int kScMaxPieces = 8;                                 // staged 8-element pieces per thread

inline size_t skinny_cu_lds(int64_t M, int64_t K, int64_t rows_max) {
  const int64_t ntile = (rows_max + 15) / 16;
  return (size_t)(M + 1) * (K + 8) * 2 + (size_t)(M + 1) * (K / 128) * 4 + kScRedBytes +
         (size_t)ntile * 16 * 4;
}

template <int DT, int YDT, bool HAS_R, int NP, int P>
__global__ __launch_bounds__(1024) void k_gemm_skinny_cu(
    const uint16_t* __restrict__ x, int M, int64_t K, int64_t ldx, const float* __restrict__ r,
    const uint32_t* __restrict__ qw, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zeros, int64_t N, void* __restrict__ y, int64_t ldy, int glog) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds_sc[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rl = lane & 15;
  const int b = lane >> 4;
  const uint32_t K8 = (uint32_t)(K >> 3);
  const int G = (int)(K >> 7);                   // 128-channel units (4 MFMA steps each)
  const int GW = (int)(K >> glog);               // weight groups per row
  const int csh = glog - 5;                      // 32-code chunk -> weight group
  const uint32_t KW = (uint32_t)(K >> 3);
  const int64_t r0 = (int64_t)blockIdx.x * N / gridDim.x;
  const int nrows = (int)((int64_t)(blockIdx.x + 1) * N / gridDim.x - r0);
  const int ntile = (nrows + 15) / 16;
  int ksl = kScWaves / (ntile > 0 ? ntile : 1);
  ksl = ksl < 1 ? 1 : (ksl > G ? G : ksl);
  const int nitems = ntile * ksl;

  // token rows K + 8 halves apart: the 16 tokens of a 128-bit read hit
  // different banks
  const int64_t KP = K + 8;
  uint16_t* xs = reinterpret_cast<uint16_t*>(lds_sc);                       // [M + 1][KP] (row M = 0)
  float* pinv = reinterpret_cast<float*>(lds_sc + (M + 1) * KP / 2);       // [M + 1][G] 2^-p
  float* red = pinv + (M + 1) * G;                                          // [16][256]
  int* erow = reinterpret_cast<int*>(red + kScWaves * 256);                 // [ntile][16]

  // ---- staging loads (issued first).  Thread t takes piece k8 = t mod K/8 of
  // the tokens t / (K/8), t / (K/8) + T, ... (T = 1024 / (K/8) token phases),
  // so 1/s is read once per piece; for K/8 > 1024 it walks k8 = t, t + 1024 ...
  const uint32_t T = K8 <= 1024u ? 1024u / K8 : 1u;
  const uint32_t tph = K8 <= 1024u ? (uint32_t)tid / K8 : 0u;
  const uint32_t k80 = K8 <= 1024u ? (uint32_t)tid - tph * K8 : (uint32_t)tid;
  const uint32_t ntok = tph < T ? ((uint32_t)M > tph ? ((uint32_t)M - tph + T - 1) / T : 0u) : 0u;
  const uint32_t nk = K8 <= 1024u ? 1u : (K8 - (uint32_t)tid + 1023u) / 1024u;   // k8 steps (K/8 > 1024)
  u32x4 sx[NP];
  f32x4 sr0[NP], sr1[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    // piece i: k8 step i / ntok_max ... with one token phase per thread for K/8 <= 1024
    const uint32_t j = (uint32_t)i;
    const bool live = K8 <= 1024u ? j < ntok : j < nk * (uint32_t)M;
    const uint32_t m = K8 <= 1024u ? tph + j * T : j % (uint32_t)M;
    const uint32_t k8 = K8 <= 1024u ? k80 : k80 + 1024u * (j / (uint32_t)M);
    if (live) {
      sx[i] = ldg128(x + (int64_t)m * ldx + (int64_t)k8 * 8);
      // with K / 8 <= 1024 every piece of the thread has the same k8, so 1/s is
      // read once (piece 0) and reused
      if (HAS_R && (K8 > 1024u || i == 0)) {
        sr0[i] = *reinterpret_cast<const f32x4*>(r + (int64_t)k8 * 8);
        sr1[i] = *reinterpret_cast<const f32x4*>(r + (int64_t)k8 * 8 + 4);
      }
    }
  }

  // ---- first item's weights in flight
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(qw + r0 * KW), (short)0, nrows * (int)KW * 4, kBufferWord3);
  const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(scales + r0 * GW), (short)0, nrows * GW * 2, kBufferWord3);
  const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(zeros + r0 * GW), (short)0, nrows * GW, kBufferWord3);
  int it = wv;
  int tile = 0, g0 = 0, g1 = 0;
  auto set_item = [&](int item) {
    tile = item / ksl;
    const int ks = item - tile * ksl;
    g0 = (int)((int64_t)ks * G / ksl);
    g1 = (int)((int64_t)(ks + 1) * G / ksl);
  };
  u32x4 wa[P];
  uint32_t sr[P], zr[P];
  bool have = it < nitems;                        // wave-uniform: this wave has an item
  auto load_group = [&](int slot, int g) {
    const int row = tile * 16 + rl;
    const bool ok = have && g < g1 && row < nrows;
    const uint32_t gw = (uint32_t)(row * GW + ((4 * g + b) >> csh));    // the chunk's weight group
    wa[slot] = __builtin_amdgcn_raw_buffer_load_b128(
        wrs, ok ? (uint32_t)row * KW * 4 + (uint32_t)(4 * g + b) * 16 : kBufferOob, 0, kBufferNt);
    sr[slot] = __builtin_amdgcn_raw_buffer_load_b16(srs, ok ? gw * 2 : kBufferOob, 0, 0);
    zr[slot] = __builtin_amdgcn_raw_buffer_load_b8(zrs, ok ? gw : kBufferOob, 0, 0);
  };
  // 16-byte pieces of the row's steps, for the row's power of two
  const int npc = (GW * 2 + 15) / 16;
  auto load_piece = [&](int pc) {
    const int row = tile * 16 + rl;
    return __builtin_amdgcn_raw_buffer_load_b128(
        srs, have && row < nrows && pc < npc ? (uint32_t)row * GW * 2 + 16 * pc : kBufferOob, 0, 0);
  };
  // branch-free (a wave without an item reads out of range): a conditional
  // block of loads here would make every later wait count all of them
  set_item(have ? it : 0);
  u32x4 sp0 = load_piece(b);
#pragma unroll
  for (int d = 0; d < P; ++d) load_group(d, g0 + d);
  __builtin_amdgcn_sched_barrier(0);

  // ---- stage fp16(x r 2^p) in unpack order (0,4,2,6,1,5,3,7) with p per
  // (token, 128-channel unit): the unit's 16 pieces sit in 16 consecutive lanes
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const uint32_t j = (uint32_t)i;
    const bool live = K8 <= 1024u ? j < ntok : j < nk * (uint32_t)M;
    if (K8 <= 1024u ? j >= (((uint32_t)M + T - 1) / T) : j >= ((K8 + 1023u) / 1024u) * (uint32_t)M) break;   // uniform
    const uint32_t m = K8 <= 1024u ? tph + j * T : j % (uint32_t)M;
    const uint32_t k8 = K8 <= 1024u ? k80 : k80 + 1024u * (j / (uint32_t)M);
    float v[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = live ? lo_f32<DT>(sx[i][q]) : 0.0f;
      v[2 * q + 1] = live ? hi_f32<DT>(sx[i][q]) : 0.0f;
    }
    if constexpr (HAS_R) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ir = K8 <= 1024u ? 0 : i;
        v[q] *= live ? sr0[ir][q] : 0.0f;
        v[4 + q] *= live ? sr1[ir][q] : 0.0f;
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) amax = fmaxf(amax, fabsf(v[q]));
    amax = fmaxf(amax, quad_xor1(amax));
    amax = fmaxf(amax, quad_xor2(amax));
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x141, 0xF, 0xF, false)));
    amax = fmaxf(amax, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(amax), 0x140, 0xF, 0xF, false)));
    const int p = pow2_exp_for(amax);
    if (live) {
      uint32_t h[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) h[q] = f32_to_f16_bits(ldexpf(v[q], p));
      u32x4 o;
      o[0] = h[0] | (h[4] << 16);
      o[1] = h[2] | (h[6] << 16);
      o[2] = h[1] | (h[5] << 16);
      o[3] = h[3] | (h[7] << 16);
      *reinterpret_cast<u32x4*>(xs + (int64_t)m * KP + (int64_t)k8 * 8) = o;
      if ((k8 & 15u) == 0u) pinv[m * G + (k8 >> 4)] = ldexpf(1.0f, -p);
    }
  }
  for (int64_t c = tid; c < (int64_t)K8; c += 1024)
    *reinterpret_cast<u32x4*>(xs + (int64_t)M * KP + c * 8) = u32x4{0u, 0u, 0u, 0u};
  for (int c = tid; c < G; c += 1024) pinv[M * G + c] = 0.0f;
  __syncthreads();

  // ---- items
  const int tok = rl < M ? rl : M;               // the lane's token row (row M = 0)
  const uint32_t xbase = (uint32_t)(tok * KP * 2);
  for (; it < nitems; it += kScWaves) {
    if (it != wv) {                               // later items of this wave (only when ksl == 1)
      set_item(it);
      sp0 = load_piece(b);
#pragma unroll
      for (int d = 0; d < P; ++d) load_group(d, g0 + d);
    }
    // row power of two from all of the row's steps
    auto piece_max = [&](const u32x4& pv, int pc, float m) {
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (pc * 8 + q < GW) m = fmaxf(m, f16_to_f32((pv[q >> 1] >> (16 * (q & 1))) & 0xFFFFu));
      return m;
    };
    float mx = piece_max(sp0, b, 0.0f);
    for (int pc = b + 4; pc < npc; pc += 4) mx = piece_max(load_piece(pc), pc, mx);
    {
      const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
      const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    }
    int e = 0;
    if (mx > 0.0f) {
      int ex;
      frexpf(mx, &ex);
      e = -9 - ex;                               // max step 2^e in [2^-10, 2^-9)
    }

    // ring of P groups: slot d is refilled with group g + P right after group
    // g is consumed (reads past the slice's end are out of range and return 0)
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int gb = g0; gb < g1; gb += P) {
#pragma unroll
      for (int d = 0; d < P; ++d) {
        const int g = gb + d;
        if (g < g1) {                             // wave-uniform
          u32x4 xb[4];
          const uint16_t* xp = reinterpret_cast<const uint16_t*>(
              reinterpret_cast<const char*>(xs) + xbase + (uint32_t)(128 * g + 32 * b) * 2);
#pragma unroll
          for (int i = 0; i < 4; ++i) xb[i] = *reinterpret_cast<const u32x4*>(xp + 8 * i);
          const float gscale = pinv[tok * G + g];
          const float D = ldexpf(f16_to_f32(sr[d]), e);
          const uint32_t h24 = f32_to_f16_bits(D * 16777216.0f);
          const uint32_t h20 = f32_to_f16_bits(D * 1048576.0f);
          const uint32_t hz = f32_to_f16_bits(-(D * (float)zr[d]));
          const f16x2 c24 = as_f16x2(h24 | (h24 << 16));
          const f16x2 c20 = as_f16x2(h20 | (h20 << 16));
          const f16x2 nzd = as_f16x2(hz | (hz << 16));
          f32x4 part = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int i = 0; i < 4; ++i) part = mfma16h(dequant_word_f16(wa[d][i], c24, c20, nzd), xb[i], part);
#pragma unroll
          for (int vv = 0; vv < 4; ++vv) acc[vv] = __builtin_fmaf(part[vv], gscale, acc[vv]);
        }
        load_group(d, g + P);
      }
    }

    // 16 x 16 layout: token = lane % 16, row = 4 (lane / 16) + v
    if (ksl == 1) {
#pragma unroll
      for (int vv = 0; vv < 4; ++vv) {
        const int row = 4 * b + vv;
        const int erw = __shfl(e, row);
        if (tile * 16 + row < nrows && rl < M)
          store_y<YDT>(y, (int64_t)rl * ldy + r0 + tile * 16 + row, ldexpf(acc[vv], -erw));
      }
    } else {
#pragma unroll
      for (int vv = 0; vv < 4; ++vv) red[it * 256 + (4 * b + vv) * 16 + rl] = acc[vv];
      if (it % ksl == 0 && b == 0) erow[tile * 16 + rl] = e;
    }
  }
  if (ksl > 1) {
    __syncthreads();
    for (int t = tid; t < ntile * 256; t += 1024) {
      const int tl = t >> 8, row = (t >> 4) & 15, tk = t & 15;
      float tot = 0.0f;
      for (int ks = 0; ks < ksl; ++ks) tot += red[(tl * ksl + ks) * 256 + row * 16 + tk];
      if (tl * 16 + row < nrows && tk < M)
        store_y<YDT>(y, (int64_t)tk * ldy + r0 + tl * 16 + row, ldexpf(tot, -erow[tl * 16 + row]));
    }
  }
}

// Pieces of 8 activations each thread stages (0 if the shape does not fit).
inline int skinny_cu_pieces(int64_t M, int64_t K) {
  const int64_t K8 = K >> 3;
  const int64_t per = K8 <= 1024 ? (M + (1024 / K8) - 1) / (1024 / K8) : ((K8 + 1023) / 1024) * M;
  return per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : per <= kScMaxPieces ? 8 : 0;
}

// Blocks of the per-CU skinny product for (M, N, K); 0 if it does not apply
// (K must be whole 128-channel units).
inline int skinny_cu_blocks(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || M > 16 || K % 128 != 0 || skinny_cu_pieces(M, K) == 0) return 0;
  const int64_t cus = awq::device_cus();
  const int64_t nblk = N < cus ? N : cus;
  const int64_t rows_max = (N + nblk - 1) / nblk;
  if (skinny_cu_lds(M, K, rows_max) > 160 * 1024 || rows_max * (K >> 1) >= (int64_t(1) << 31)) return 0;
  return (int)nblk;
}

template <int DT, int YDT, bool HAS_R, int P = 2>
hipError_t skinny_cu_dispatch(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint32_t* qw,
                              const uint16_t* scales, const uint8_t* zeros, int64_t N, int glog,
                              const float* r, void* y, int64_t ldy, int nblk, hipStream_t st) {
  if (nblk > N) nblk = (int)N;
  const int64_t rows_max = (N + nblk - 1) / nblk;
  size_t lds = skinny_cu_lds(M, K, rows_max);
  const int np = skinny_cu_pieces(M, K);
  if (M < 1 || M > 16 || np == 0 || K % 128 != 0 || lds > 160 * 1024 ||
      rows_max * (K >> 1) >= (int64_t(1) << 31))
    return hipErrorInvalidValue;
  if (lds < 81 * 1024) lds = 81 * 1024;           // one block per compute unit
  const dim3 grid((unsigned)nblk), block(1024);
#define AWQ_SC(NP)                                                                                    \
  hipLaunchKernelGGL((k_gemm_skinny_cu<DT, YDT, HAS_R, NP, P>), grid, block, lds, st, x, (int)M, K, ldx, r, \
                     qw, scales, zeros, N, y, ldy, glog)
  if (np == 1) AWQ_SC(1);
  else if (np == 2) AWQ_SC(2);
  else if (np == 4) AWQ_SC(4);
  else AWQ_SC(8);
#undef AWQ_SC
  return hipGetLastError();
}

template <int DT, int YDT, bool HAS_R, int P = kSkP>
hipError_t skinny_dispatch(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint32_t* qw,
                           const uint16_t* scales, const uint8_t* zeros, int64_t N, int glog,
                           const float* r, void* y, int64_t ldy, void* ws, hipStream_t st) {
  const GemmWs w = gemm_ws(ws, M, N, K, 1 << glog);
  hipLaunchKernelGGL((k_rows_f16<DT, HAS_R, true>), dim3((unsigned)M), dim3(256), 0, st, x, K, ldx,
                     r, w.xq, w.pm);
  hipLaunchKernelGGL((k_gemm_skinny<YDT, P>), dim3((unsigned)((N + 15) / 16)), dim3(64 * kSkW), 0, st,
                     w.xq, (int)M, K, w.pm, qw, scales, zeros, N, y, ldy, glog);
  return hipGetLastError();
}

template <int DT, int YDT>
hipError_t w4a16_dispatch(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint32_t* qw,
                          const uint16_t* scales, const uint8_t* zeros, int64_t N, int glog,
                          const float* r, void* y, int64_t ldy, void* ws, hipStream_t st) {
  if (M == 1 && awq::gemv1_supported(K, N))
    return awq::launch_gemv1(x, DT, K, qw, scales, zeros, N, 1 << glog, r, y, YDT, st);
  if (awq::mid_supported(M, N, K))
    return awq::launch_mid(x, DT, M, K, ldx, qw, scales, zeros, N, 1 << glog, r, y, YDT, ldy, ws, st);
  if (awq::skinny_st_blocks(M, N, K, 1 << glog))
    return awq::launch_skinny_st(x, DT, M, K, ldx, qw, scales, zeros, N, 1 << glog, r, y, YDT, ldy, st);
  if (awq::skinny_st_chunks(M, N, K, 1 << glog))
    return awq::launch_skinny_st_chunked(x, DT, M, K, ldx, qw, scales, zeros, N, 1 << glog, r, y, YDT, ldy, st);
  if (const int nblk = skinny_cu_blocks(M, N, K)) {
    // deeper ring for long K slices (few rows per block)
    const int64_t rows = (N + nblk - 1) / nblk, tiles = (rows + 15) / 16;
    const bool deep = (K / 128) * tiles >= 16 * 16;
    if (r) return deep ? skinny_cu_dispatch<DT, YDT, true, 4>(x, M, K, ldx, qw, scales, zeros, N, glog, r, y, ldy, nblk, st)
                       : skinny_cu_dispatch<DT, YDT, true, 2>(x, M, K, ldx, qw, scales, zeros, N, glog, r, y, ldy, nblk, st);
    return deep ? skinny_cu_dispatch<DT, YDT, false, 4>(x, M, K, ldx, qw, scales, zeros, N, glog, r, y, ldy, nblk, st)
                : skinny_cu_dispatch<DT, YDT, false, 2>(x, M, K, ldx, qw, scales, zeros, N, glog, r, y, ldy, nblk, st);
  }
  if (M <= kSkMaxM && K % 128 == 0) {
    if (r) return skinny_dispatch<DT, YDT, true>(x, M, K, ldx, qw, scales, zeros, N, glog, r, y, ldy, ws, st);
    return skinny_dispatch<DT, YDT, false>(x, M, K, ldx, qw, scales, zeros, N, glog, r, y, ldy, ws, st);
  }
  if (r) return gemm_dispatch<DT, YDT, true>(x, M, K, ldx, qw, scales, zeros, N, glog, r, y, ldy, ws, st);
  return gemm_dispatch<DT, YDT, false>(x, M, K, ldx, qw, scales, zeros, N, glog, r, y, ldy, ws, st);
}

}  // namespace awqk

namespace awq {

size_t gemm_ws_bytes(int64_t M, int64_t N, int64_t K, int group) {
  if (M <= 0 || N <= 0 || K <= 0 || group <= 0 || (M == 1 && gemv1_supported(K, N))) return 0;
  if (mid_supported(M, N, K)) return mid_ws_bytes(M, N, K);
  if (skinny_st_chunks(M, N, K, group) || awqk::skinny_cu_blocks(M, N, K)) return 0;
  return awqk::gemm_ws(nullptr, M, N, K, group).bytes;
}

hipError_t launch_w4a16(const void* x, int xdt, int64_t M, int64_t K, int64_t ldx,
                        const uint32_t* qw, const uint16_t* scales, const uint8_t* zeros,
                        int64_t N, int group, const float* inv_s, void* y, int ydt, int64_t ldy,
                        void* ws, hipStream_t st) {
  using namespace awqk;
  const uint16_t* xp = (const uint16_t*)x;
  const int glog = group == 64 ? 6 : group == 128 ? 7 : group == 256 ? 8 : -1;
  if (glog < 0) return hipErrorInvalidValue;
#define AWQ_WD(XT, YT) \
  return w4a16_dispatch<XT, YT>(xp, M, K, ldx, qw, scales, zeros, N, glog, inv_s, y, ldy, ws, st)
  if (xdt == DT_F16) {
    if (ydt == DT_F16) AWQ_WD(DT_F16, DT_F16);
    if (ydt == DT_BF16) AWQ_WD(DT_F16, DT_BF16);
    AWQ_WD(DT_F16, DT_F32);
  }
  if (ydt == DT_F16) AWQ_WD(DT_BF16, DT_F16);
  if (ydt == DT_BF16) AWQ_WD(DT_BF16, DT_BF16);
  AWQ_WD(DT_BF16, DT_F32);
#undef AWQ_WD
}

}  // namespace awq
