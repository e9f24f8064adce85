// W4A16 product for 2..16 tokens ("AWQ > Benefits and Practical
// Considerations": unpack the 4-bit integers, apply the group's step and zero
// point and the optional per-channel inverse scale, fused with the multiply).
// At decode batch sizes the product is bound by the packed weight stream
// ("AWQ Math", "Weight-only quantization and where it breaks"), so this kernel
// keeps every compute unit's weight loads in flight and spends few vector
// instructions per packed word:
//
//  * One block of 16 waves per compute unit; block b owns the weight rows
//    [b N / B, (b + 1) N / B) in 16-row tiles.  With t tiles each tile's
//    128-channel units are split into S = 16 / t slices; wave w takes the
//    items (tile, slice) w, w + 16, ... and keeps up to kStQ units of its
//    packed words in flight.
//  * v_mfma_f32_16x16x32_f16 with the tokens as A (16 rows; rows past M
//    repeat token M - 1 and their outputs are dropped) and 16 weight rows as
//    B.  A result lane holds the outputs of the weight row whose packed words
//    it loaded, so the group's step multiplies the product once, in fp32.
//  * The codes reach the matrix cores as fp16 subnormals: word & 0x000F000F is
//    q 2^-24 for nibbles 0 and 4, word & 0x00F000F0 is q 2^-20 for nibbles 1
//    and 5, and the same masks on word >> 8 give nibbles 2, 6 and 3, 7 (one
//    shift and four ANDs per word; the matrix cores keep fp16 subnormal
//    inputs).  The activations staged for odd nibbles are divided by 16, so
//    every product is X q 2^-24.
//  * The zero point enters as each unit's starting accumulator,
//    -z 2^-24 sum_k X_k, from per-(token, unit) sums staged with the
//    activations, and the step is staged as D 2^24:
//    y = sum_units (D 2^24) 2^-p (sum_k X_k q_k 2^-24 - z 2^-24 sum_k X_k).
//  * The block stages in LDS: X = fp16(x r 2^p) with one power of two per
//    (token, 128-channel unit) (max |X| in [2^13, 2^14)), in the order the
//    unpack yields (k0,k4,k2,k6,k1,k5,k3,k7 per word); the sums and 2^-p; and
//    the block's steps and zero points as fp32 pairs.  Every thread stages
//    pieces of one 8-channel column and holds one 1/s vector, so a pass covers
//    at most 8192 channels.  When the tokens' activations do not fit LDS or
//    the block's threads at once, they are staged in passes of whole units
//    (blocks of at most 16 tiles, one item per wave): in every pass each wave
//    runs its slice of the pass's units, issues its first units of the next
//    pass, and the block restages once every wave has left X.
//  * When LDS has room beside the staged activations (one pass, groups of 128
//    or 256), the packed words come through a per-wave LDS ring: each copy
//    moves 8 rows x 128 bytes (whole lines, two units) by LDS DMA, and a lane
//    reads its row's 16 bytes of a unit back in the matrix-core layout.  A
//    load of 16 rows x 64 bytes straight into registers (the other path)
//    streams the same bytes markedly slower.
//  * A wave's instructions issue in order, and the memory pipeline holds a
//    wave at a load's issue while the weight stream flows, so a wave that
//    issues its weight loads first cannot stage until the stream has mostly
//    passed.  For blocks of two or more tiles, waves 8..15 therefore issue
//    their weight loads at once and stage nothing, while waves 0..7 stage
//    everything and then issue theirs.
#include "awq_device.h"
#include "awq_internal.h"
#include "k_rows_f16.h"

#include <type_traits>

namespace awqk {

constexpr int kStWaves = 16;
constexpr int kStQ = 8;              // 128-channel units of packed words in flight per wave
constexpr int kStMetaPer = 8;        // staged (step, zero point) pairs per thread
constexpr int kStMaxPieces = 8;      // staged 8-channel activation pieces per thread
constexpr size_t kStLdsMax = 160 * 1024;
constexpr int kStPQ = 2;             // unit pairs in flight per wave when the words come through LDS
constexpr size_t kStRing = (size_t)kStWaves * kStPQ * 2048;   // those pairs' LDS ring

template <int YDT>
__device__ __forceinline__ void store_yst(void* y, int64_t idx, float v) {
  if constexpr (YDT == DT_F32) reinterpret_cast<float*>(y)[idx] = v;
  else reinterpret_cast<uint16_t*>(y)[idx] = (uint16_t)from_f32<YDT>(v);
}

// One packed word -> its 8 codes as fp16 subnormals, in the order
// (0,4 | 2,6 | 1,5 | 3,7): q 2^-24 for the even nibbles, q 2^-20 for the odd.
__device__ __forceinline__ u32x4 st_unpack(uint32_t w) {
  const uint32_t w8 = w >> 8;
  return u32x4{w & 0x000F000Fu, w8 & 0x000F000Fu, w & 0x00F000F0u, w8 & 0x00F000F0u};
}

// This wave's LDS operations done, then every wave of the block at this point.
__device__ __forceinline__ void st_sync() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Byte offsets of the LDS regions.
struct StLayout {
  size_t sums, pinv, meta, total;
  int meta_pitch;   // (step, zero) pairs per staged row
  size_t ring, total_lw;   // the words' LDS ring after the rest, and the total with it
};

inline StLayout st_layout(int64_t M, int64_t K, int64_t rows_max, int glog, int64_t kpass) {
  StLayout L;
  const size_t xs = (size_t)M * (size_t)(kpass + 8) * 2;       // X [M][kpass + 8]
  const size_t red = (size_t)kStWaves * 256 * 4;              // slices' 16 x 16 tiles (reuses X)
  const int64_t gw = K >> glog;
  L.meta_pitch = (int)gw + 2;                                 // rows 16 B apart across banks
  L.sums = awq::align_up(xs > red ? xs : red, 16);
  L.pinv = L.sums + (size_t)(glog == 6 ? K / 64 : K / 128) * 16 * 4;
  L.meta = L.pinv + (size_t)(K / 128) * 16 * 4;
  L.total = L.meta + (size_t)rows_max * L.meta_pitch * 8;
  L.ring = awq::align_up(L.total, 16);
  L.total_lw = L.ring + kStRing;
  return L;
}

// Activation pieces per staging thread for (M, K) with nthr staging threads:
// nthr / (K/8) token phases of K/8 threads; 0 if K/8 > nthr or over 8 pieces.
inline int st_pieces(int64_t M, int64_t K, int64_t nthr = 1024) {
  const int64_t K8 = K >> 3;
  if (K8 < 1 || K8 > nthr) return 0;
  const int64_t per = (M + (nthr / K8) - 1) / (nthr / K8);
  return per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : per <= kStMaxPieces ? 8 : 0;
}

// Whether waves 8..15 only load weights while waves 0..7 stage: blocks of more
// than one 16-row tile (with one tile the 16 waves' items are short and the
// staging on half the waves costs more than it hides), groups of 128 or 256,
// the pieces fit 512 threads, at most 4096 (step, zero point) pairs.
inline bool st_split(int64_t M, int64_t K, int64_t rows_max, int glog) {
  return rows_max > 16 && glog != 6 && st_pieces(M, K, 512) != 0 && rows_max * (K >> glog) <= 512 * kStMetaPer;
}

// Channels staged per pass: K when every token's activations fit at once;
// else the fewest passes of equal whole 128-channel units whose pieces fit the
// block's threads and whose LDS fits, for blocks of at most 16 tiles (one item
// per wave, so the waves meet at every pass); 0 if none.  Blocks of one
// nearly full tile (13..16 rows) with 8 or more tokens are left to the other
// kernels: there each block stages every token's activations for at most 16
// rows of weights, and the staging passes (loads, conversion, barriers) cost
// about as much as the row-tile kernel's shared pre-converted activations,
// which then fill the chip.
inline int64_t st_kpass(int64_t M, int64_t K, int64_t rows_max, int glog) {
  if (st_pieces(M, K) != 0 && st_layout(M, K, rows_max, glog, K).total <= kStLdsMax) return K;
  if (rows_max > 16 * 16 || (rows_max > 12 && rows_max <= 16 && M >= 8)) return 0;
  const int64_t G = K >> 7;
  const int maxp = glog == 6 ? 4 : kStMaxPieces;   // groups of 64: at most 4 pieces (registers)
  for (int64_t np = 2; np <= G; ++np) {
    const int64_t kp = (G + np - 1) / np * 128;
    const int pc = st_pieces(M, kp);
    if (pc != 0 && pc <= maxp && st_layout(M, K, rows_max, glog, kp).total <= kStLdsMax) return kp;
  }
  return 0;
}

// 16 bytes per lane into LDS (LDS DMA, non-temporal; an offset past the
// buffer's range writes 0).  Issued from asm, so the compiler adds no wait of
// its own before the LDS reads: the caller waits on the vector memory counter.
__device__ __forceinline__ void st_dma16(const i32x4& rs, uint32_t lds, uint32_t voff) {
  uint32_t keep;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, 0 offen nt lds\n\ts_mov_b32 m0, %0"
               : "=&s"(keep) : "s"(lds), "v"(voff), "s"(rs) : "memory");
}

template <int DT, int YDT, bool HAS_R, int NP, bool G64, bool SPLIT, bool MULTI, bool LW>
__global__ __launch_bounds__(1024) void k_gemm_skinny_st(
    const uint16_t* __restrict__ x, int M, int64_t K, int64_t ldx, const float* __restrict__ r,
    const uint32_t* __restrict__ qw, const uint16_t* __restrict__ scales,
    const uint8_t* __restrict__ zeros, int64_t N, void* __restrict__ y, int64_t ldy, int glog,
    uint32_t o_sums, uint32_t o_pinv, uint32_t o_meta, int mp, int kpass, uint32_t o_ring) {
  static_assert(!LW || (!MULTI && !G64), "words through LDS: one pass, groups >= 128");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_st[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rl = lane & 15;
  const int b = lane >> 4;
  // MULTI: the activations are staged in passes of kpass channels (the
  // block's items then hold one item per wave); otherwise in one pass
  const int kp = MULTI ? kpass : (int)K;
  const uint32_t K8 = (uint32_t)(kp >> 3);        // 8-channel pieces per token in a full pass
  const int UPp = kp >> 7;                        // 128-channel units per pass
  const int npass = MULTI ? (int)((K + kp - 1) / kp) : 1;
  const int G = (int)(K >> 7);
  const int GW = (int)(K >> glog);
  const int64_t KP = kp + 8;                      // LDS pitch of a staged token row
  const int64_t r0 = (int64_t)blockIdx.x * N / gridDim.x;
  const int nrows = (int)((int64_t)(blockIdx.x + 1) * N / gridDim.x - r0);
  const int ntile = (nrows + 15) / 16;
  int ksl = kStWaves / (ntile > 0 ? ntile : 1);
  ksl = ksl < 1 ? 1 : (ksl > G ? G : ksl);
  const int nitems = ntile * ksl;

  uint16_t* xs = reinterpret_cast<uint16_t*>(lds_st);
  float* red = reinterpret_cast<float*>(lds_st);                        // after the items
  float* sums = reinterpret_cast<float*>(lds_st + o_sums);              // [piece][16 tokens]
  float* pinv = reinterpret_cast<float*>(lds_st + o_pinv);              // [unit][16 tokens]
  float2* meta = reinterpret_cast<float2*>(lds_st + o_meta);            // [row][mp]

  const int nmeta = nrows * GW;
  const uint32_t T = (SPLIT ? 512u : 1024u) / K8;
  const uint32_t tph = (uint32_t)tid / K8;
  const uint32_t k8 = tph < T ? (uint32_t)tid - tph * K8 : 0u;
  const uint32_t ntok = tph < T && (uint32_t)M > tph ? ((uint32_t)M - tph + T - 1) / T : 0u;
  // ---- the first item's packed words
  const uint32_t KW = (uint32_t)(K >> 3);
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(qw + r0 * KW), (short)0, nrows * (int)KW * 4, kBufferWord3);
  int it = wv;
  int tile = 0, ksi = 0, g0 = 0, g1 = 0;
  auto set_item = [&](int item) {
    tile = item / ksl;
    ksi = item - tile * ksl;
    if constexpr (LW) {
      // slices of whole unit pairs (the last pair of an odd G holds one unit)
      const int G2 = (G + 1) >> 1;
      g0 = 2 * (int)((int64_t)ksi * G2 / ksl);
      g1 = 2 * (int)((int64_t)(ksi + 1) * G2 / ksl);
      g1 = g1 < G ? g1 : G;
    } else {
      g0 = (int)((int64_t)ksi * G / ksl);
      g1 = (int)((int64_t)(ksi + 1) * G / ksl);
    }
  };
  // with passes, the item's units in pass ps: slice ksi of the pass's units
  auto pass_range = [&](int ps, int& a, int& e) {
    const int p0 = ps * UPp;
    const int up = G - p0 < UPp ? G - p0 : UPp;
    a = p0 + ksi * up / ksl;
    e = p0 + (ksi + 1) * up / ksl;
  };
  const bool have = it < nitems;                 // wave-uniform
  u32x4 wq[kStQ];
  // unit g of the item's tile: one 128-bit chunk b of the lane's row (words
  // 4b .. 4b + 3), or with groups of 64 the words 2b, 2b + 1 of each half
  // Rows past the block's last lie past the descriptor's range and read as
  // zeros by themselves, so the only choice left is the wave-uniform one (a
  // unit outside the item), which keeps the loads free of branches.
  const uint32_t lane_off = (uint32_t)rl * KW * 4 + (uint32_t)b * (G64 ? 8 : 16);
  auto load_unit = [&](int slot, int g, int gend) {
    // the unit's wave-uniform offset, or 2^31 (past any range) at or past
    // gend: a scalar choice, the load itself unconditional
    const bool ok = have && g < gend;
    const uint32_t uoff = __builtin_amdgcn_readfirstlane(ok ? (uint32_t)(tile * 16) * KW * 4 + (uint32_t)g * 64 : kBufferOob);
    const uint32_t off = lane_off + uoff;
    if constexpr (!G64) {
      wq[slot] = __builtin_amdgcn_raw_buffer_load_b128(wrs, off, 0, kBufferNt);
    } else {
      const auto lo = __builtin_amdgcn_raw_buffer_load_b64(wrs, off, 0, kBufferNt);
      const auto hi = __builtin_amdgcn_raw_buffer_load_b64(wrs, off + 32, 0, kBufferNt);
      wq[slot] = u32x4{lo[0], lo[1], hi[0], hi[1]};
    }
  };
  // With LW the words come through a per-wave LDS ring of kStPQ unit pairs:
  // a pair is two 1 KB copies (rows 0..7 and 8..15 of the tile, 128 bytes =
  // both units of each row, so every copy reads whole 128-byte lines), with
  // chunk c of row r' of half h at 16-byte slot 8 r' + (c ^ (r'/2 + 4h)); a
  // lane then reads its row's 16 bytes of a unit with one conflict-free
  // 128-bit LDS read.  (Loads of 16 rows x 64 bytes each, the register path,
  // read the same bytes markedly slower.)
  const uint32_t rowb = KW * 4;
  const i32x4 wrs4 = rsrc4(qw + r0 * KW, (uint32_t)nrows * rowb);
  const uint32_t ring_w = __builtin_amdgcn_readfirstlane(lds_addr(lds_st) + o_ring + (uint32_t)wv * kStPQ * 2048);
  const int dq = lane >> 3, ds = lane & 7;
  const uint32_t dv0 = (uint32_t)dq * rowb + (uint32_t)((ds ^ (dq >> 1)) * 16);
  const uint32_t dv1 = (uint32_t)(dq + 8) * rowb + (uint32_t)((ds ^ ((dq >> 1) | 4)) * 16);
  auto issue_pair = [&](int slot, int q, int qend) {
    const bool ok = have && q < qend;
    const uint32_t uo = __builtin_amdgcn_readfirstlane(ok ? (uint32_t)(tile * 16) * rowb + (uint32_t)q * 128 : kBufferOob);
    st_dma16(wrs4, ring_w + (uint32_t)slot * 2048, dv0 + uo);
    st_dma16(wrs4, ring_w + (uint32_t)slot * 2048 + 1024, dv1 + uo);
  };
  auto issue_weights = [&]() {
    set_item(have ? it : 0);
    if constexpr (LW) {
#pragma unroll
      for (int d = 0; d < kStPQ; ++d) issue_pair(d, (g0 >> 1) + d, (g1 + 1) >> 1);
    } else {
      int a = g0, e = g1;
      if constexpr (MULTI) pass_range(0, a, e);
#pragma unroll
      for (int d = 0; d < kStQ; ++d) load_unit(d, a + d, e);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // ---- staging: its loads, then mid() (the weights' issue when every wave
  // stages), then the conversion.  Thread t takes piece k8 = t mod K/8 of the
  // tokens t / (K/8), t / (K/8) + T, ... (T = 1024 / (K/8) token phases, or
  // 512 / (K/8) when only waves 0..7 stage).  Threads past the last phase load
  // piece 0 of token 0 and drop it (no branch around the loads).  The steps
  // and zero points come 8 per thread: one 128-bit and one 64-bit load.
  // pass ps covers channels [ps kp, ps kp + kp) (the last pass may be
  // shorter); with_meta: also the steps and zero points (the first pass)
  auto stage = [&](auto mid, int ps, auto with_meta) {
    const int64_t c0 = (int64_t)ps * kp;
    const uint32_t k8n = (uint32_t)((K - c0 < kp ? K - c0 : kp) >> 3);   // pieces in this pass
    const bool kin = k8 < k8n;
    uint32_t k8c = kin ? k8 : 0u, tphc = tph;
    uint64_t xa = (uint64_t)x, ra = (uint64_t)r;
    if constexpr (MULTI) {
      // with passes, opaque copies: the pieces' addresses are formed here, not
      // kept live across the passes, and the loads stay ahead of the weights'
      // (a load from a read-only argument may otherwise sink to its use)
      asm volatile("" : "+v"(k8c), "+v"(tphc));
      asm volatile("" : "+s"(xa), "+s"(ra));
    }
    using gu16 = const __attribute__((address_space(1))) uint16_t;
    using gu32x4 = const __attribute__((address_space(1))) u32x4;
    using gf32 = const __attribute__((address_space(1))) float;
    using gf32x4 = const __attribute__((address_space(1))) f32x4;
    u32x4 sx[NP];
    f32x4 sr0, sr1;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const uint32_t m = tphc + (uint32_t)i * T;
      const int64_t off = (int64_t)((uint32_t)i < ntok ? m : 0u) * ldx + c0 + (int64_t)k8c * 8;
      if constexpr (MULTI) sx[i] = *(gu32x4*)((gu16*)xa + off);
      else sx[i] = ldg128(x + off);
    }
    if constexpr (HAS_R) {
      const int64_t off = c0 + (int64_t)k8c * 8;
      if constexpr (MULTI) {
        sr0 = *(gf32x4*)((gf32*)ra + off);
        sr1 = *(gf32x4*)((gf32*)ra + off + 4);
      } else {
        sr0 = *reinterpret_cast<const f32x4*>(r + off);
        sr1 = *reinterpret_cast<const f32x4*>(r + off + 4);
      }
    }
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(scales + r0 * GW), (short)0, nmeta * 2, kBufferWord3);
    const __amdgpu_buffer_rsrc_t zrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(zeros + r0 * GW), (short)0, nmeta, kBufferWord3);
    // thread t takes entries [e0, e0 + 8) with e0 = min(8 t, nmeta - 8), so
    // every load lies wholly inside the block's range (nmeta >= 8); the last
    // window overlaps its neighbour's and writes the same values
    const bool mlive = decltype(with_meta)::value && tid * kStMetaPer < nmeta;
    const int e0 = mlive ? (tid * kStMetaPer < nmeta - kStMetaPer ? tid * kStMetaPer : nmeta - kStMetaPer) : 0;
    const u32x4 mst = __builtin_amdgcn_raw_buffer_load_b128(srs, mlive ? (uint32_t)e0 * 2 : kBufferOob, 0, 0);
    const auto mze = __builtin_amdgcn_raw_buffer_load_b64(zrs, mlive ? (uint32_t)e0 : kBufferOob, 0, 0);

    mid();


    // ---- the block's steps (times 2^24, exact: it undoes the codes' 2^-24)
    // and zero points
#pragma unroll
    for (int j = 0; j < kStMetaPer; ++j) {
      const int e = e0 + j;
      if (mlive) {
        const int row = e / GW;
        const uint32_t sb = (mst[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
        const uint32_t zb = (mze[j >> 2] >> (8 * (j & 3))) & 0xFFu;
        meta[row * mp + (e - row * GW)] = make_float2(ldexpf(f16_to_f32(sb), 24), (float)zb);
      }
    }

    // ---- X = fp16(x r 2^p), p per (token, 128-channel unit) from the unit's
    // max |x r| (max |X| in [2^13, 2^14)); the odd nibbles' channels get
    // 2^(p - 4).  The 16 pieces of a unit sit in 16 consecutive lanes.  Beside
    // X: 2^-24 sum X per piece of the zero point's granularity, and 2^-p.
    const int npl = (int)(((uint32_t)M + T - 1) / T);   // pieces any thread stages
    const f16x2 one2 = as_f16x2(0x3C003C00u), sixteen2 = as_f16x2(0x4C004C00u);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (i >= npl) break;                         // uniform
      const uint32_t m = tph + (uint32_t)i * T;
      const bool live = (uint32_t)i < ntok && kin;
      float v[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] = lo_f32<DT>(sx[i][q]);
        v[2 * q + 1] = hi_f32<DT>(sx[i][q]);
      }
      if constexpr (HAS_R) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q] *= sr0[q];
          v[4 + q] *= sr1[q];
        }
      }
      float am = 0.0f;
#pragma unroll
      for (int q = 0; q < 8; ++q) am = fmaxf(am, fabsf(v[q]));
      am = fmaxf(am, quad_xor1(am));
      am = fmaxf(am, quad_xor2(am));
      am = fmaxf(am, dpp_f<0x141>(am));            // row_half_mirror
      am = fmaxf(am, dpp_f<0x140>(am));            // row_mirror: the unit's max
      const int p = pow2_exp_for(am);
      uint32_t h[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) h[c] = f32_to_f16_bits(ldexpf(v[c], (c & 1) ? p - 4 : p));
      u32x4 o;
      o[0] = h[0] | (h[4] << 16);
      o[1] = h[2] | (h[6] << 16);
      o[2] = h[1] | (h[5] << 16);
      o[3] = h[3] | (h[7] << 16);
      // sum X of the piece, exactly as the products see the operands
      float sx8 = __builtin_amdgcn_fdot2(as_f16x2(o[0]), one2, 0.0f, false);
      sx8 = __builtin_amdgcn_fdot2(as_f16x2(o[1]), one2, sx8, false);
      sx8 = __builtin_amdgcn_fdot2(as_f16x2(o[2]), sixteen2, sx8, false);
      sx8 = __builtin_amdgcn_fdot2(as_f16x2(o[3]), sixteen2, sx8, false);
      float s = live ? ldexpf(sx8, -24) : 0.0f;
      s += quad_xor1(s);
      s += quad_xor2(s);
      s += dpp_f<0x141>(s);                        // 8 channels x 8 lanes: a 64-channel half unit
      if constexpr (!G64) s += dpp_f<0x140>(s);     // 16 lanes: the 128-channel unit
      if (live) {
        *reinterpret_cast<u32x4*>(xs + (int64_t)m * KP + (int64_t)k8 * 8) = o;
        if ((lane & (G64 ? 7 : 15)) == 0) sums[((uint32_t)(c0 >> (G64 ? 6 : 7)) + (k8 >> (G64 ? 3 : 4))) * 16 + m] = s;
        if ((lane & 15) == 0) pinv[((uint32_t)(c0 >> 7) + (k8 >> 4)) * 16 + m] = ldexpf(1.0f, -p);
      }
    }
  };
  // With SPLIT, waves 8..15 issue their weight loads at once and stage
  // nothing, while waves 0..7 stage every activation piece and then issue
  // theirs: a wave held at a load's issue by the memory pipeline does not
  // delay the conversion, and half of the weight stream overlaps it.
  if constexpr (SPLIT) {
    if (wv < 8) {
      stage([] {}, 0, std::true_type{});
      issue_weights();
    } else {
      issue_weights();
    }
  } else if constexpr (LW) {
    // the copies after the conversion: the compiler's waits for the staging
    // loads would otherwise wait for the copies issued after them too
    stage([] {}, 0, std::true_type{});
    issue_weights();
  } else {
    stage(issue_weights, 0, std::true_type{});
  }
  st_sync();

  // ---- items
  const int tok = rl < M ? rl : M - 1;           // rows past M repeat a token; dropped
  const uint8_t* xrow = reinterpret_cast<const uint8_t*>(xs) + (size_t)tok * (size_t)KP * 2;
  const int gsh = glog - 7;                       // unit -> group (groups of 128, 256)
  // units [ga, ge) of the item, the first kStQ already in flight in slots
  // 0 .. kStQ - 1; refills run past ge (out of range, no traffic).  ubase: the
  // first unit of the staged pass.  Per unit: part = -z 2^-24 sum X +
  // sum X q 2^-24 on the matrix cores, then acc += (D 2^24) 2^-p part.
  auto run_item = [&](f32x4 acc, int ga, int ge, int ubase) {
    const int rowc = tile * 16 + rl < nrows ? tile * 16 + rl : nrows - 1;
    const float2* mrow = meta + rowc * mp;
    for (int gb = ga; gb < ge; gb += kStQ) {
#pragma unroll
      for (int d = 0; d < kStQ; ++d) {
        const int g = gb + d;
        if (g < ge) {                             // wave-uniform
          u32x4 xa[4];
          const f32x4 pv = *reinterpret_cast<const f32x4*>(pinv + g * 16 + 4 * b);
          if constexpr (!G64) {
            const uint8_t* p = xrow + (size_t)(128 * (g - ubase) + 32 * b) * 2;
#pragma unroll
            for (int i = 0; i < 4; ++i) xa[i] = *reinterpret_cast<const u32x4*>(p + 16 * i);
            const f32x4 sv = *reinterpret_cast<const f32x4*>(sums + g * 16 + 4 * b);
            const float2 md = mrow[g >> gsh];
            f32x4 part;
#pragma unroll
            for (int v = 0; v < 4; ++v) part[v] = -md.y * sv[v];
#pragma unroll
            for (int i = 0; i < 4; ++i) part = mfma16h(xa[i], st_unpack(wq[d][i]), part);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(md.x * pv[v], part[v], acc[v]);
          } else {
            const uint8_t* p = xrow + (size_t)(128 * (g - ubase) + 16 * b) * 2;
            xa[0] = *reinterpret_cast<const u32x4*>(p);
            xa[1] = *reinterpret_cast<const u32x4*>(p + 16);
            xa[2] = *reinterpret_cast<const u32x4*>(p + 128);
            xa[3] = *reinterpret_cast<const u32x4*>(p + 144);
            const f32x4 sv0 = *reinterpret_cast<const f32x4*>(sums + (2 * g) * 16 + 4 * b);
            const f32x4 sv1 = *reinterpret_cast<const f32x4*>(sums + (2 * g + 1) * 16 + 4 * b);
            const f32x4 md = *reinterpret_cast<const f32x4*>(mrow + 2 * g);   // (D0, z0, D1, z1)
            f32x4 p0, p1;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              p0[v] = -md[1] * sv0[v];
              p1[v] = -md[3] * sv1[v];
            }
            p0 = mfma16h(xa[0], st_unpack(wq[d][0]), p0);
            p0 = mfma16h(xa[1], st_unpack(wq[d][1]), p0);
            p1 = mfma16h(xa[2], st_unpack(wq[d][2]), p1);
            p1 = mfma16h(xa[3], st_unpack(wq[d][3]), p1);
#pragma unroll
            for (int v = 0; v < 4; ++v)
              acc[v] = __builtin_fmaf(md[2] * pv[v], p1[v], __builtin_fmaf(md[0] * pv[v], p0[v], acc[v]));
          }
        }
        load_unit(d, g + kStQ, ge);
      }
    }
    return acc;
  };
  // The item through the LDS ring: per pair, wait for its copies (the later
  // pairs' may stay in flight), run its units, wait for the LDS reads, then
  // copy pair q + kStPQ into the slot.
  const uint8_t* wrow = lds_st + o_ring + (uint32_t)wv * kStPQ * 2048 + (rl >> 3) * 1024 + (rl & 7) * 128;
  const int wsw = ((rl & 7) >> 1) | ((rl >> 3) << 2);
  auto run_item_lw = [&](f32x4 acc) {
    const int rowc = tile * 16 + rl < nrows ? tile * 16 + rl : nrows - 1;
    const float2* mrow = meta + rowc * mp;
    const int qa = g0 >> 1, qe = (g1 + 1) >> 1;
    for (int qb = qa; qb < qe; qb += kStPQ) {
#pragma unroll
      for (int d = 0; d < kStPQ; ++d) {
        const int q = qb + d;
        if (q < qe) {                             // wave-uniform
          asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * (kStPQ - 1)) : "memory");
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int g = 2 * q + u;
            if (g < g1) {                         // wave-uniform
              const u32x4 w = *reinterpret_cast<const u32x4*>(wrow + d * 2048 + (((4 * u + b) ^ wsw) * 16));
              u32x4 xa[4];
              const f32x4 pv = *reinterpret_cast<const f32x4*>(pinv + g * 16 + 4 * b);
              const uint8_t* p = xrow + (size_t)(128 * g + 32 * b) * 2;
#pragma unroll
              for (int i = 0; i < 4; ++i) xa[i] = *reinterpret_cast<const u32x4*>(p + 16 * i);
              const f32x4 sv = *reinterpret_cast<const f32x4*>(sums + g * 16 + 4 * b);
              const float2 md = mrow[g >> gsh];
              f32x4 part;
#pragma unroll
              for (int v = 0; v < 4; ++v) part[v] = -md.y * sv[v];
#pragma unroll
              for (int i = 0; i < 4; ++i) part = mfma16h(xa[i], st_unpack(w[i]), part);
#pragma unroll
              for (int v = 0; v < 4; ++v) acc[v] = __builtin_fmaf(md.x * pv[v], part[v], acc[v]);
            }
          }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        issue_pair(d, q + kStPQ, qe);
      }
    }
    return acc;
  };
  // 16 x 16 result layout: weight row = lane % 16, tokens 4 (lane / 16) + v
  auto store_direct = [&](const f32x4& a) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = 4 * b + v;
      if (t < M && tile * 16 + rl < nrows) store_yst<YDT>(y, (int64_t)t * ldy + r0 + tile * 16 + rl, a[v]);
    }
  };
  // The first item runs on the words loaded before the staging; later items
  // (only when ksl == 1) load their own.  Two copies of the item code keep the
  // ring in the same registers from the loads to the products.
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  if constexpr (MULTI) {
    // one item per wave.  In pass ps the item runs slice ksi of the pass's
    // units (so every wave works in every pass); before the next pass is
    // staged over X, the wave issues that pass's first units and every wave
    // leaves X.
    for (int ps = 0;; ++ps) {
      int pa, pe;
      pass_range(ps, pa, pe);
      if (have) acc = run_item(acc, pa, pe, ps * UPp);
      if (ps + 1 >= npass) break;
      int na, ne;
      pass_range(ps + 1, na, ne);
      stage(
          [&] {
            __builtin_amdgcn_sched_barrier(0);    // the activations' loads first
#pragma unroll
            for (int d = 0; d < kStQ; ++d) load_unit(d, na + d, ne);
            __builtin_amdgcn_sched_barrier(0);
            st_sync();                            // every wave done with this pass's X
          },
          ps + 1, std::false_type{});
      st_sync();
    }
    if (have && ksl == 1) store_direct(acc);
  } else if constexpr (LW) {
    if (have) {
      acc = run_item_lw(acc);
      if (ksl == 1) store_direct(acc);
    }
    if (ksl == 1) {
      for (it = wv + kStWaves; it < nitems; it += kStWaves) {
        set_item(it);
#pragma unroll
        for (int d = 0; d < kStPQ; ++d) issue_pair(d, (g0 >> 1) + d, (g1 + 1) >> 1);
        store_direct(run_item_lw(f32x4{0.0f, 0.0f, 0.0f, 0.0f}));
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the ring's last (empty) copies
  } else {
    if (have) {
      acc = run_item(acc, g0, g1, 0);
      if (ksl == 1) store_direct(acc);
    }
    if (ksl == 1) {
      for (it = wv + kStWaves; it < nitems; it += kStWaves) {
        set_item(it);
#pragma unroll
        for (int d = 0; d < kStQ; ++d) load_unit(d, g0 + d, g1);
        store_direct(run_item(f32x4{0.0f, 0.0f, 0.0f, 0.0f}, g0, g1, 0));
      }
    }
  }
  if (ksl > 1) {
    // one item per wave: the slices of a tile meet in LDS in slice order
    st_sync();                                    // every wave done with X
    if (wv < nitems) {
#pragma unroll
      for (int v = 0; v < 4; ++v) red[wv * 256 + (4 * b + v) * 16 + rl] = acc[v];
    }
    st_sync();
    for (int t = tid; t < ntile * 256; t += 1024) {
      const int tl = t >> 8, tk = (t >> 4) & 15, row = t & 15;
      float tot = 0.0f;
      for (int ks = 0; ks < ksl; ++ks) tot += red[(tl * ksl + ks) * 256 + tk * 16 + row];
      if (tk < M && tl * 16 + row < nrows) store_yst<YDT>(y, (int64_t)tk * ldy + r0 + tl * 16 + row, tot);
    }
  }
}

template <int DT, int YDT, bool HAS_R>
hipError_t st_dispatch(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, const uint32_t* qw,
                       const uint16_t* scales, const uint8_t* zeros, int64_t N, int glog, const float* r,
                       void* y, int64_t ldy, int nblk, hipStream_t st) {
  const int64_t rows_max = (N + nblk - 1) / nblk;
  const int64_t kp = st_kpass(M, K, rows_max, glog);
  const bool multi = kp < K;
  const StLayout L = st_layout(M, K, rows_max, glog, kp);
  const bool split = !multi && st_split(M, K, rows_max, glog);
  const bool lw = glog != 6 && !multi && L.total_lw <= kStLdsMax;
  size_t lds = lw ? L.total_lw : L.total;
  if (lds < 81 * 1024) lds = 81 * 1024;           // one block per compute unit
  const int np = split ? st_pieces(M, K, 512) : st_pieces(M, kp);
  const dim3 grid((unsigned)nblk), block(1024);
#define AWQ_ST(NP, G64, SPLIT, MULTI, LW)                                                            \
  hipLaunchKernelGGL((k_gemm_skinny_st<DT, YDT, HAS_R, NP, G64, SPLIT, MULTI, LW>), grid, block, lds, st, x, \
                     (int)M, K, ldx, r, qw, scales, zeros, N, y, ldy, glog, (uint32_t)L.sums,         \
                     (uint32_t)L.pinv, (uint32_t)L.meta, L.meta_pitch, (int)kp, (uint32_t)L.ring)
#define AWQ_STG(NP)                                     \
  if (multi) {                                          \
    if (glog == 6) AWQ_ST(NP < 4 ? NP : 4, true, false, true, false); \
    else AWQ_ST(NP, false, false, true, false);         \
  } else if (glog == 6) AWQ_ST(NP, true, false, false, false); \
  else if (split && lw) AWQ_ST(NP, false, true, false, true); \
  else if (split) AWQ_ST(NP, false, true, false, false); \
  else if (lw) AWQ_ST(NP, false, false, false, true);   \
  else AWQ_ST(NP, false, false, false, false)
  if (np == 1) AWQ_STG(1);
  else if (np == 2) AWQ_STG(2);
  else if (np == 4) AWQ_STG(4);
  else AWQ_STG(8);
#undef AWQ_STG
#undef AWQ_ST
  return hipGetLastError();
}

}  // namespace awqk

namespace awq {

int skinny_st_blocks(int64_t M, int64_t N, int64_t K, int group) {
  using namespace awqk;
  const int glog = group == 64 ? 6 : group == 128 ? 7 : group == 256 ? 8 : -1;
  if (glog < 0 || M < 2 || M > 16 || N < 1 || K % 128 != 0 || K % group != 0) return 0;
  const int64_t cus = device_cus();
  const int64_t nblk = N < cus ? N : cus;
  const int64_t rows_max = (N + nblk - 1) / nblk;
  // every block stages between 8 and 8192 (step, zero point) pairs
  if (rows_max * (K >> glog) > 1024 * kStMetaPer || (N / nblk) * (K >> glog) < kStMetaPer) return 0;
  if (rows_max * (K >> 1) >= (int64_t(1) << 31)) return 0;
  if (st_kpass(M, K, rows_max, glog) == 0) return 0;
  return (int)nblk;
}

// Row chunks that the kernel takes one launch at a time: 1 when one launch
// covers the layer; when only the block's steps and zero points (at most 8192
// pairs) keep one launch from covering it, the fewest chunks (2..16) whose
// every chunk one launch covers; else 0.
int skinny_st_chunks(int64_t M, int64_t N, int64_t K, int group) {
  if (skinny_st_blocks(M, N, K, group)) return 1;
  if (group <= 0 || K % group != 0 || N < 1) return 0;
  const int64_t cus = device_cus();
  const int64_t nblk = N < cus ? N : cus;
  const int64_t rows_max = (N + nblk - 1) / nblk;
  if (rows_max * (K / group) <= 1024 * awqk::kStMetaPer) return 0;
  for (int64_t c = 2; c <= 16 && c <= N; ++c)
    if (skinny_st_blocks(M, N / c, K, group) && skinny_st_blocks(M, (N + c - 1) / c, K, group)) return (int)c;
  return 0;
}

hipError_t launch_skinny_st(const void* x, int xdt, int64_t M, int64_t K, int64_t ldx,
                            const uint32_t* qw, const uint16_t* scales, const uint8_t* zeros,
                            int64_t N, int group, const float* inv_s, void* y, int ydt, int64_t ldy,
                            hipStream_t st) {
  using namespace awqk;
  const int nblk = skinny_st_blocks(M, N, K, group);
  if (nblk == 0) return hipErrorInvalidValue;
  const int glog = group == 64 ? 6 : group == 128 ? 7 : 8;
  const uint16_t* xp = (const uint16_t*)x;
#define AWQ_SD(XT, YT)                                                                                \
  return inv_s ? st_dispatch<XT, YT, true>(xp, M, K, ldx, qw, scales, zeros, N, glog, inv_s, y, ldy, nblk, st) \
               : st_dispatch<XT, YT, false>(xp, M, K, ldx, qw, scales, zeros, N, glog, inv_s, y, ldy, nblk, st)
  if (xdt == DT_F16) {
    if (ydt == DT_F16) AWQ_SD(DT_F16, DT_F16);
    if (ydt == DT_BF16) AWQ_SD(DT_F16, DT_BF16);
    AWQ_SD(DT_F16, DT_F32);
  }
  if (ydt == DT_F16) AWQ_SD(DT_BF16, DT_F16);
  if (ydt == DT_BF16) AWQ_SD(DT_BF16, DT_BF16);
  AWQ_SD(DT_BF16, DT_F32);
#undef AWQ_SD
}

hipError_t launch_skinny_st_chunked(const void* x, int xdt, int64_t M, int64_t K, int64_t ldx,
                                    const uint32_t* qw, const uint16_t* scales, const uint8_t* zeros,
                                    int64_t N, int group, const float* inv_s, void* y, int ydt, int64_t ldy,
                                    hipStream_t st) {
  const int c = skinny_st_chunks(M, N, K, group);
  if (c == 0) return hipErrorInvalidValue;
  const int64_t G = K / group;
  const int64_t yb = ydt == awqk::DT_F32 ? 4 : 2;
  for (int i = 0; i < c; ++i) {
    const int64_t n0 = (int64_t)i * N / c, n1 = (int64_t)(i + 1) * N / c;
    const hipError_t e = launch_skinny_st(x, xdt, M, K, ldx, qw + n0 * (K >> 3), scales + n0 * G, zeros + n0 * G,
                                          n1 - n0, group, inv_s, (uint8_t*)y + n0 * yb, ydt, ldy, st);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace awq
