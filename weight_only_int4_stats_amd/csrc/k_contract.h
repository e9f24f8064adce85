// One 256 x 256 tile of C = A B^T with 16-bit operands on the matrix cores
// (fp32 accumulation), shared by the search's contractions.
//
// Both operands are 256 rows (tokens, error rows, channels ...) of 16-bit
// values along the contraction index k, each row at its own stride in a raw
// buffer (rows past the buffer's end arrive as zeros).  The block has 4 waves,
// one per SIMD (2 x 2; each wave 128 x 128 = 4 x 4 blocks of 32 x 32, its 256
// accumulators per lane in the accumulation registers).  32 k per stage; four
// LDS stages, filled by LDS DMA (buffer_load ... lds) three stages ahead of the
// matrix-core work.  A stage holds both operands, 256 rows x 32 k each (64
// bytes a row, a quarter of the 64 banks); row r's 16-byte chunk c sits at
// chunk c ^ ((r / 4) mod 4), so the 16 rows that one 16-lane pass of a
// 128-bit read touches land on 16 different bank slots.  Inside a wave the
// operand fragments of the next 16 k are read from LDS while the 16 products
// of the current 16 k run (two register sets), and the copies of the next
// stages go out between the products.
#pragma once

#include "awq_device.h"

namespace awqk {

constexpr int kCT = 256;                 // tile edge
constexpr int kCBK = 32;                 // k per stage
constexpr int kCOp = kCT * kCBK * 2;     // bytes per operand and stage (16 KB)
constexpr int kCWaves = 4;
constexpr int kCCopies = 2 * (kCOp / 1024) / kCWaves;   // 1 KB copies per wave and stage (8)
constexpr int kCStage = 2 * kCOp;        // LDS bytes per stage

__device__ __forceinline__ f32x16 mfma32bf(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

struct ContractSrc {
  i32x4 ars;          // A rows (raw buffer)
  uint32_t a_ld;      // A row stride in bytes
  i32x4 brs;          // B rows
  uint32_t b_ld;      // B row stride in bytes
  uint32_t k0;        // first k, in bytes from each row's start
  uint32_t a_dup_sh;  // > 0: every 2^a_dup_sh-byte block of A's k range serves two
                      // consecutive such blocks of k (B's range is twice A's)
  int64_t S;          // stages of 32 k; a multiple of 4, at least 4
};

struct ContractFrags {
  u32x4 a[4], b[4];
};

// acc[mb][nb] (zeroed by the caller) += A rows wm 128 + mb 32 + 0..31 times
// B rows wn 128 + nb 32 + 0..31 over the source's k range, for wave (wm, wn) =
// (wave / 2, wave % 2).  Result layout (32 x 32 blocks): lane holds B row
// lane % 32 and A rows 8 (v / 4) + 4 (lane / 32) + v % 4 of its 16 values.
template <bool BF16>
__device__ __forceinline__ void contract_tile(const ContractSrc& cs, uint8_t* lds0, uint8_t* lds1,
                                              uint8_t* lds2, uint8_t* lds3, f32x16 (&acc)[4][4]) {
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wv >> 1, wn = wv & 1;
  const int64_t S = cs.S;

  // Copy j (0..15) of an operand fills its bytes [1024 j, 1024 j + 1024) =
  // rows 16 j .. 16 j + 15; wave w issues j = 4 w + u.  Lane i: row
  // r = 16 j + i / 4 at chunk i % 4, which holds global chunk (i % 4) ^ ((r / 4) % 4).
  uint32_t aoff[4], boff[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 16 * (4 * wv + u) + (lane >> 2);
    const uint32_t ch = (uint32_t)(((lane & 3) ^ ((r >> 2) & 3)) * 16);
    aoff[u] = (uint32_t)r * cs.a_ld + ch;
    boff[u] = (uint32_t)r * cs.b_ld + ch;
  }
  // copy u (0..7) of stage s into the stage array at base: A copies 0..3, B 4..7
  auto copy = [&](int64_t s, const uint8_t* base, int u) {
    const uint32_t kb = cs.k0 + (uint32_t)(s * kCBK * 2);
    const uint32_t ka =
        cs.a_dup_sh ? ((kb >> (cs.a_dup_sh + 1)) << cs.a_dup_sh) | (kb & ((1u << cs.a_dup_sh) - 1u)) : kb;
    const uint32_t lb = __builtin_amdgcn_readfirstlane(lds_addr(base));
    if (u < 4) dma16(cs.ars, lb + (4 * wv + u) * 1024, aoff[u], ka);
    else dma16(cs.brs, lb + kCOp + (4 * wv + u - 4) * 1024, boff[u - 4], kb);
  };
  auto issue = [&](int64_t s, const uint8_t* base) {
#pragma unroll
    for (int u = 0; u < kCCopies; ++u) copy(s, base, u);
  };

  // fragment i (0..7) of 16 k (half ks of a stage), in the order the products
  // use them: a0 b0 b1 b2 b3 a1 a2 a3 (8 k of chunk 2 ks + lane / 32)
  auto read1 = [&](const uint8_t* base, int ks, ContractFrags& f, int i) {
    const int c = 2 * ks + (lane >> 5);
    if (i >= 1 && i <= 4) {
      const int r = wn * 128 + (i - 1) * 32 + (lane & 31);
      f.b[i - 1] = *reinterpret_cast<const u32x4*>(base + kCOp + r * 64 + ((c ^ ((r >> 2) & 3)) * 16));
    } else {
      const int mb = i == 0 ? 0 : i - 4;
      const int r = wm * 128 + mb * 32 + (lane & 31);
      f.a[mb] = *reinterpret_cast<const u32x4*>(base + r * 64 + ((c ^ ((r >> 2) & 3)) * 16));
    }
  };
  // products 2 i and 2 i + 1 of the 16 (A block i / 2, B blocks 2 (i % 2) + 0, 1)
  auto mma2 = [&](const ContractFrags& f, int i) {
    const int mb = i >> 1, nb = (i & 1) * 2;
    if constexpr (BF16) {
      acc[mb][nb] = mfma32bf(f.a[mb], f.b[nb], acc[mb][nb]);
      acc[mb][nb + 1] = mfma32bf(f.a[mb], f.b[nb + 1], acc[mb][nb + 1]);
    } else {
      acc[mb][nb] = mfma32h(f.a[mb], f.b[nb], acc[mb][nb]);
      acc[mb][nb + 1] = mfma32h(f.a[mb], f.b[nb + 1], acc[mb][nb + 1]);
    }
  };

  // S is a multiple of 4 (and at least 4): the loop below runs whole groups of
  // four stages and the last group is peeled, which keeps every wait count a
  // constant.
  ContractFrags f0, f1;
  // prologue: stages 0..2 in flight, stage 0 published, stage 3 issued
  issue(0, lds0);
  issue(1, lds1);
  issue(2, lds2);
  __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kCCopies));
  lds_barrier();
  issue(3, lds3);
#pragma unroll
  for (int i = 0; i < 8; ++i) read1(lds0, 0, f0, i);

  // Stage s in two halves of 16 products.  First half: the products of f0
  // (first 16 k), with the second 16 k read into f1 one fragment per two
  // products.  Then stage s + 1 is published, once all but the `ahead` stages
  // copied after it have landed and every LDS read of the wave has returned
  // (so all of stage s has been read); second half: the products of f1, with
  // one copy of stage s + 4 into stage s's array and one fragment of stage
  // s + 1's first 16 k per two products.  Issuing copies and reads between
  // products keeps the matrix pipe fed while they queue; scheduling barriers
  // hold that order.
  auto stage = [&](int64_t s, const uint8_t* cur, const uint8_t* nxt, int ahead, bool refill) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mma2(f0, i);
      read1(cur, 1, f1, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (ahead == 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(2 * kCCopies));
    else if (ahead == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(kCCopies));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    lds_barrier();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      mma2(f1, i);
      if (refill) copy(s + 4, cur, i);
      read1(nxt, 0, f0, i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  int64_t s = 0;
  for (; s < S - 4; s += 4) {
    stage(s, lds0, lds1, 2, true);
    stage(s + 1, lds1, lds2, 2, true);
    stage(s + 2, lds2, lds3, 2, true);
    stage(s + 3, lds3, lds0, 2, true);
  }
  stage(s, lds0, lds1, 2, false);
  stage(s + 1, lds1, lds2, 1, false);
  stage(s + 2, lds2, lds3, 0, false);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    mma2(f0, i);
    read1(lds3, 1, f1, i);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) mma2(f1, i);
}

}  // namespace awqk
