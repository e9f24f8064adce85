// Device-side helpers shared by the gfx950 kernels of the AWQ hot path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awqk {

constexpr int kWave = 64;             // CDNA wavefront width

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Element type tags: 0 = fp16, 1 = bf16 (same values as awq_dtype).
enum : int { DT_F16 = 0, DT_BF16 = 1, DT_F32 = 2 };

// Two fp16 from a 32-bit pattern.  Takes the value: a vector element such as
// v[1] must not be handed to __builtin_bit_cast directly (this compiler then
// reads element 0 of the vector).
__device__ __forceinline__ f16x2 as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits16);
  return (float)h;
}
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
template <int DT>
__device__ __forceinline__ float to_f32(uint32_t bits16) {
  if constexpr (DT == DT_F16) return f16_to_f32(bits16);
  else return bf16_to_f32(bits16);
}
// The low / high 16-bit element of a 32-bit word as float.
template <int DT>
__device__ __forceinline__ float lo_f32(uint32_t w) {
  if constexpr (DT == DT_F16) return f16_to_f32(w & 0xFFFFu);
  else return __uint_as_float(w << 16);
}
template <int DT>
__device__ __forceinline__ float hi_f32(uint32_t w) {
  if constexpr (DT == DT_F16) return f16_to_f32(w >> 16);
  else return __uint_as_float(w & 0xFFFF0000u);
}

// Round-to-nearest-even conversions to 16-bit storage.
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
template <int DT>
__device__ __forceinline__ uint32_t from_f32(float f) {
  if constexpr (DT == DT_F16) return f32_to_f16_bits(f);
  else return f32_to_bf16_bits(f);
}

// Smallest fp16 >= d for finite d > 0 (round toward +inf), as bits.  For a
// positive fp16 the next larger value is the next bit pattern (0x7BFF + 1 is
// +inf, matching IEEE nextUp).
__device__ __forceinline__ uint32_t f16_round_up_bits(float d) {
  _Float16 h = (_Float16)d;
  uint32_t b = __builtin_bit_cast(uint16_t, h);
  if ((float)h < d) b += 1u;
  return b;
}

// One quantizer grid.  Asymmetric N bits: 2^N levels, the step is the
// group's range (holding 0) over 2^N - 1 and the zero point an integer code.
// Symmetric N bits: the step is max|w| / 2^(N-1) and the codes run over
// -2^(N-1) .. 2^(N-1) (2^N + 1 levels), stored shifted up by 2^(N-1).
struct QSpec {
  float div;     // asymmetric: 2^N - 1; symmetric: 2^(N-1)
  float cmax;    // largest stored code: 2^N - 1, or 2^N
  bool sym;
};
constexpr QSpec kQ4 = {15.0f, 15.0f, false};     // the 4-bit asymmetric grid
__host__ __device__ constexpr QSpec qspec(int bits, bool sym) {
  return sym ? QSpec{(float)(1 << (bits - 1)), (float)(1 << bits), true}
             : QSpec{(float)((1 << bits) - 1), (float)((1 << bits) - 1), false};
}

// Integer zero point and step of one group, shared by the quantizer and the
// search's error generator so both score and store the same grid.
struct GroupGrid {
  float D;          // step as float (fp16 value)
  float z;          // zero point as float
  float d;          // step before rounding
  float cmax;       // largest stored code
  uint32_t step_bits;
};

// SYM must equal q.sym: the grid is chosen at compile time so that each thread
// computes only its own step.
template <bool SYM = false>
__device__ __forceinline__ GroupGrid group_grid(float mn, float mx, const QSpec q = kQ4) {
  GroupGrid g;
  float lo = 0.0f;
  if constexpr (SYM) {
    // max|w| / 2^(N-1), exact; 0 when every weight of the group is left out
    g.d = fmaxf(fmaxf(-mn, mx), 0.0f) / q.div;
  } else {
    lo = fminf(mn, 0.0f);
    const float hi = fmaxf(mx, 0.0f);
    g.d = (hi - lo) / q.div;                          // IEEE division
  }
  g.step_bits = f16_round_up_bits(fmaxf(g.d, 0x1p-24f));
  g.D = f16_to_f32(g.step_bits);
  if constexpr (SYM) g.z = q.div;
  else g.z = fminf(fmaxf(rintf(-lo / g.D), 0.0f), q.cmax);
  g.cmax = q.cmax;
  return g;
}

__device__ __forceinline__ float quant_code(float wp, const GroupGrid& g) {
  return fminf(fmaxf(rintf(wp / g.D) + g.z, 0.0f), g.cmax);
}

// Raw buffer access: the fourth descriptor word for untyped 32-bit data, an
// offset that is always out of range (the load returns 0 and reads nothing),
// and the non-temporal cache policy bit for streamed weights.
constexpr int kBufferWord3 = 0x00020000;
constexpr uint32_t kBufferOob = 0x80000000u;
constexpr int kBufferNt = 2;

// Min / max across the GL lanes of an aligned GL-lane segment (one group:
// GL threads of 8 weights each).
template <int GL>
__device__ __forceinline__ void seg_minmax(float& mn, float& mx) {
  static_assert(GL == 8 || GL == 16 || GL == 32, "group of 64, 128 or 256");
#pragma unroll
  for (int off = GL / 2; off >= 1; off >>= 1) {
    mn = fminf(mn, __shfl_xor(mn, off, GL));
    mx = fmaxf(mx, __shfl_xor(mx, off, GL));
  }
}

__device__ __forceinline__ u32x4 ldg128(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Streaming 128-bit load that is not expected to be reused (packed weights).
__device__ __forceinline__ u32x4 ldg128_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// A 32-bit constant held in a scalar register.  Three-operand VALU
// instructions cannot encode a 32-bit literal on this target, so a mask that is
// meant to feed v_and_or_b32 lives in an SGPR (one scalar operand per VALU op).
template <uint32_t V>
__device__ __forceinline__ uint32_t sgpr_const() {
  uint32_t r;
  asm("s_mov_b32 %0, %1" : "=s"(r) : "i"(V));
  return r;
}
// The same, held in a vector register (the second non-literal operand).
template <uint32_t V>
__device__ __forceinline__ uint32_t vgpr_const() {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(V));
  return r;
}

// Butterfly steps across a wave.  pair_sum32(a, b): lanes 0..31 return
// a(l) + a(l + 32), lanes 32..63 return b(l - 32) + b(l) (one v_permlane32_swap
// moves the upper half of a and the lower half of b across).  pair_sum16 is the
// same between the even and odd 16-lane rows.
__device__ __forceinline__ float pair_sum32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_sum16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Value of lane l ^ 1 / l ^ 2 (DPP quad permutes).
__device__ __forceinline__ float quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}
// Sum over each 16-lane row; lane 16 j ends with the total of row j (DPP
// mirror, half-mirror and quad exchanges, no LDS traffic).
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row_mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  v += quad_xor2(v);
  v += quad_xor1(v);
  return v;
}

// ---- matrix cores and LDS DMA ----------------------------------------------
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// D += A B for one 32 x 32 x 16 fp16 block (fp32 accumulation).  A lane holds
// 8 k of row l % 32 (k half l / 32); the result lane holds column l % 32 and
// rows 8 (v / 4) + 4 (l / 32) + v % 4 of its 16 values.
__device__ __forceinline__ f32x16 mfma32h(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16h(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Raw buffer descriptor: base address, stride 0, size in bytes, untyped dwords.
// The arguments must be the same in every lane; the words are taken from the
// first active lane so that the descriptor lives in scalar registers.
__device__ __forceinline__ i32x4 rsrc4(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int32_t)((uint32_t)(a >> 32) & 0xFFFFu));
  r[2] = __builtin_amdgcn_readfirstlane((int32_t)bytes);
  r[3] = kBufferWord3;
  return r;
}

// 16 bytes per lane from a raw buffer into LDS at lds + 16 lane (LDS DMA; an
// offset past the buffer's end writes 0).  The copy writes no register.  It is
// issued from asm so that the compiler, which cannot tell which LDS stage a
// copy fills, adds no wait of its own before the other stages' LDS reads: the
// caller waits for the copies explicitly (vector memory counter, in order)
// before the barrier that publishes a stage.
// m0 (the LDS base of the copy) is saved and restored around it.
__device__ __forceinline__ void dma16(const i32x4& r, uint32_t lds, uint32_t voff, uint32_t soff) {
  uint32_t keep;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, %4 offen lds\n\ts_mov_b32 m0, %0"
               : "=&s"(keep) : "s"(lds), "v"(voff), "s"(r), "s"(soff) : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// Workgroup barrier that waits for nothing: the LDS DMA copies a wave has in
// flight are waited for explicitly (waitcnt_vm) before it, where __syncthreads
// would wait for all of them.  The memory clobber keeps the compiler from
// moving LDS reads across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt immediates on this target: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt[5:4] in bits [15:14].  waitcnt_vm waits for the vector memory counter
// only (n <= 63), waitcnt_vm_lgkm0 also for every LDS access of the wave.
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int waitcnt_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

}  // namespace awqk
