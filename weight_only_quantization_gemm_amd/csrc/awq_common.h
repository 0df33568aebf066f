// Device-side helpers shared by the libawq kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kGroup = 128;     // input channels per quantization group
constexpr int kQmax = 15;       // largest 4-bit code

// Nibble position of the code of channel 8w+i inside packed word w: channels
// 8w+{0,2,4,6} sit in nibbles 0..3 and 8w+{1,3,5,7} in nibbles 4..7, so that
// (word >> 4j) & 0x000F000F holds channels 8w+2j and 8w+2j+1 in its halves.
__host__ __device__ constexpr int nibble_pos(int i) { return 4 * (i & 1) + (i >> 1); }

__device__ inline uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ inline f16x2 as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }

// The two codes of pair j of a packed word as fp16 (1024 + code): OR-ing a
// 4-bit integer into the mantissa of fp16 1024.0 (0x6400) yields 1024 + code
// exactly.
__device__ inline f16x2 pair_biased(uint32_t word, int j) {
  return as_f16x2(((word >> (4 * j)) & 0x000F000Fu) | 0x64006400u);
}

// The fp16x2 (1024, 1024) bit pattern in a vector register.  A VOP3 operand
// may not be a literal, so with the pattern in a register (and the mask in a
// scalar one) each pair unpacks with one and-or instead of an and and an or.
__device__ inline uint32_t bias_in_vgpr() {
  uint32_t v;
  __asm__ volatile("v_mov_b32 %0, 0x64006400" : "=v"(v));
  return v;
}

// pair_biased with the bias pattern from bias_in_vgpr().
__device__ inline f16x2 pair_biased(uint32_t word, int j, uint32_t bias) {
  return as_f16x2(((word >> (4 * j)) & 0x000F000Fu) | bias);
}

// fp16x2 (1024 + zero, 1024 + zero) for subtracting the zero point exactly.
__device__ inline f16x2 zero_biased(uint32_t zero) {
  return as_f16x2(0x64006400u | zero | (zero << 16));
}

// The zero point in the two forms word_minus_zero() subtracts: the fp16x2
// pairs (1024 + zero) and -(64 + zero) (64 has spacing 1/16, so zero sits at
// bit 4 of the mantissa; 0xD400 is -64).
struct ZeroForms {
  f16x2 zb1, nz64;
};
__device__ inline ZeroForms zero_forms(uint32_t zero) {
  return {as_f16x2(0x64006400u | zero | (zero << 16)), as_f16x2(0xD400D400u | (zero << 4) | (zero << 20))};
}

// The eight (code - zero) values of packed word w in channel order, exact, as
// a matrix-core operand.  With w8 = w >> 8, the four channel pairs are the
// 0x000F000F and 0x00F000F0 fields of w and of w8.  An and-or with the bias
// turns the low field into 1024 + code and the high field into 1024 + 16 code
// (below 2048, where the fp16 spacing is 1).  One packed subtraction of
// (1024 + zero) leaves code - zero for the low fields; one packed fma,
// (1024 + 16 code) / 16 - (64 + zero), does so for the high ones (the exact
// result is an integer of magnitude at most 15, so the single rounding is
// exact).  One shift per word instead of three.
__device__ inline f16x8 word_minus_zero(uint32_t w, uint32_t bias, ZeroForms z) {
  const f16x2 sixteenth = {(f16)0.0625f, (f16)0.0625f};
  const uint32_t w8 = w >> 8;
  const f16x2 q0 = as_f16x2((w & 0x000F000Fu) | bias) - z.zb1;
  const f16x2 q1 = __builtin_elementwise_fma(as_f16x2((w & 0x00F000F0u) | bias), sixteenth, z.nz64);
  const f16x2 q2 = as_f16x2((w8 & 0x000F000Fu) | bias) - z.zb1;
  const f16x2 q3 = __builtin_elementwise_fma(as_f16x2((w8 & 0x00F000F0u) | bias), sixteenth, z.nz64);
  return f16x8{q0.x, q0.y, q1.x, q1.y, q2.x, q2.y, q3.x, q3.y};
}

__device__ inline uint32_t zero_of(const uint8_t* zeros_row, int g) {
  return (zeros_row[g >> 1] >> (4 * (g & 1))) & 0xFu;
}

// Block barrier for LDS hand-offs only.  __syncthreads() also waits for every
// outstanding global load of the wave (vmcnt(0)), which would drain the
// prefetches of later pipeline stages; this waits for the wave's LDS
// operations (lgkmcnt(0)) and then meets the other waves at s_barrier.
// s_waitcnt immediate on gfx9: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] |
// vmcnt[5:4] in bits 15:14, so 0xC07F leaves vmcnt and expcnt at their maxima.
__device__ inline void lds_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

template <typename T>
__device__ inline T wave_sum(T v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

}  // namespace awq
