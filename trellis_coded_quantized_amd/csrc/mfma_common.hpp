// mfma_common.hpp -- register-level helpers shared by the MFMA matvec
// kernels: the 1MAD word in one v_mad_u64_u32, exact f16 code pairs built
// from the byte sum, and MFMA operand types.
#pragma once

#include "trellis_device.hpp"

namespace trellis {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// 1MAD multiplier and addend in full (34038481, 76625530).
constexpr uint32_t kMul = 34038481u;

// Low 32 bits of s * 34038481 + 76625530 in one v_mad_u64_u32; its unused
// carry-out goes to a dead SGPR pair.  mul and add64 are loop-invariant registers.
__device__ __forceinline__ uint32_t onemad_word_mad64(uint32_t s, uint32_t mul, uint64_t add64) {
  uint64_t r;
  uint64_t carry;
  asm("v_mad_u64_u32 %0, %1, %2, %3, %4" : "=v"(r), "=s"(carry) : "v"(s), "v"(mul), "v"(add64));
  return (uint32_t)r;
}

// f16 bits 0x6402 + b encode 1026 + b exactly for a byte sum b in [0, 1020]
// (binade [1024, 2048) has unit spacing), i.e. y + 1536 with y = b - 510.
constexpr uint32_t kHalfMagic = 0x6402u;

// Pack the exact codes y(lo), y(hi) of two 1MAD words as an f16 pair:
// two byte sums land directly in f16 bits, then one packed subtract of 1536
// (exact: the difference is an integer of magnitude <= 510).
__device__ __forceinline__ uint32_t code_pair_f16(uint32_t word_lo, uint32_t word_hi,
                                                  uint32_t magic) {
  const uint32_t hi = __builtin_amdgcn_sad_u8(word_hi, 0u, magic);
  const uint32_t both = __builtin_amdgcn_sad_u8(word_lo, 0u, (hi << 16) | magic);
  half2v h = __builtin_bit_cast(half2v, both);
  h = h + half2v{(_Float16)-1536.0f, (_Float16)-1536.0f};
  return __builtin_bit_cast(uint32_t, h);
}

}  // namespace trellis
