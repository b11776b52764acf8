// mfma_common.hpp -- register-level helpers shared by the MFMA matvec
// kernels: the 1MAD word in one v_mad_u64_u32, exact f16 code pairs built
// from the byte sums, and MFMA operand types.
#pragma once

#include "trellis_device.hpp"

namespace trellis {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

// Two f32 values as a packed f16 pair (round to nearest even, a first in the
// low half): one v_cvt_pk_f16_f32.
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v{a, b}, half2v));
}
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

// The exact codes y = b - 510 of two 1MAD words as a pair of f16 integers
// (normal numbers for y != 0; every integer up to 2048 is exact in f16).
// The byte sums b land in f16 bits directly: v_sad_hi_u8 / v_sad_u8 add them
// to the pattern 0x6402 in each half, which encodes 1026 + b in the binade
// [1024, 2048) of unit spacing (b <= 1020 keeps the mantissa below 1024, so
// no half carries into the other), and one packed f16 add of -1536 leaves
// y exactly.  Normal operands matter for the MFMA: it aligns its products
// to the operands' exponents, and a subnormal operand always counts with
// the smallest normal exponent, so products of subnormal codes with small
// activations would lose their low bits; integer codes keep each product
// aligned to its own magnitude.
constexpr uint32_t kHalfMagic2 = 0x64026402u;   // f16 1026 in both halves
constexpr uint32_t kNeg1536Pair = 0xE600E600u;  // f16 -1536 in both halves

__device__ __forceinline__ uint32_t code_pair_y(uint32_t word_lo, uint32_t word_hi) {
  const uint32_t both = __builtin_amdgcn_sad_u8(word_lo, 0u, __builtin_amdgcn_sad_hi_u8(word_hi, 0u, kHalfMagic2));
  const half2v h = __builtin_bit_cast(half2v, both) + __builtin_bit_cast(half2v, kNeg1536Pair);
  return __builtin_bit_cast(uint32_t, h);
}

// The 32 codes of one 32-position run (words w[0 .. K-1] and the word after
// it, wrapped in its block) as four MFMA A operands of 8 f16 integers: A[u]
// element e is the code y of run position 8u + e, whose state is the 12-bit
// window at bit (31 - 8u - e) K of the run.
template <int K>
__device__ __forceinline__ void decode_run_codes(const uint32_t (&w)[K + 1], uint32_t mul, uint64_t add64,
                                               u32x4 (&A)[4]) {
  uint32_t a[2 * K];                           // a[j] holds bits 16j .. 16j+31 of the run
#pragma unroll
  for (int m = 0; m < K; ++m) {
    a[2 * m] = w[m];
    a[2 * m + 1] = __builtin_amdgcn_alignbit(w[m + 1], w[m], 16);
  }
  // three phases, so no 1MAD result is consumed right after it is produced:
  // all 32 windows, all 32 1MAD words, then the 16 code pairs
  uint32_t st[32];
#pragma unroll
  for (int p = 0; p < 32; ++p) {
    const int b = (31 - p) * K;                 // window start of position p
    st[p] = __builtin_amdgcn_ubfe(a[b >> 4], b & 15, kL);
  }
  uint32_t xw[32];
#pragma unroll
  for (int p = 0; p < 32; ++p) xw[p] = onemad_word_mad64(st[p], mul, add64);
#pragma unroll
  for (int v = 0; v < 16; ++v) A[v >> 2][v & 3] = code_pair_y(xw[2 * v], xw[2 * v + 1]);
}

// Half a run: the 16 codes of positions 0..15 (upper = false) or 16..31
// (upper = true) of the run, as two MFMA A operands (A[u] element e is
// position 16 upper + 8u + e).  The windows of the upper half start 16 K
// bits lower in the run than those of the lower half, so both halves read
// the same compile-time offsets from a lane-selected set of 16-bit chunks.
template <int K>
__device__ __forceinline__ void decode_half_codes(const uint32_t (&w)[K + 1], bool upper, uint32_t mul,
                                                  uint64_t add64, u32x4 (&A)[2]) {
  uint32_t a[2 * K];                           // a[j] holds bits 16j .. 16j+31 of the run
#pragma unroll
  for (int m = 0; m < K; ++m) {
    a[2 * m] = w[m];
    a[2 * m + 1] = __builtin_amdgcn_alignbit(w[m + 1], w[m], 16);
  }
  uint32_t h[K];                               // chunks K .. 2K-1 (lower half) or 0 .. K-1 (upper)
#pragma unroll
  for (int j = 0; j < K; ++j) h[j] = upper ? a[j] : a[j + K];
  uint32_t st[16];
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const int b = (15 - p) * K;                 // window start of half position p, from the chunk base
    st[p] = __builtin_amdgcn_ubfe(h[b >> 4], b & 15, kL);
  }
  uint32_t xw[16];
#pragma unroll
  for (int p = 0; p < 16; ++p) xw[p] = onemad_word_mad64(st[p], mul, add64);
#pragma unroll
  for (int v = 0; v < 8; ++v) A[v >> 2][v & 3] = code_pair_y(xw[2 * v], xw[2 * v + 1]);
}

}  // namespace trellis
