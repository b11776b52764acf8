// trellis_device.hpp -- gfx950 device-side decode primitive for packed
// trellis-coded weights, kept entirely in registers (no table).
//
// Format and decode: mlx-bun 0.2.0 -> 0.4.0 diff (page 55),
// src/model/trellis-linear.ts, file header comment (uint32 bitstream
// [rows, cols*k/32], one fp16 scale per stored row, blocks of T symbols) and
// the HEADER helpers: trellis_state (cyclic L-bit window at bit (T-1-t)*k of
// the block), trellis_y (1MAD code), trellis_val / trellis_val_rcp (value =
// y / 147.800537109375, correctly rounded via one residual step).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace trellis {

constexpr int kL = 12;                         // state bits
constexpr int kT = 256;                        // symbols per block
constexpr uint32_t kStateMask = (1u << kL) - 1u;

// 1MAD: x = s * 34038481 + 76625530 (mod 2^32).  34038481 = 2 * 2^24 + 484049,
// so for a 12-bit state the product is a 24-bit multiply plus s << 25.
constexpr uint32_t kMulLow24 = 484049u;
constexpr uint32_t kAdd = 76625530u;
constexpr int kYOffset = 510;                  // the byte sum minus this is y

constexpr float kDiv = 147.800537109375f;      // exact in binary32 (605391 / 4096)
constexpr float kRcp = 1.0f / 147.800537109375f;

// Words per block of T k-bit symbols.
__host__ __device__ constexpr int words_per_block(int k) { return kT * k / 32; }

// L-bit window starting `off` (0..31) bits into the 64-bit little-endian pair
// (lo, hi): bits [off, off + 12) with lo holding bits 0..31.
__device__ __forceinline__ uint32_t window(uint32_t lo, uint32_t hi, uint32_t off) {
  return __builtin_amdgcn_alignbit(hi, lo, off) & kStateMask;
}

// The 32-bit 1MAD word of a 12-bit state.
__device__ __forceinline__ uint32_t onemad_word(uint32_t s) {
  return __umul24(s, kMulLow24) + (s << 25) + kAdd;
}

// y = (sum of the four bytes of the 1MAD word) - 510, in [-510, 510].
// v_sad_u8 against zero is the byte sum in one instruction.
__device__ __forceinline__ int code_y(uint32_t s) {
  return (int)__builtin_amdgcn_sad_u8(onemad_word(s), 0u, 0u) - kYOffset;
}

// Code value y / d rounded to nearest binary32, in two operations: the
// reciprocal split as kRcp + kRcpLo (kRcpLo = 1/d - kRcp rounded to binary32)
// and y * kRcp + RN(y * kRcpLo) under one fused rounding.  Checked exactly,
// with rational arithmetic, to be correctly rounded for every |y| <= 510.
constexpr float kRcpLo = -0x1.e90d7cp-33f;

__device__ __forceinline__ float code_value(int y) {
  const float yf = (float)y;
  return __builtin_fmaf(yf, kRcp, yf * kRcpLo);
}

__device__ __forceinline__ float half_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Round to nearest even bf16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float round_bf16(float f) {
  return bf16_bits_to_f32(f32_to_bf16_bits(f));
}

}  // namespace trellis
