// expand.hip -- decode a whole packed matrix on gfx950.
//
// trellis_expand_bf16: a thread owns one run of 32 consecutive positions of
// one block (an eighth of a block).  The run's windows start on
// a word boundary, so its k + 1 code words (the last wrapping to word 0 at
// the block end) hold all 32 states.  value * scale is rounded to f32 and
// then to bf16 (nearest even); a wave's 64 runs fill one contiguous 4 KB
// block of the output, which leaves through LDS as four fully coalesced
// 1 KB stores.  The decode is VALU work of about nine operations per weight and
// the kernel is otherwise bound by its 2-byte-per-weight writes.
//   Source: mlx-bun 0.2.0 -> 0.4.0 diff (page 55), trellis-linear.ts EXPAND
//   kernel; page 56, trellis-vector-expand.ts (several weights per window).
//
// trellis_decode_states: the same decode, one thread per weight, exporting
// the state, the 1MAD code and the f32 code value for bit-exact tests.
#include "internal.hpp"
#include "mfma_common.hpp"
#include "trellis_device.hpp"

namespace trellis {
namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int K>
__global__ __launch_bounds__(256) void expand_kernel(const uint32_t* __restrict__ codes,
                                                     const uint16_t* __restrict__ scales,
                                                     uint16_t* __restrict__ out, int R, int C,
                                                     int interleave) {
  constexpr int WPB = words_per_block(K);
  __shared__ u32x4 tb[256 * 4];                              // 4 KB per wave
  const int runs = C / 32;                                   // runs per row
  const int total = R * runs;
  const int idx = (int)blockIdx.x * 256 + (int)threadIdx.x;
  const bool live = idx < total;
  const int r = live ? idx / runs : 0, run = live ? idx - r * runs : 0;
  const int blk = run >> 3, j = run & 7;
  // Positions 32 j .. 32 j + 31 of the block: lowest window bit (224 - 32 j) K,
  // i.e. word (7 - j) K; position 32 j + i sits (31 - i) K bits above it.
  // row-major [R, C*k/32], or block-interleaved [C/512, R, 2 WPB] (two blocks
  // of a row side by side, rows one after another within each pair of blocks)
  const uint32_t* bw = interleave ? codes + (((int64_t)(blk >> 1) * R + r) * 2 + (blk & 1)) * WPB
                                  : codes + (int64_t)r * (C / kT) * WPB + blk * WPB;
  const int w0 = (7 - j) * K;
  uint32_t w[K + 1];
#pragma unroll
  for (int q = 0; q <= K; ++q) w[q] = live ? bw[(w0 + q >= WPB) ? w0 + q - WPB : w0 + q] : 0u;
  const float sc = half_bits_to_f32(scales[r]);               // row 0 for idle threads
  const uint32_t mul = kMul;
  const uint64_t add64 = kAdd;
  uint32_t pk[16];
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    float f[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int rel = (31 - (2 * p + e)) * K;
      const int wi = rel >> 5, ro = rel & 31;
      const uint32_t st = (ro + kL <= 32) ? (w[wi] >> ro) & kStateMask : window(w[wi], w[wi + 1], (uint32_t)ro);
      // y = byte sum - 510: v_sad_u8 accumulates onto -510 (mod 2^32)
      const int y = (int)__builtin_amdgcn_sad_u8(onemad_word_mad64(st, mul, add64), 0u, (uint32_t)-kYOffset);
      f[e] = code_value(y) * sc;
    }
    pk[p] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){f[0], f[1]}, bf16x2));
  }
  // Thread idx's 64 bytes belong at byte 64 idx of out (runs are consecutive
  // along rows and rows are consecutive), so a wave's output is one 4 KB
  // block.  It goes through LDS so that every store instruction writes 1 KB
  // of consecutive 16-byte pieces.
  const int lane = (int)threadIdx.x & 63, wbase = (int)threadIdx.x & ~63;
#pragma unroll
  for (int q = 0; q < 4; ++q) tb[(int)threadIdx.x * 4 + q] = u32x4{pk[4 * q], pk[4 * q + 1], pk[4 * q + 2], pk[4 * q + 3]};
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int first = (int)blockIdx.x * 256 + wbase;           // first run of this wave
  u32x4* dst = reinterpret_cast<u32x4*>(out) + (int64_t)first * 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = lane + 64 * q;                             // 16-byte piece c of the wave's block
    if (first + (c >> 2) < total) dst[c] = tb[wbase * 4 + c];
  }
}

template <int K>
__global__ __launch_bounds__(256) void decode_states_kernel(const uint32_t* __restrict__ codes,
                                                            int64_t R, int64_t C,
                                                            uint16_t* __restrict__ states,
                                                            int16_t* __restrict__ ys,
                                                            float* __restrict__ values) {
  constexpr int WPB = words_per_block(K);
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= R * C) return;
  const int64_t r = idx / C, c = idx - r * C;
  const int blk = (int)(c / kT), t = (int)(c % kT);
  const uint32_t* bw = codes + r * (C / kT) * WPB + (int64_t)blk * WPB;
  const int p = (kT - 1 - t) * K;
  const int wi = p >> 5, off = p & 31;
  const int wn = (wi + 1 == WPB) ? 0 : wi + 1;
  const uint32_t s = window(bw[wi], bw[wn], off);
  const int y = code_y(s);
  if (states) states[idx] = (uint16_t)s;
  if (ys) ys[idx] = (int16_t)y;
  if (values) values[idx] = code_value(y);
}

}  // namespace

hipError_t launch_expand(const uint32_t* codes, const uint16_t* scales, uint16_t* out, int64_t R,
                         int64_t C, int k, hipStream_t stream, int interleave) {
  const int64_t n = R * (C / 32);
  if (n >= ((int64_t)1 << 31)) return hipErrorInvalidValue;   // one thread per run, 32-bit indices
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  const int r = (int)R, c = (int)C;
  switch (k) {
    case 2: hipLaunchKernelGGL(expand_kernel<2>, grid, block, 0, stream, codes, scales, out, r, c, interleave); break;
    case 3: hipLaunchKernelGGL(expand_kernel<3>, grid, block, 0, stream, codes, scales, out, r, c, interleave); break;
    case 4: hipLaunchKernelGGL(expand_kernel<4>, grid, block, 0, stream, codes, scales, out, r, c, interleave); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_states(const uint32_t* codes, int64_t R, int64_t C, int k,
                                uint16_t* states, int16_t* y, float* value, hipStream_t stream) {
  const int64_t n = R * C;
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  switch (k) {
    case 2: hipLaunchKernelGGL(decode_states_kernel<2>, grid, block, 0, stream, codes, R, C, states, y, value); break;
    case 3: hipLaunchKernelGGL(decode_states_kernel<3>, grid, block, 0, stream, codes, R, C, states, y, value); break;
    case 4: hipLaunchKernelGGL(decode_states_kernel<4>, grid, block, 0, stream, codes, R, C, states, y, value); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace trellis
