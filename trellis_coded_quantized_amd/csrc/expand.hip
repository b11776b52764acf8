// expand.hip -- decode a whole packed matrix on gfx950.
//
// trellis_expand_bf16: a thread owns four adjacent positions of one block;
// one 64-bit circular window (two words, the second wrapping to word 0 at
// the block end) holds all four states.  value * scale is rounded to f32 and
// then to bf16 (nearest even), and the four bf16 go out as one 8-byte store.
//   Source: mlx-bun 0.2.0 -> 0.4.0 diff (page 55), trellis-linear.ts EXPAND
//   kernel; page 56, trellis-vector-expand.ts (four weights per window).
//
// trellis_decode_states: the same decode, one thread per weight, exporting
// the state, the 1MAD code and the f32 code value for bit-exact tests.
#include "internal.hpp"
#include "trellis_device.hpp"

namespace trellis {
namespace {

template <int K>
__device__ __forceinline__ uint64_t quad_window(const uint32_t* __restrict__ blk, int t0) {
  constexpr int WPB = words_per_block(K);
  const int pos = (kT - 1 - (t0 + 3)) * K;
  const int wi = pos >> 5, off = pos & 31;
  const int wn = (wi + 1 == WPB) ? 0 : wi + 1;
  return ((uint64_t)blk[wn] << 32 | blk[wi]) >> off;
}

template <int K>
__global__ __launch_bounds__(256) void expand_kernel(const uint32_t* __restrict__ codes,
                                                     const uint16_t* __restrict__ scales,
                                                     uint16_t* __restrict__ out, int64_t R,
                                                     int64_t C) {
  constexpr int WPB = words_per_block(K);
  const int64_t quads = C / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= R * quads) return;
  const int64_t r = idx / quads;
  const int64_t c0 = (idx - r * quads) * 4;
  const int blk = (int)(c0 / kT), t0 = (int)(c0 % kT);
  const uint32_t* bw = codes + r * (C / kT) * WPB + (int64_t)blk * WPB;
  const uint64_t win = quad_window<K>(bw, t0);
  const float sc = half_bits_to_f32(scales[r]);
  uint32_t h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t s = (uint32_t)(win >> ((3 - i) * K)) & kStateMask;
    h[i] = f32_to_bf16_bits(code_value(code_y(s)) * sc);
  }
  uint2 v;
  v.x = h[0] | (h[1] << 16);
  v.y = h[2] | (h[3] << 16);
  *reinterpret_cast<uint2*>(out + r * C + c0) = v;
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
                         int64_t C, int k, hipStream_t stream) {
  const int64_t n = R * (C / 4);
  const dim3 grid((unsigned)((n + 255) / 256)), block(256);
  switch (k) {
    case 2: hipLaunchKernelGGL(expand_kernel<2>, grid, block, 0, stream, codes, scales, out, R, C); break;
    case 3: hipLaunchKernelGGL(expand_kernel<3>, grid, block, 0, stream, codes, scales, out, R, C); break;
    case 4: hipLaunchKernelGGL(expand_kernel<4>, grid, block, 0, stream, codes, scales, out, R, C); break;
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
