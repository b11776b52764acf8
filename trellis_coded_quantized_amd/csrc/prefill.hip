// prefill.hip -- fused axis-1 prefill on gfx950: packed codes are decoded
// into an LDS tile of bf16 weights that feeds bf16 MFMA directly, so no
// expanded weight matrix ever exists in HBM.
//
// out[m, r] = bf16( sum_c wb(r, c) * x[m, c] ),  wb = bf16(f32(value * scale))
// Source: mlx-bun 0.2.0 -> 0.4.0 diff (page 56), trellis-tiled-prefill.ts
// (x tile and reconstructed bf16 weight tile in threadgroup memory, matrix
// multiply-accumulate in f32; precise value before the bf16 weight rounding).
//
// Tiling: workgroup of 4 waves computes a 128 (m) x 128 (r) output tile with
// K steps of 64 columns; each wave owns a 64 x 64 quadrant made of 4 x 4
// v_mfma_f32_16x16x32_bf16 tiles.  Per K step every thread decodes one run
// of 32 positions of one weight row (k + 1 words, constant shifts).
#include "internal.hpp"
#include "trellis_device.hpp"

namespace trellis {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLds = kBK + 8;   // padded LDS row (elements): spreads 16-byte reads over banks

template <int K>
__global__ __launch_bounds__(256) void prefill_fused_kernel(const uint32_t* __restrict__ codes,
                                                            const uint16_t* __restrict__ scales,
                                                            const uint16_t* __restrict__ x,
                                                            uint16_t* __restrict__ out, int64_t R,
                                                            int64_t C, int64_t M) {
  constexpr int WPB = words_per_block(K);
  __shared__ __attribute__((aligned(16))) uint16_t As[kBM * kLds];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[kBN * kLds];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int drow = tid >> 1, dhalf = tid & 1;   // decode: one 32-position run per thread
  const int64_t grow = n0 + drow;
  const bool rvalid = grow < R;
  const uint32_t* crow = codes + (rvalid ? grow : 0) * (C / kT) * WPB;
  const float sc = rvalid ? half_bits_to_f32(scales[grow]) : 0.0f;

  for (int64_t kb = 0; kb < C; kb += kBK) {
    // x tile [128 m][64 k] -> As
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int idx = tid + 256 * j;
      const int r = idx >> 3, cv = idx & 7;
      const int64_t gm = m0 + r;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (gm < M) v = *reinterpret_cast<const uint4*>(x + gm * C + kb + 8 * cv);
      *reinterpret_cast<uint4*>(&As[r * kLds + 8 * cv]) = v;
    }
    // weight tile [128 r][64 k] -> Bs, decoded in registers
    {
      uint32_t packed[16];
      if (rvalid) {
        const int64_t c0 = kb + 32 * dhalf;
        const int blk = (int)(c0 / kT), q = (int)((c0 % kT) / 32);
        const uint32_t* bw = crow + (int64_t)blk * WPB;
        const int w0 = (7 - q) * K;
        uint32_t w[K + 1];
#pragma unroll
        for (int i = 0; i < K; ++i) w[i] = bw[w0 + i];
        w[K] = bw[(w0 + K == WPB) ? 0 : w0 + K];
#pragma unroll
        for (int i = 0; i < 32; i += 2) {
          const int pa = (31 - i) * K, pb = (30 - i) * K;
          const uint32_t sa = window(w[pa >> 5], w[(pa >> 5) + 1], pa & 31);
          const uint32_t sb = window(w[pb >> 5], w[(pb >> 5) + 1], pb & 31);
          const uint32_t ha = f32_to_bf16_bits(code_value(code_y(sa)) * sc);
          const uint32_t hb = f32_to_bf16_bits(code_value(code_y(sb)) * sc);
          packed[i >> 1] = ha | (hb << 16);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) packed[i] = 0u;
      }
      uint4* dst = reinterpret_cast<uint4*>(&Bs[drow * kLds + 32 * dhalf]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        dst[j] = make_uint4(packed[4 * j], packed[4 * j + 1], packed[4 * j + 2], packed[4 * j + 3]);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      bf16x8 a[4], b[4];
      const int kofs = kk + 8 * (lane >> 4);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(&As[(wm * 64 + 16 * i + (lane & 15)) * kLds + kofs]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(&Bs[(wn * 64 + 16 * j + (lane & 15)) * kLds + kofs]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // D of a 16x16 tile: lane holds rows 4*(lane/16) + e, column lane % 16.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t gm = m0 + wm * 64 + 16 * i + 4 * (lane >> 4) + e;
        const int64_t gn = n0 + wn * 64 + 16 * j + (lane & 15);
        if (gm < M && gn < R) out[gm * R + gn] = f32_to_bf16_bits(acc[i][j][e]);
      }
}

}  // namespace

hipError_t launch_prefill_fused(const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                                uint16_t* out, int64_t R, int64_t C, int64_t M, int k,
                                hipStream_t stream) {
  const dim3 grid((unsigned)((R + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM)), block(256);
  switch (k) {
    case 2: hipLaunchKernelGGL(prefill_fused_kernel<2>, grid, block, 0, stream, codes, scales, x, out, R, C, M); break;
    case 3: hipLaunchKernelGGL(prefill_fused_kernel<3>, grid, block, 0, stream, codes, scales, x, out, R, C, M); break;
    case 4: hipLaunchKernelGGL(prefill_fused_kernel<4>, grid, block, 0, stream, codes, scales, x, out, R, C, M); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace trellis
