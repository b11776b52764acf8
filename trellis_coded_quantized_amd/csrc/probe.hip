// probe.hip -- the register-only decode probe: the decode of the matvec
// loop (window extract, 1MAD multiply-add, byte sums to f16 integer codes)
// and its four MFMAs per 32-weight run, with no memory traffic, to measure
// the rate at which the decode alone can run on the chip (the ALU ceiling of
// the matvec kernels).  Decode per page 55 (mlx-bun 0.2.0 -> 0.4.0 diff),
// trellis-linear.ts HEADER helpers trellis_state and trellis_y.
//
// Thread g starts from the K + 1 words runs[g][0 .. K] -- K words of one
// 32-position run and the word after it -- and decodes the run `iters`
// times, adding 1 to every word after each pass.  Each decoded run feeds
// four v_mfma_f32_16x16x32_f16 against an all-ones B operand, so every
// element of a wave's accumulators is a sum of codes; the wave writes the
// sum of all its accumulator elements, which equals 16 times the sum of the
// codes its 64 lanes decoded (each code is summed once per B column).
#include "internal.hpp"
#include "mfma_common.hpp"

namespace trellis {
namespace {

template <int K>
__global__ __launch_bounds__(kProbeThreads) void decode_only_kernel(const uint32_t* __restrict__ runs,
                                                                    float* __restrict__ wave_sums, int iters) {
  const int g = blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t w[K + 1];
#pragma unroll
  for (int j = 0; j <= K; ++j) w[j] = runs[(int64_t)g * (K + 1) + j];
  const half8 ones = __builtin_bit_cast(half8, u32x4{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u});
  f32x4 acc[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  const uint32_t mul = kMul;
  const uint64_t add64 = kAdd;
  for (int t = 0; t < iters; ++t) {
    u32x4 A[4];
    decode_run_codes<K>(w, mul, add64, A);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, A[u]), ones, acc[u], 0, 0, 0);
#pragma unroll
    for (int j = 0; j <= K; ++j) w[j] += 1u;
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) s += (acc[u][0] + acc[u][1]) + (acc[u][2] + acc[u][3]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if ((threadIdx.x & 63) == 0) wave_sums[g >> 6] = s;
}

}  // namespace

hipError_t launch_decode_only(const uint32_t* runs, float* wave_sums, int blocks, int iters, int k,
                              hipStream_t stream) {
  const dim3 grid((unsigned)blocks), block(kProbeThreads);
  switch (k) {
    case 2: hipLaunchKernelGGL(decode_only_kernel<2>, grid, block, 0, stream, runs, wave_sums, iters); break;
    case 3: hipLaunchKernelGGL(decode_only_kernel<3>, grid, block, 0, stream, runs, wave_sums, iters); break;
    case 4: hipLaunchKernelGGL(decode_only_kernel<4>, grid, block, 0, stream, runs, wave_sums, iters); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace trellis
