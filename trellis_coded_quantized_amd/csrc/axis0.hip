// axis0.hip -- axis-0 (down projection) matvec for M <= 4 on gfx950.
//
// The stored matrix is W^T [R_in, C_out], coded along C_out.  A thread owns
// four adjacent output columns of one block (one 64-bit circular window
// covers their four states) and a split of the stored rows; per row it scales
// its four weights by the row's scale and FMAs them against the broadcast
// x[m, r].  Partials [S, M, C_out] in f32 are folded by a second kernel.
// Source: mlx-bun 0.2.0 -> 0.4.0 diff (page 55), trellis-linear.ts SCATTER
// kernel comment and #scatter (split-K partials, one sum, cast); page 56,
// trellis-vector-expand.ts (four weights from one 64-bit window).
#include "internal.hpp"
#include "trellis_device.hpp"

namespace trellis {
namespace {

template <int K, int M>
__global__ __launch_bounds__(256) void axis0_partial_kernel(
    const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ x, float* __restrict__ partial, int64_t R, int64_t C,
    int64_t rows_per_split) {
  constexpr int WPB = words_per_block(K);
  const int64_t c0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (c0 >= C) return;
  const int split = blockIdx.y;
  const int blk = (int)(c0 / kT), t0 = (int)(c0 % kT);
  const int pos = (kT - 1 - (t0 + 3)) * K;     // window start of the last of the four
  const int wi = pos >> 5, off = pos & 31;
  const int wn = (wi + 1 == WPB) ? 0 : wi + 1;
  const int64_t row_words = (C / kT) * WPB;
  const uint32_t* base = codes + (int64_t)blk * WPB;
  const int64_t r0 = split * rows_per_split;
  const int64_t r1 = (r0 + rows_per_split < R) ? r0 + rows_per_split : R;

  float acc[4][M];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int m = 0; m < M; ++m) acc[i][m] = 0.0f;

  for (int64_t r = r0; r < r1; ++r) {
    const uint32_t* bw = base + r * row_words;
    const uint64_t win = ((uint64_t)bw[wn] << 32 | bw[wi]) >> off;
    const float sc = half_bits_to_f32(scales[r]);
    float xr[M];
#pragma unroll
    for (int m = 0; m < M; ++m) xr[m] = bf16_bits_to_f32(x[(int64_t)m * R + r]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t s = (uint32_t)(win >> ((3 - i) * K)) & kStateMask;
      const float w = code_value(code_y(s)) * sc;
#pragma unroll
      for (int m = 0; m < M; ++m) acc[i][m] = __builtin_fmaf(w, xr[m], acc[i][m]);
    }
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float4 v = make_float4(acc[0][m], acc[1][m], acc[2][m], acc[3][m]);
    *reinterpret_cast<float4*>(partial + ((int64_t)split * M + m) * C + c0) = v;
  }
}

__global__ __launch_bounds__(256) void axis0_fold_kernel(const float* __restrict__ partial,
                                                         void* __restrict__ out, int out_f32,
                                                         int M, int64_t C, int S) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // over M * C
  if (i >= (int64_t)M * C) return;
  const int64_t m = i / C, c = i % C;
  float s = 0.0f;
  for (int j = 0; j < S; ++j) s += partial[((int64_t)j * M + m) * C + c];
  if (out_f32) reinterpret_cast<float*>(out)[i] = s;
  else reinterpret_cast<uint16_t*>(out)[i] = f32_to_bf16_bits(s);
}

int axis0_splits(int64_t R) {
  int64_t s = R / 64;
  if (s < 1) s = 1;
  if (s > 128) s = 128;
  return (int)s;
}

template <int K>
hipError_t axis0_dispatch_m(const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                            float* partial, int64_t R, int64_t C, int M, int S,
                            hipStream_t stream) {
  const int64_t rows_per_split = (R + S - 1) / S;
  const dim3 grid((unsigned)((C / 4 + 255) / 256), (unsigned)S), block(256);
#define TRELLIS_AXIS0_CASE(MM)                                                                 \
  case MM:                                                                                      \
    hipLaunchKernelGGL((axis0_partial_kernel<K, MM>), grid, block, 0, stream, codes, scales, x, \
                       partial, R, C, rows_per_split);                                          \
    break;
  switch (M) {
    TRELLIS_AXIS0_CASE(1)
    TRELLIS_AXIS0_CASE(2)
    TRELLIS_AXIS0_CASE(3)
    TRELLIS_AXIS0_CASE(4)
    default: return hipErrorInvalidValue;
  }
#undef TRELLIS_AXIS0_CASE
  return hipGetLastError();
}

}  // namespace

size_t axis0_workspace_bytes(int64_t R, int64_t C, int M, int) {
  return (size_t)axis0_splits(R) * (size_t)M * (size_t)C * sizeof(float);
}

hipError_t launch_axis0(const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                        void* out, int out_f32, int64_t R, int64_t C, int M, int k,
                        void* workspace, hipStream_t stream) {
  const int S = axis0_splits(R);
  float* partial = reinterpret_cast<float*>(workspace);
  hipError_t e;
  switch (k) {
    case 2: e = axis0_dispatch_m<2>(codes, scales, x, partial, R, C, M, S, stream); break;
    case 3: e = axis0_dispatch_m<3>(codes, scales, x, partial, R, C, M, S, stream); break;
    case 4: e = axis0_dispatch_m<4>(codes, scales, x, partial, R, C, M, S, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)M * C;
  hipLaunchKernelGGL(axis0_fold_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     partial, out, out_f32, M, C, S);
  return hipGetLastError();
}

}  // namespace trellis
