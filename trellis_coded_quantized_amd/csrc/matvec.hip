// matvec.hip -- packed trellis matvecs for M <= 4 on gfx950.
//
// axis 1 (and fused gate/up + SwiGLU): one wave64 per output row.  A lane
// owns runs of 32 consecutive block positions; a run's symbols fill exactly
// k words and the windows of its first positions spill into the next word up
// (word index wrapping to 0 at the block end), so each lane loads k + 1 words
// per run and every window is one funnel shift of two registers.  Decoded
// weights are reused across the M vectors; the row's partial sums end in a
// wave reduction.
//   Source: mlx-bun 0.2.0 -> 0.4.0 diff (page 55), trellis-linear.ts REDUCE
//   and GATEUP kernels and their comments; page 56, trellis-shared-m.ts.
//
// axis 0: stored W^T [R_in, C_out].  A thread owns four adjacent output
// columns of one block (one 64-bit circular window covers their four states)
// and a split of the stored rows; per row it scales its four weights by the
// row's scale and FMAs them against the broadcast x[m, r].  Partials
// [S, M, C_out] in f32 are folded by a second kernel.
//   Source: page 55, trellis-linear.ts SCATTER kernel comment and #scatter
//   (split-K partials, one sum, cast); page 56, trellis-vector-expand.ts
//   (four weights from one 64-bit window).
#include "internal.hpp"
#include "trellis_device.hpp"

namespace trellis {
namespace {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// bf16 element e (0..7) of a 16-byte vector of eight bf16 values.
__device__ __forceinline__ float bf16_of(const uint4& v, int e) {
  const uint32_t u = (e >> 1) == 0 ? v.x : (e >> 1) == 1 ? v.y : (e >> 1) == 2 ? v.z : v.w;
  return (e & 1) ? __uint_as_float(u & 0xFFFF0000u) : __uint_as_float(u << 16);
}

template <int K>
__device__ __forceinline__ void load_run(const uint32_t* __restrict__ row, int blk, int q,
                                         uint32_t (&w)[K + 1]) {
  constexpr int WPB = words_per_block(K);
  const uint32_t* bw = row + (int64_t)blk * WPB;
  const int w0 = (7 - q) * K;            // run q covers positions 32q .. 32q+31
#pragma unroll
  for (int i = 0; i < K; ++i) w[i] = bw[w0 + i];
  w[K] = bw[(w0 + K == WPB) ? 0 : w0 + K];
}

template <int K, int M, bool GATEUP>
__global__ __launch_bounds__(256) void axis1_valu_kernel(
    const uint32_t* __restrict__ codes0, const uint16_t* __restrict__ scales0,
    const uint32_t* __restrict__ codes1, const uint16_t* __restrict__ scales1,
    const uint16_t* __restrict__ x, void* __restrict__ out, int out_f32,
    float* __restrict__ gate_f32, float* __restrict__ up_f32, int64_t R, int64_t C) {
  constexpr int WPB = words_per_block(K);
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= R) return;
  const int64_t row_words = (C / kT) * WPB;
  const uint32_t* crow0 = codes0 + row * row_words;
  const uint32_t* crow1 = GATEUP ? codes1 + row * row_words : nullptr;
  const float sc0 = half_bits_to_f32(scales0[row]);
  const float sc1 = GATEUP ? half_bits_to_f32(scales1[row]) : 0.0f;

  float a0[M][2], a1[M][2];
#pragma unroll
  for (int m = 0; m < M; ++m) a0[m][0] = a0[m][1] = a1[m][0] = a1[m][1] = 0.0f;

  const int nruns = (int)(C / 32);
  for (int run = lane; run < nruns; run += 64) {
    const int blk = run >> 3, q = run & 7;
    uint32_t w0[K + 1], w1[K + 1];
    load_run<K>(crow0, blk, q, w0);
    if constexpr (GATEUP) load_run<K>(crow1, blk, q, w1);
    const int64_t c0 = (int64_t)blk * kT + q * 32;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 xv[M];
#pragma unroll
      for (int m = 0; m < M; ++m)
        xv[m] = *reinterpret_cast<const uint4*>(x + (int64_t)m * C + c0 + 8 * j);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int i = 8 * j + e;                 // position c0 + i
        const int pl = (31 - i) * K;             // its window's first bit in w[]
        const int wi = pl >> 5, off = pl & 31;
        const float v0 = code_value(code_y(window(w0[wi], w0[wi + 1], off))) * sc0;
        float v1 = 0.0f;
        if constexpr (GATEUP) v1 = code_value(code_y(window(w1[wi], w1[wi + 1], off))) * sc1;
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const float xf = bf16_of(xv[m], e);
          a0[m][e & 1] = __builtin_fmaf(v0, xf, a0[m][e & 1]);
          if constexpr (GATEUP) a1[m][e & 1] = __builtin_fmaf(v1, xf, a1[m][e & 1]);
        }
      }
    }
  }

#pragma unroll
  for (int m = 0; m < M; ++m) {
    const float g = wave_sum(a0[m][0] + a0[m][1]);
    if constexpr (GATEUP) {
      const float u = wave_sum(a1[m][0] + a1[m][1]);
      if (lane == 0) {
        const int64_t o = (int64_t)m * R + row;
        if (gate_f32) gate_f32[o] = g;
        if (up_f32) up_f32[o] = u;
        const float gT = round_bf16(g);
        const float uT = round_bf16(u);
        const float sig = round_bf16(1.0f / (1.0f + expf(-gT)));
        const float silu = round_bf16(gT * sig);
        reinterpret_cast<uint16_t*>(out)[o] = f32_to_bf16_bits(silu * uT);
      }
    } else if (lane == 0) {
      const int64_t o = (int64_t)m * R + row;
      if (out_f32) reinterpret_cast<float*>(out)[o] = g;
      else reinterpret_cast<uint16_t*>(out)[o] = f32_to_bf16_bits(g);
    }
  }
}

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
hipError_t axis1_dispatch_m(const uint32_t* c0, const uint16_t* s0, const uint32_t* c1,
                            const uint16_t* s1, const uint16_t* x, void* out, int out_f32,
                            float* gf, float* uf, int64_t R, int64_t C, int M,
                            hipStream_t stream) {
  const dim3 grid((unsigned)((R + 3) / 4)), block(256);
  const bool gu = c1 != nullptr;
#define TRELLIS_AXIS1_CASE(MM)                                                                   \
  case MM:                                                                                        \
    if (gu)                                                                                       \
      hipLaunchKernelGGL((axis1_valu_kernel<K, MM, true>), grid, block, 0, stream, c0, s0, c1, s1, \
                         x, out, out_f32, gf, uf, R, C);                                          \
    else                                                                                          \
      hipLaunchKernelGGL((axis1_valu_kernel<K, MM, false>), grid, block, 0, stream, c0, s0, c1,    \
                         s1, x, out, out_f32, gf, uf, R, C);                                      \
    break;
  switch (M) {
    TRELLIS_AXIS1_CASE(1)
    TRELLIS_AXIS1_CASE(2)
    TRELLIS_AXIS1_CASE(3)
    TRELLIS_AXIS1_CASE(4)
    default: return hipErrorInvalidValue;
  }
#undef TRELLIS_AXIS1_CASE
  return hipGetLastError();
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

size_t axis1_workspace_bytes(int64_t, int64_t, int, int) { return 0; }

hipError_t launch_axis1(const uint32_t* codes0, const uint16_t* scales0, const uint32_t* codes1,
                        const uint16_t* scales1, const uint16_t* x, void* out, int out_f32,
                        float* gate_f32, float* up_f32, int64_t R, int64_t C, int M, int k,
                        void*, hipStream_t stream) {
  switch (k) {
    case 2: return axis1_dispatch_m<2>(codes0, scales0, codes1, scales1, x, out, out_f32, gate_f32, up_f32, R, C, M, stream);
    case 3: return axis1_dispatch_m<3>(codes0, scales0, codes1, scales1, x, out, out_f32, gate_f32, up_f32, R, C, M, stream);
    case 4: return axis1_dispatch_m<4>(codes0, scales0, codes1, scales1, x, out, out_f32, gate_f32, up_f32, R, C, M, stream);
    default: return hipErrorInvalidValue;
  }
}

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
