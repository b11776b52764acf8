// axis1.hip -- launchers of the axis-1 matvec and the fused gate/up + SwiGLU
// for M <= 4 on gfx950 (the kernel body and its geometry are in
// axis1_kernel.hpp), and the fold of column chunks for rows wider than 5120.
#include "axis1_kernel.hpp"

namespace trellis {
namespace {

template <int K, bool GATEUP, int NG, bool GROUP = false, bool DECODE = true>
__global__ __launch_bounds__(kThreads) void axis1_kernel(
    const uint32_t* __restrict__ codes0, const uint16_t* __restrict__ scales0,
    const uint32_t* __restrict__ codes1, const uint16_t* __restrict__ scales1,
    const uint16_t* __restrict__ x, void* __restrict__ out, int out_f32,
    float* __restrict__ gate_f32, float* __restrict__ up_f32, const Axis1Geom g) {
  axis1_body<K, GATEUP, NG, GROUP, DECODE>(codes0, scales0, codes1, scales1, x, out, out_f32, gate_f32, up_f32, g,
                                          (int)blockIdx.x, (int)gridDim.x);
}

// Sum of the column chunks' f32 partial outputs ([n][M * R], or [n][2][M *
// R] gate and up for GATEUP), in chunk order, then the output cast or the
// SwiGLU chain.
template <bool GATEUP>
__global__ __launch_bounds__(256) void axis1_chunk_fold_kernel(const float* __restrict__ part, int n, int64_t MR,
                                                               void* __restrict__ out, int out_f32,
                                                               float* __restrict__ gate_f32,
                                                               float* __restrict__ up_f32) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= MR) return;
  const int64_t stride = GATEUP ? 2 * MR : MR;
  float v0 = 0.f, v1 = 0.f;
  for (int j = 0; j < n; ++j) {
    v0 += part[j * stride + i];
    if constexpr (GATEUP) v1 += part[j * stride + MR + i];
  }
  if constexpr (GATEUP) {
    if (gate_f32) gate_f32[i] = v0;
    if (up_f32) up_f32[i] = v1;
    reinterpret_cast<uint16_t*>(out)[i] = swiglu_bf16(v0, v1);
  } else if (out_f32) {
    reinterpret_cast<float*>(out)[i] = v0;
  } else {
    reinterpret_cast<uint16_t*>(out)[i] = f32_to_bf16_bits(v0);
  }
}

template <int K, bool GU, int NG, bool GROUP = false, bool DECODE = true>
hipError_t axis1_launch_one(const uint32_t* c0, const uint16_t* s0, const uint32_t* c1,
                            const uint16_t* s1, const uint16_t* x, void* out, int out_f32,
                            float* gf, float* uf, const Axis1Geom& g, int64_t grid, hipStream_t stream) {
  static uint64_t lds_attr = 0;                // devices whose dynamic LDS limit is raised
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(lds_attr & bit)) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&axis1_kernel<K, GU, NG, GROUP, DECODE>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kAxis1MaxLdsBytes);
    if (e != hipSuccess) return e;
    lds_attr |= bit;
  }
  hipLaunchKernelGGL((axis1_kernel<K, GU, NG, GROUP, DECODE>), dim3((unsigned)grid), dim3(kThreads), g.total,
                     stream, c0, s0, c1, s1, x, out, out_f32, gf, uf, g);
  return hipGetLastError();
}

template <int K, int NG>
hipError_t axis1_dispatch_gu(const uint32_t* c0, const uint16_t* s0, const uint32_t* c1,
                             const uint16_t* s1, const uint16_t* x, void* out, int out_f32, float* gf,
                             float* uf, const Axis1Geom& g, int64_t grid, hipStream_t stream) {
  return c1 ? axis1_launch_one<K, true, NG>(c0, s0, c1, s1, x, out, out_f32, gf, uf, g, grid, stream)
            : axis1_launch_one<K, false, NG>(c0, s0, c1, s1, x, out, out_f32, gf, uf, g, grid, stream);
}

template <int K>
hipError_t axis1_launch_geom(const uint32_t* c0, const uint16_t* s0, const uint32_t* c1, const uint16_t* s1,
                             const uint16_t* x, void* out, int out_f32, float* gf, float* uf, const Axis1Geom& g,
                             int64_t grid, hipStream_t stream) {
  switch (axis1_ng(g.C)) {
    case 2: return axis1_dispatch_gu<K, 2>(c0, s0, c1, s1, x, out, out_f32, gf, uf, g, grid, stream);
    case 5: return axis1_dispatch_gu<K, 5>(c0, s0, c1, s1, x, out, out_f32, gf, uf, g, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int K>
hipError_t axis1_main(const uint32_t* c0, const uint16_t* s0, const uint32_t* c1,
                      const uint16_t* s1, const uint16_t* x, void* out, int out_f32, float* gf,
                      float* uf, int64_t R, int64_t C, int M, void* workspace, hipStream_t stream) {
  const bool gu = c1 != nullptr;
  const int64_t grid = axis1_grid(R, gu);
  const int64_t nch = axis1_nchunks(C);
  if (nch == 1) {
    Axis1Geom g;
    if (!axis1_geom(R, C, M, K, gu, grid, g)) return hipErrorInvalidValue;
    return axis1_launch_geom<K>(c0, s0, c1, s1, x, out, out_f32, gf, uf, g, grid, stream);
  }
  // column chunks into f32 partials [chunk][gate/up][M][R], then the fold
  if (!workspace) return hipErrorInvalidValue;
  float* part = reinterpret_cast<float*>(workspace);
  const int64_t MR = (int64_t)M * R, nb = C / 256, per_chunk = (gu ? 2 : 1) * MR;
  constexpr int WPB = words_per_block(K);
  for (int64_t j = 0; j < nch; ++j) {
    const int64_t b0 = axis1_chunk_first(nb, nch, j), b1 = axis1_chunk_first(nb, nch, j + 1);
    Axis1Geom g;
    if (!axis1_geom(R, (b1 - b0) * 256, M, K, gu, grid, g)) return hipErrorInvalidValue;
    g.ldx = C;
    g.row_bytes = C * K / 8;
    float* pj = part + j * per_chunk;
    const uint32_t* cc0 = c0 + b0 * WPB;
    const uint32_t* cc1 = gu ? c1 + b0 * WPB : nullptr;
    const uint16_t* xc = x + b0 * 256;
    const hipError_t e = gu ? axis1_launch_geom<K>(cc0, s0, cc1, s1, xc, nullptr, 0, pj, pj + MR, g, grid, stream)
                            : axis1_launch_geom<K>(cc0, s0, nullptr, nullptr, xc, pj, 1, nullptr, nullptr, g, grid,
                                                   stream);
    if (e != hipSuccess) return e;
  }
  const unsigned blocks = (unsigned)((MR + 255) / 256);
  if (gu)
    hipLaunchKernelGGL(axis1_chunk_fold_kernel<true>, dim3(blocks), dim3(256), 0, stream, part, (int)nch, MR, out,
                       0, gf, uf);
  else
    hipLaunchKernelGGL(axis1_chunk_fold_kernel<false>, dim3(blocks), dim3(256), 0, stream, part, (int)nch, MR, out,
                       out_f32, nullptr, nullptr);
  return hipGetLastError();
}

template <int K>
hipError_t axis1_group_main(const uint32_t* const* codes, const uint16_t* const* scales, void* const* outs,
                            const int64_t* R, int n, const uint16_t* x, int out_f32, int64_t C, int M,
                            hipStream_t stream) {
  int64_t nrg = 0;
  for (int j = 0; j < n; ++j) nrg += (R[j] + 15) / 16;
  const int64_t grid = axis1_grid(R[0], false, nrg);
  Axis1Geom g;
  if (!axis1_geom(R[0], C, M, K, false, grid, g, nrg)) return hipErrorInvalidValue;
  g.ngroup = n;
  int64_t end = 0;
  for (int j = 0; j < n; ++j) {
    end += (R[j] + 15) / 16;
    g.gend[j] = end;
    g.gR[j] = R[j];
    g.gcodes[j] = codes[j];
    g.gscales[j] = scales[j];
    g.gout[j] = outs[j];
  }
  switch (axis1_ng(C)) {
    case 2:
      return axis1_launch_one<K, false, 2, true>(codes[0], scales[0], nullptr, nullptr, x, outs[0], out_f32,
                                                 nullptr, nullptr, g, grid, stream);
    case 5:
      return axis1_launch_one<K, false, 5, true>(codes[0], scales[0], nullptr, nullptr, x, outs[0], out_f32,
                                                 nullptr, nullptr, g, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int K>
hipError_t axis1_decode_free_main(const uint32_t* c0, const uint16_t* s0, const uint32_t* c1, const uint16_t* s1,
                                  const uint16_t* x, uint16_t* out, int64_t R, int64_t C, int M, hipStream_t stream) {
  const int64_t grid = axis1_grid(R, true);
  Axis1Geom g;
  if (!axis1_geom(R, C, M, K, true, grid, g)) return hipErrorInvalidValue;
  switch (axis1_ng(C)) {
    case 2:
      return axis1_launch_one<K, true, 2, false, false>(c0, s0, c1, s1, x, out, 0, nullptr, nullptr, g, grid,
                                                        stream);
    case 5:
      return axis1_launch_one<K, true, 5, false, false>(c0, s0, c1, s1, x, out, 0, nullptr, nullptr, g, grid,
                                                        stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gateup_decode_free(const uint32_t* c0, const uint16_t* s0, const uint32_t* c1, const uint16_t* s1,
                                     const uint16_t* x, uint16_t* out, int64_t R, int64_t C, int M, int k,
                                     hipStream_t stream) {
  switch (k) {
    case 2: return axis1_decode_free_main<2>(c0, s0, c1, s1, x, out, R, C, M, stream);
    case 3: return axis1_decode_free_main<3>(c0, s0, c1, s1, x, out, R, C, M, stream);
    case 4: return axis1_decode_free_main<4>(c0, s0, c1, s1, x, out, R, C, M, stream);
    default: return hipErrorInvalidValue;
  }
}

size_t axis1_workspace_bytes(int64_t R, int64_t C, int M, int, bool gateup) {
  const int64_t n = axis1_nchunks(C);
  return n == 1 ? 0 : (size_t)n * (gateup ? 2 : 1) * (size_t)M * (size_t)R * sizeof(float);
}

int axis1_max_group() { return kMaxGroup; }

bool axis1_group_supported(const int64_t* R, int n, int64_t C, int M, int k) {
  if (n < 1 || n > kMaxGroup) return false;
  int64_t nrg = 0;
  for (int j = 0; j < n; ++j) nrg += (R[j] + 15) / 16;
  Axis1Geom g;
  return axis1_geom(R[0], C, M, k, false, axis1_grid(R[0], false, nrg), g, nrg);
}

hipError_t launch_axis1_group(const uint32_t* const* codes, const uint16_t* const* scales, void* const* outs,
                              const int64_t* R, int n, const uint16_t* x, int out_f32, int64_t C, int M, int k,
                              hipStream_t stream) {
  if (n < 1 || n > kMaxGroup) return hipErrorInvalidValue;
  switch (k) {
    case 2: return axis1_group_main<2>(codes, scales, outs, R, n, x, out_f32, C, M, stream);
    case 3: return axis1_group_main<3>(codes, scales, outs, R, n, x, out_f32, C, M, stream);
    case 4: return axis1_group_main<4>(codes, scales, outs, R, n, x, out_f32, C, M, stream);
    default: return hipErrorInvalidValue;
  }
}

bool axis1_supported(int64_t R, int64_t C, int M, int k, bool gateup) {
  if (C % 256 != 0 || C < 256) return false;
  const int64_t nb = C / 256, n = axis1_nchunks(C);
  for (int64_t j = 0; j < n; ++j) {            // every chunk's geometry fits
    const int64_t w = (axis1_chunk_first(nb, n, j + 1) - axis1_chunk_first(nb, n, j)) * 256;
    Axis1Geom g;
    if (!axis1_geom(R, w, M, k, gateup, axis1_grid(R, gateup), g)) return false;
    if (n == 1) break;
  }
  return true;
}

hipError_t launch_axis1(const uint32_t* codes0, const uint16_t* scales0, const uint32_t* codes1,
                        const uint16_t* scales1, const uint16_t* x, void* out, int out_f32,
                        float* gate_f32, float* up_f32, int64_t R, int64_t C, int M, int k,
                        void* workspace, hipStream_t stream) {
  switch (k) {
    case 2:
      return axis1_main<2>(codes0, scales0, codes1, scales1, x, out, out_f32, gate_f32, up_f32, R, C, M, workspace,
                           stream);
    case 3:
      return axis1_main<3>(codes0, scales0, codes1, scales1, x, out, out_f32, gate_f32, up_f32, R, C, M, workspace,
                           stream);
    case 4:
      return axis1_main<4>(codes0, scales0, codes1, scales1, x, out, out_f32, gate_f32, up_f32, R, C, M, workspace,
                           stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace trellis
