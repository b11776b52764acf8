// axis0.hip -- launchers of the axis-0 (down projection) matvec for M <= 4
// on gfx950 (the kernel body and its geometry are in axis0_kernel.hpp), the
// fold of its split partials, and the static scratch of the allocation-free
// call.
#include <mutex>

#include "axis0_kernel.hpp"

namespace trellis {
namespace {

template <int K>
__global__ __launch_bounds__(kThreads) void axis0_kernel(const uint32_t* __restrict__ codes,
                                                         const uint16_t* __restrict__ scales,
                                                         const uint16_t* __restrict__ x,
                                                         float* __restrict__ partial, const Axis0Geom g) {
  axis0_body<K>(codes, scales, x, partial, g, (int)blockIdx.x);
}

// The splits' partials [S][M][C] added in split order, one output per
// thread, one wave per 64 outputs.  The fold is one memory round trip, and
// single-wave workgroups spread its loads over more CUs than 256-thread
// ones would, which shortens it.
__global__ __launch_bounds__(64) void axis0_fold_kernel(const float* __restrict__ partial,
                                                         void* __restrict__ out, int out_f32,
                                                         int M, int64_t C, int S) {
  const int64_t i = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (i >= (int64_t)M * C) return;
  const int64_t stride = (int64_t)M * C;
  float a = 0.f;
  for (int j0 = 0; j0 < S; j0 += 16) {         // up to sixteen splits' loads in flight at once
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = (j0 + u < S) ? partial[(j0 + u) * stride + i] : 0.f;
#pragma unroll
    for (int u = 0; u < 16; ++u) a += v[u];
  }
  if (out_f32) reinterpret_cast<float*>(out)[i] = a;
  else reinterpret_cast<uint16_t*>(out)[i] = f32_to_bf16_bits(a);
}


template <int K>
hipError_t axis0_launch(const uint32_t* codes, const uint16_t* scales, const uint16_t* x, float* partial,
                        const Axis0Geom& g, hipStream_t stream) {
  static uint64_t lds_attr = 0;                // devices whose dynamic LDS limit is raised
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(lds_attr & bit)) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&axis0_kernel<K>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBudget);
    if (e != hipSuccess) return e;
    lds_attr |= bit;
  }
  const int units = ((g.ncg + 3) / 4) * g.S;
  const unsigned grid = (unsigned)(4 * kXcds * ((units + kXcds - 1) / kXcds));
  hipLaunchKernelGGL((axis0_kernel<K>), dim3(grid), dim3(kThreads), g.total, stream, codes, scales, x,
                     partial, g);
  return hipGetLastError();
}

// Static scratch of the allocation-free axis-0 call: the split-K partials
// live here instead of in a caller's workspace.  Each device holds its own
// copy of the array until the process ends; host code reaches it only
// through the per-device address from hipGetSymbolAddress (the name itself
// is a host-side stand-in, not a device address).
static __device__ __align__(256) uint8_t scratch[kAxis0ScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t axis0_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {                  // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

bool axis0_supported(int64_t R, int64_t C, int M, int k) {
  Axis0Geom g;
  return axis0_geom(R, C, M, k, g);
}

size_t axis0_workspace_bytes(int64_t R, int64_t C, int M, int k) {
  Axis0Geom g;
  if (!axis0_geom(R, C, M, k, g)) return 0;
  return (size_t)g.S * (size_t)M * (size_t)C * sizeof(float);
}

hipError_t launch_axis0(const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                        void* out, int out_f32, int64_t R, int64_t C, int M, int k,
                        void* workspace, hipStream_t stream, int interleave) {
  Axis0Geom g;
  if (!axis0_geom(R, C, M, k, g)) return hipErrorInvalidValue;
  if (interleave) {
    if (C % 512 != 0) return hipErrorInvalidValue;
    g.interleave = 1;
    g.row_bytes = 2 * (256 * k / 8);
  }
  g.scales16 = reinterpret_cast<uintptr_t>(scales) % 16 == 0;
  g.x16 = reinterpret_cast<uintptr_t>(x) % 16 == 0 && R % 8 == 0;
  float* partial = reinterpret_cast<float*>(workspace);
  hipError_t e;
  switch (k) {
    case 2: e = axis0_launch<2>(codes, scales, x, partial, g, stream); break;
    case 3: e = axis0_launch<3>(codes, scales, x, partial, g, stream); break;
    case 4: e = axis0_launch<4>(codes, scales, x, partial, g, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  const int64_t nout = (int64_t)M * C;          // a multiple of 64 (C is a multiple of 256)
  hipLaunchKernelGGL(axis0_fold_kernel, dim3((unsigned)((nout + 63) / 64)), dim3(64), 0, stream,
                     partial, out, out_f32, M, C, g.S);
  return hipGetLastError();
}

}  // namespace trellis
