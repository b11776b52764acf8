// internal.hpp -- host-side launchers shared between the C-ABI layer
// (api.hip) and the kernel translation units.  Every launcher assumes the
// caller already validated geometry, pointers and workspace size.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace trellis {

// axis 1 (gate/up when codes1 != nullptr).  The persistent kernel keeps a
// ring of 16-row code tiles in LDS and x in registers; axis1_supported says
// whether a shape fits (LDS and register budget), checked on the host.
// Rows wider than 5120 columns run as column chunks into f32 partials in the
// workspace (axis1_workspace_bytes), folded by a second kernel.
constexpr size_t kAxis1MaxLdsBytes = 160 * 1024;
bool axis1_supported(int64_t R, int64_t C, int M, int k, bool gateup);
// grouped plain axis-1 call: n <= axis1_max_group() matrices of the same C
// and k over the same x, one launch (the row groups of all of them)
int axis1_max_group();
bool axis1_group_supported(const int64_t* R, int n, int64_t C, int M, int k);
hipError_t launch_axis1_group(const uint32_t* const* codes, const uint16_t* const* scales, void* const* outs,
                              const int64_t* R, int n, const uint16_t* x, int out_f32, int64_t C, int M, int k,
                              hipStream_t stream);
size_t axis1_workspace_bytes(int64_t R, int64_t C, int M, int k, bool gateup);
hipError_t launch_axis1(const uint32_t* codes0, const uint16_t* scales0, const uint32_t* codes1,
                        const uint16_t* scales1, const uint16_t* x, void* out, int out_f32,
                        float* gate_f32, float* up_f32, int64_t R, int64_t C, int M, int k,
                        void* workspace, hipStream_t stream);

// measurement probes: the gate/up kernel without the decode (timing floor,
// one launch, C <= 5120), and the register-only decode of `iters` runs per
// thread (the instruction mix of the matvec loop without memory)
hipError_t launch_gateup_decode_free(const uint32_t* c0, const uint16_t* s0, const uint32_t* c1, const uint16_t* s1,
                                     const uint16_t* x, uint16_t* out, int64_t R, int64_t C, int M, int k,
                                     hipStream_t stream);
constexpr int kProbeThreads = 512;
hipError_t launch_decode_only(const uint32_t* runs, float* wave_sums, int blocks, int iters, int k,
                              hipStream_t stream);

// axis 0 (split-K over stored rows, MFMA on 32-row blocks, then a fold)
bool axis0_supported(int64_t R, int64_t C, int M, int k);
size_t axis0_workspace_bytes(int64_t R, int64_t C, int M, int k);
// The static device scratch that stands in for the axis-0 workspace in the
// allocation-free call: kAxis0ScratchBytes per device, its address resolved
// once per device (the current one) and cached.
constexpr size_t kAxis0ScratchBytes = (size_t)4 << 20;
constexpr int kMaxDevices = 64;
hipError_t axis0_scratch(void** ptr);
// interleave: codes in the block-interleaved k = 3 layout [C/512, R, 48]
hipError_t launch_axis0(const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                        void* out, int out_f32, int64_t R, int64_t C, int M, int k,
                        void* workspace, hipStream_t stream, int interleave = 0);

// expansion and decode export
hipError_t launch_expand(const uint32_t* codes, const uint16_t* scales, uint16_t* out, int64_t R,
                         int64_t C, int k, hipStream_t stream, int interleave = 0);
hipError_t launch_decode_states(const uint32_t* codes, int64_t R, int64_t C, int k,
                                uint16_t* states, int16_t* y, float* value, hipStream_t stream);

// compute units of the current device (cached per device)
int device_cus();

// fused prefill (32-bit buffer offsets: x and the codes each below 2 GiB);
// the workspace holds x in operand order and the f32 partial tiles of the
// tiles split along the contraction.  R is the output count, C the
// contraction length: axis 1 codes [R, C k / 32]; axis0 != 0: codes
// [C, R k / 32] (the stored transpose), scales [C].
bool prefill_fused_supported(int64_t R, int64_t C, int64_t M, int k);
size_t prefill_fused_workspace_bytes(int64_t R, int64_t C, int64_t M, int axis0 = 0);
// interleave (axis 0, k = 3, R % 512 == 0): codes in the block-interleaved
// layout [R/512, C, 48].
hipError_t launch_prefill_fused(const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                                uint16_t* out, int64_t R, int64_t C, int64_t M, int k,
                                void* workspace, hipStream_t stream, int axis0 = 0, int interleave = 0);

}  // namespace trellis
