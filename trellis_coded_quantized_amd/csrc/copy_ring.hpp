// copy_ring.hpp -- device helpers shared by the kernels that stream packed
// codes HBM -> LDS with global_load_lds and wait for them with explicit
// vmcnt counts: the counted wait, an LDS-only workgroup barrier (no wait on
// copies in flight), and a wave-wide maximum through DPP.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace trellis {

// s_waitcnt vmcnt(n) with expcnt / lgkmcnt left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void waitcnt_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void wait_vmcnt(int n) {   // n is wave-uniform
  switch (n) {
#define TRELLIS_VM(N) \
  case N: waitcnt_vm<N>(); break;
    TRELLIS_VM(0) TRELLIS_VM(1) TRELLIS_VM(2) TRELLIS_VM(3) TRELLIS_VM(4) TRELLIS_VM(5) TRELLIS_VM(6)
    TRELLIS_VM(7) TRELLIS_VM(8) TRELLIS_VM(9) TRELLIS_VM(10) TRELLIS_VM(11) TRELLIS_VM(12) TRELLIS_VM(13)
    TRELLIS_VM(14) TRELLIS_VM(15) TRELLIS_VM(16) TRELLIS_VM(17) TRELLIS_VM(18) TRELLIS_VM(19) TRELLIS_VM(20)
    TRELLIS_VM(21) TRELLIS_VM(22) TRELLIS_VM(23) TRELLIS_VM(24) TRELLIS_VM(25) TRELLIS_VM(26) TRELLIS_VM(27)
    TRELLIS_VM(28) TRELLIS_VM(29) TRELLIS_VM(30) TRELLIS_VM(31) TRELLIS_VM(32) TRELLIS_VM(33) TRELLIS_VM(34)
    TRELLIS_VM(35) TRELLIS_VM(36) TRELLIS_VM(37) TRELLIS_VM(38) TRELLIS_VM(39) TRELLIS_VM(40) TRELLIS_VM(41)
    TRELLIS_VM(42) TRELLIS_VM(43) TRELLIS_VM(44) TRELLIS_VM(45) TRELLIS_VM(46) TRELLIS_VM(47) TRELLIS_VM(48)
    TRELLIS_VM(49) TRELLIS_VM(50) TRELLIS_VM(51) TRELLIS_VM(52) TRELLIS_VM(53) TRELLIS_VM(54) TRELLIS_VM(55)
    TRELLIS_VM(56) TRELLIS_VM(57) TRELLIS_VM(58) TRELLIS_VM(59) TRELLIS_VM(60) TRELLIS_VM(61) TRELLIS_VM(62)
#undef TRELLIS_VM
    default: break;                  // the counter holds at most 63: always satisfied
  }
}

// Workgroup barrier that orders LDS only: it does not wait for copies in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Largest value over the wave (non-negative inputs), through DPP row shifts
// and row broadcasts: prefix maxima within each row of 16, then across rows.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));   // row_shr:1
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));   // row_shr:2
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));   // row_shr:4
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));   // row_shr:8
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));   // row_bcast:15
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));   // row_bcast:31
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

}  // namespace trellis
