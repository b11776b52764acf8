// copy_ring.hpp -- device helpers shared by the kernels that stream packed
// codes HBM -> LDS with global_load_lds and wait for them with explicit
// vmcnt counts: the counted wait, LDS reads and writes that do not wait for
// copies in flight, an LDS-only workgroup barrier, and a wave-wide maximum
// through DPP.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace trellis {

// Word 3 of a raw buffer resource (32-bit data format, no swizzle): the
// copies address a tile through such a resource, with its size in bytes as
// the record count, so reads past it return zeros.
constexpr int kRawBufferWord3 = 0x00020000;

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

// ---- LDS next to copies in flight.  After a global_load_lds the compiler
// treats every later LDS access as one that may touch that copy's target and
// waits for all copies in flight (vmcnt(0)) before it, which would void a
// ring's prefetch.  LDS that copies can reach is therefore read and written
// through the inline-asm blocks below.  A read block issues its reads and
// waits for them (lgkmcnt(0)) inside the block, so no output register is
// live before its data has arrived.  The order against the copies is the
// kernel's own vmcnt wait; LDS operations of one wave complete in issue order.
typedef uint32_t lds_u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t lds_u32x4 __attribute__((ext_vector_type(4)));

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

__device__ __forceinline__ void lds_write_b128(uint32_t a, lds_u32x4 v) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(a), "v"(v) : "memory");
}

__device__ __forceinline__ void lds_write_b32(uint32_t a, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" : : "v"(a), "v"(v) : "memory");
}

__device__ __forceinline__ uint32_t lds_read_b32(uint32_t a) {
  uint32_t r;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r) : "v"(a) : "memory");
  return r;
}

__device__ __forceinline__ lds_u32x4 lds_read_b128(uint32_t a) {
  lds_u32x4 r;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(r) : "v"(a) : "memory");
  return r;
}

// four consecutive 16-byte reads at a
__device__ __forceinline__ void lds_read_b128x4(uint32_t a, lds_u32x4 (&o)[4]) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:16\n\t"
      "ds_read_b128 %2, %4 offset:32\n\t"
      "ds_read_b128 %3, %4 offset:48\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
      : "v"(a)
      : "memory");
}

// four consecutive 16-byte reads at each of N addresses (N = 2 or 5), one wait
template <int N>
__device__ __forceinline__ void lds_read_b128x4n(const uint32_t (&a)[N], lds_u32x4 (&o)[N][4]) {
  static_assert(N == 2 || N == 5, "two or five groups");
  if constexpr (N == 2) {
    asm volatile(
        "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:16\n\t"
        "ds_read_b128 %2, %8 offset:32\n\tds_read_b128 %3, %8 offset:48\n\t"
        "ds_read_b128 %4, %9\n\tds_read_b128 %5, %9 offset:16\n\t"
        "ds_read_b128 %6, %9 offset:32\n\tds_read_b128 %7, %9 offset:48\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0][0]), "=&v"(o[0][1]), "=&v"(o[0][2]), "=&v"(o[0][3]), "=&v"(o[1][0]), "=&v"(o[1][1]),
          "=&v"(o[1][2]), "=&v"(o[1][3])
        : "v"(a[0]), "v"(a[1])
        : "memory");
  } else {
    asm volatile(
        "ds_read_b128 %0, %20\n\tds_read_b128 %1, %20 offset:16\n\t"
        "ds_read_b128 %2, %20 offset:32\n\tds_read_b128 %3, %20 offset:48\n\t"
        "ds_read_b128 %4, %21\n\tds_read_b128 %5, %21 offset:16\n\t"
        "ds_read_b128 %6, %21 offset:32\n\tds_read_b128 %7, %21 offset:48\n\t"
        "ds_read_b128 %8, %22\n\tds_read_b128 %9, %22 offset:16\n\t"
        "ds_read_b128 %10, %22 offset:32\n\tds_read_b128 %11, %22 offset:48\n\t"
        "ds_read_b128 %12, %23\n\tds_read_b128 %13, %23 offset:16\n\t"
        "ds_read_b128 %14, %23 offset:32\n\tds_read_b128 %15, %23 offset:48\n\t"
        "ds_read_b128 %16, %24\n\tds_read_b128 %17, %24 offset:16\n\t"
        "ds_read_b128 %18, %24 offset:32\n\tds_read_b128 %19, %24 offset:48\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0][0]), "=&v"(o[0][1]), "=&v"(o[0][2]), "=&v"(o[0][3]), "=&v"(o[1][0]), "=&v"(o[1][1]),
          "=&v"(o[1][2]), "=&v"(o[1][3]), "=&v"(o[2][0]), "=&v"(o[2][1]), "=&v"(o[2][2]), "=&v"(o[2][3]),
          "=&v"(o[3][0]), "=&v"(o[3][1]), "=&v"(o[3][2]), "=&v"(o[3][3]), "=&v"(o[4][0]), "=&v"(o[4][1]),
          "=&v"(o[4][2]), "=&v"(o[4][3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4])
        : "memory");
  }
}

// five 16-byte reads at independent addresses
__device__ __forceinline__ void lds_read_b128x5(const uint32_t (&a)[5], lds_u32x4 (&o)[5]) {
  asm volatile(
      "ds_read_b128 %0, %5\n\t"
      "ds_read_b128 %1, %6\n\t"
      "ds_read_b128 %2, %7\n\t"
      "ds_read_b128 %3, %8\n\t"
      "ds_read_b128 %4, %9\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4])
      : "memory");
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
