// axis1_kernel.hpp -- device body of the axis-1 matvec and fused gate/up +
// SwiGLU for M <= 4 on gfx950, and its host geometry (the launchers are in
// axis1.hip).
//
// y[m, r] = sum_c w(r, c) x[m, c],  w(r, c) = value(s(r, c)) * scale[r].
// Source: mlx-bun 0.2.0 -> 0.4.0 diff (page 55), trellis-linear.ts REDUCE and
// GATEUP kernels (one pass over x, gate/up never materialised, SwiGLU cast
// chain in the epilogue); page 56, trellis-shared-m.ts (decode once, reuse
// for every vector).
//
// The sum is refactored so the inner product runs on v_mfma_f32_16x16x32_f16
// with exact operands:
//   A (16 rows x 32 k): the code y of each weight as an exact f16 integer:
//     v_sad_hi_u8 / v_sad_u8 write the byte sums b = y + 510 of two 1MAD
//     words into one register as f16 1026 + b, and one packed f16 add of
//     -1536 leaves y (code_pair_y).
//   B (32 k x 16 n): x'[n, c] = f16(x[n, c] * 2^e), e chosen per vector and
//     per column slice so the slice's largest |x| lands in [2^14, 2^15); every
//     bf16 value down to 2^-17 of that maximum is exact in f16.
//   D: f32, D = sum_c y x' (signed products: the accumulator carries no
//     offset, so its rounding is relative to the terms themselves).  Each
//     slice's D is scaled back by 2^-e; the sum over slices times scale / d
//     is the output.
//
// Rows wider than one launch's register-resident x (C > 5120) run as column
// chunks of at most 5120 columns, one launch each, into f32 partial outputs
// in the caller's workspace; axis1_chunk_fold_kernel adds the chunks in
// order and applies the output cast or the SwiGLU chain.  (The pages' REDUCE
// and GATEUP kernels loop over any number of runs per row.)
//
// Schedule: one workgroup of 8 waves per CU walks row groups b, b + grid, ...
// (16 A-rows each: 16 output rows, or 8 gate + 8 up rows sharing B).  Wave w
// owns column slice w (C / 8 columns) for the whole kernel: its B operand
// lives in registers, and it copies only the code blocks of its slice
// (HBM -> its own LDS ring, global_load_lds_dwordx4, explicit vmcnt waits).
// The waves never wait for each other inside the loop: each leaves its
// partial D tile of every row group in LDS, and after one barrier at the end
// all threads add the eight partials in a fixed order and run the epilogue.
#pragma once
#include "copy_ring.hpp"
#include "internal.hpp"
#include "mfma_common.hpp"

namespace trellis {
namespace {
namespace a1 {


constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxSlots = 4;           // tile ring depth per wave
constexpr int kMaxDma = 8;             // copies per wave per tile (C <= 5120, k <= 4: 2 x 8 rows x 25 granules)
// copies per wave per tile for a given k (k = 2: windows of at most four
// 64-byte blocks, 16 rows x 17 granules)
__host__ __device__ constexpr int max_dma(int k) { return k == 2 ? 6 : kMaxDma; }
constexpr int kXPer = 5;               // x granules per lane of a wave's slice (M * C <= 4 * 5120)
constexpr uint32_t kPartBytes = kWaves * 4 * 16 * 4;   // one row group's partial tiles: f32 [wave][n][16 rows]
constexpr int kMaxGroup = 4;           // matrices of one grouped call
constexpr uint32_t kProgBytes = 64;    // row groups each wave has finished: u32 [wave]
constexpr uint32_t kScaleBytes = 32;   // one row group's fp16 scales: 16 rows, or 8 gate then 8 up rows

// Geometry shared by the host (LDS sizing) and the kernel.
struct Axis1Geom {
  // the fields the first copies need come first, so they share the first
  // lines of the kernel argument segment
  int64_t R, row_bytes;
  int64_t ldx;          // elements between rows of x (C, or the full width for a column chunk)
  int M;
  int per;              // runs of 32 columns per wave (C / 256)
  int gsw;              // granules per tile row of a wave's window (its blocks + one pad granule)
  int nwd;              // copy slots per wave per tile (ceil(rows gsw / 64) per matrix)
  uint32_t gsw_magic;   // ceil(2^24 / gsw): p / gsw == (p * gsw_magic) >> 24 for p < 4096
  int nslots, xslots;
  int nfull, nrem;      // row groups per workgroup: nfull, plus one for workgroups b < nrem
  // half = 1: the last nrem row groups run as 2 nrem halves (ROWS / 2 output
  // rows each), one on each workgroup b < 2 nrem, after its nfull whole ones
  int half;
  uint32_t slot_bytes, part_off, prog_off, sc_off, total;
  int nmine_max;
  int64_t C, nrg;
  // Grouped call (plain axis 1 only): ngroup matrices of the same C and k
  // over the same x.  Matrix j owns the launch's row groups [gend[j - 1],
  // gend[j]) (gend[-1] = 0) and has gR[j] rows; matrix 0 is the kernel's
  // codes0 / scales0 / out and R.  ngroup == 1 for every other call.
  int ngroup;
  int64_t gend[kMaxGroup], gR[kMaxGroup];
  const uint32_t* gcodes[kMaxGroup];
  const uint16_t* gscales[kMaxGroup];
  void* gout[kMaxGroup];
};

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Largest |x| bit pattern of each half over the eight bf16 of a granule,
// folded into r (packed unsigned 16-bit maxima: the bit patterns of
// non-negative bf16 values order as their values).
__device__ __forceinline__ u16x2 max_abs8(const uint4& v, u16x2 r) {
  const uint32_t u4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int h = 0; h < 4; ++h) r = __builtin_elementwise_max(r, __builtin_bit_cast(u16x2, u4[h] & 0x7FFF7FFFu));
  return r;
}

// The fused gate/up epilogue: the SwiGLU cast chain of the pages' GATEUP
// kernel -- gate and up to bf16, sigmoid of the bf16 gate to bf16, silu =
// bf16(gate * sigmoid), out = bf16(silu * up).  The sigmoid takes e^-|g|, so
// no exponential overflows: for g below about -88, 1 / (1 + e^-g) would
// overflow f32 to 0 where the sigmoid is still a bf16 subnormal.
__device__ __forceinline__ uint16_t swiglu_bf16(float gate, float up) {
  const float gT = round_bf16(gate);
  const float uT = round_bf16(up);
  const float t = expf(-fabsf(gT));
  const float sig = round_bf16(gT >= 0.0f ? 1.0f / (1.0f + t) : t / (1.0f + t));
  const float silu = round_bf16(gT * sig);
  return f32_to_bf16_bits(silu * uT);
}

// The code words of five run groups of one tile row, read from the ring and
// waited for in one block: for group g the K words at LDS byte address aw[g]
// and the spill word at as[g] (the word after the run, wrapped in its block);
// the same block reads the dword at ax into xv.
template <int K>
__device__ __forceinline__ void lds_read_runs5(const uint32_t (&aw)[5], const uint32_t (&as)[5],
                                               uint32_t (&W)[5][K + 1], uint32_t ax, uint32_t& xv) {
  if constexpr (K == 2) {
    lds_u32x2 p[5];
    uint32_t sp[5];
    asm volatile(
        "ds_read_b64 %0, %11\n\tds_read_b32 %1, %12\n\t"
        "ds_read_b64 %2, %13\n\tds_read_b32 %3, %14\n\t"
        "ds_read_b64 %4, %15\n\tds_read_b32 %5, %16\n\t"
        "ds_read_b64 %6, %17\n\tds_read_b32 %7, %18\n\t"
        "ds_read_b64 %8, %19\n\tds_read_b32 %9, %20\n\t"
        "ds_read_b32 %10, %21\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(p[0]), "=&v"(sp[0]), "=&v"(p[1]), "=&v"(sp[1]), "=&v"(p[2]), "=&v"(sp[2]), "=&v"(p[3]), "=&v"(sp[3]),
          "=&v"(p[4]), "=&v"(sp[4]), "=&v"(xv)
        : "v"(aw[0]), "v"(as[0]), "v"(aw[1]), "v"(as[1]), "v"(aw[2]), "v"(as[2]), "v"(aw[3]), "v"(as[3]), "v"(aw[4]),
          "v"(as[4]), "v"(ax)
        : "memory");
#pragma unroll
    for (int g = 0; g < 5; ++g) {
      W[g][0] = p[g][0];
      W[g][1] = p[g][1];
      W[g][2] = sp[g];
    }
  } else if constexpr (K == 4) {
    lds_u32x4 p[5];
    uint32_t sp[5];
    asm volatile(
        "ds_read_b128 %0, %11\n\tds_read_b32 %1, %12\n\t"
        "ds_read_b128 %2, %13\n\tds_read_b32 %3, %14\n\t"
        "ds_read_b128 %4, %15\n\tds_read_b32 %5, %16\n\t"
        "ds_read_b128 %6, %17\n\tds_read_b32 %7, %18\n\t"
        "ds_read_b128 %8, %19\n\tds_read_b32 %9, %20\n\t"
        "ds_read_b32 %10, %21\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(p[0]), "=&v"(sp[0]), "=&v"(p[1]), "=&v"(sp[1]), "=&v"(p[2]), "=&v"(sp[2]), "=&v"(p[3]), "=&v"(sp[3]),
          "=&v"(p[4]), "=&v"(sp[4]), "=&v"(xv)
        : "v"(aw[0]), "v"(as[0]), "v"(aw[1]), "v"(as[1]), "v"(aw[2]), "v"(as[2]), "v"(aw[3]), "v"(as[3]), "v"(aw[4]),
          "v"(as[4]), "v"(ax)
        : "memory");
#pragma unroll
    for (int g = 0; g < 5; ++g) {
#pragma unroll
      for (int m = 0; m < 4; ++m) W[g][m] = p[g][m];
      W[g][4] = sp[g];
    }
  } else {                                     // K == 3: words 4-byte aligned only
    lds_u32x2 p[5];
    uint32_t t3[5], sp[5];
    asm volatile(
        "ds_read2_b32 %0, %16 offset1:1\n\tds_read_b32 %1, %16 offset:8\n\tds_read_b32 %2, %17\n\t"
        "ds_read2_b32 %3, %18 offset1:1\n\tds_read_b32 %4, %18 offset:8\n\tds_read_b32 %5, %19\n\t"
        "ds_read2_b32 %6, %20 offset1:1\n\tds_read_b32 %7, %20 offset:8\n\tds_read_b32 %8, %21\n\t"
        "ds_read2_b32 %9, %22 offset1:1\n\tds_read_b32 %10, %22 offset:8\n\tds_read_b32 %11, %23\n\t"
        "ds_read2_b32 %12, %24 offset1:1\n\tds_read_b32 %13, %24 offset:8\n\tds_read_b32 %14, %25\n\t"
        "ds_read_b32 %15, %26\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(p[0]), "=&v"(t3[0]), "=&v"(sp[0]), "=&v"(p[1]), "=&v"(t3[1]), "=&v"(sp[1]), "=&v"(p[2]),
          "=&v"(t3[2]), "=&v"(sp[2]), "=&v"(p[3]), "=&v"(t3[3]), "=&v"(sp[3]), "=&v"(p[4]), "=&v"(t3[4]),
          "=&v"(sp[4]), "=&v"(xv)
        : "v"(aw[0]), "v"(as[0]), "v"(aw[1]), "v"(as[1]), "v"(aw[2]), "v"(as[2]), "v"(aw[3]), "v"(as[3]), "v"(aw[4]),
          "v"(as[4]), "v"(ax)
        : "memory");
#pragma unroll
    for (int g = 0; g < 5; ++g) {
      W[g][0] = p[g][0];
      W[g][1] = p[g][1];
      W[g][2] = t3[g];
      W[g][3] = sp[g];
    }
  }
}

// GROUP: the launch spans the row groups of several matrices (a grouped
// call); the plain and gate/up instantiations compile the lookup out.
// DECODE = false is the decode-free timing floor: the raw code words go to
// the MFMA in place of the decoded codes (meaningless outputs), so a launch
// costs the copies, the MFMAs, the prologue and the epilogue without the
// decode.
template <int K, bool GATEUP, int NG, bool GROUP = false, bool DECODE = true>
__device__ __forceinline__ void axis1_body(
    const uint32_t* __restrict__ codes0, const uint16_t* __restrict__ scales0,
    const uint32_t* __restrict__ codes1, const uint16_t* __restrict__ scales1,
    const uint16_t* __restrict__ x, void* __restrict__ out, int out_f32,
    float* __restrict__ gate_f32, float* __restrict__ up_f32, const Axis1Geom g, const int bid, int gdim) {
  constexpr int WPB = words_per_block(K);
  constexpr int BLK = WPB * 4;                 // bytes per packed block
  constexpr int ROWS = GATEUP ? 8 : 16;        // output rows per row group
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // the pointers the first copies need are read with the geometry at entry
  // (one wait for all of them instead of one per use)
  asm volatile("" : "+s"(gdim) : "s"(codes0), "s"(codes1), "s"(x), "s"(g.R), "s"(g.row_bytes), "s"(g.ldx), "s"(g.M),
               "s"(g.per));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, q = lane >> 4;
  const int M = g.M;
  const int64_t R = g.R;
  const int NS = g.nslots, nwd = g.nwd, gsw = g.gsw;
  const bool hit = g.half && bid < 2 * g.nrem;                                  // this workgroup has a half row group
  const int nmine = g.nfull + ((g.half ? hit : bid < g.nrem) ? 1 : 0);          // row groups (the half last)
  const int nwhole = hit ? g.nfull : nmine;
  uint8_t* ring = smem + (size_t)wave * NS * g.slot_bytes;                      // this wave's slots
  float* part = reinterpret_cast<float*>(smem + g.part_off);
  // progress of the two waves of a SIMD (w and w ^ 4): the one ahead yields
  const uint32_t prog_mine = lds_addr(smem + g.prog_off) + (uint32_t)wave * 4u;
  const uint32_t prog_other = lds_addr(smem + g.prog_off) + (uint32_t)(wave ^ 4) * 4u;
  lds_write_b32(prog_mine, 0u);

  // Grouped calls: the matrix gi of row group rg and its row group lrg in
  // that matrix (compile-time indices only, so the table stays in SGPRs).
  auto locate = [&](int64_t rg, int& gi, int64_t& lrg) {
    gi = 0;
    int64_t start = 0;
    if constexpr (GROUP && !GATEUP) {
#pragma unroll
      for (int j = 0; j + 1 < kMaxGroup; ++j)
        if (j + 1 < g.ngroup && rg >= g.gend[j]) {
          gi = j + 1;
          start = g.gend[j];
        }
    }
    lrg = rg - start;
  };
  auto pick = [&](auto p0, auto const (&tab)[kMaxGroup], int gi) {
    auto p = p0;
    if constexpr (GROUP) {
#pragma unroll
      for (int j = 1; j < kMaxGroup; ++j)
        if (gi == j) p = tab[j];
    }
    return p;
  };
  // row group of item t: whole ones bid + t grid, the half nfull grid + bid / 2
  auto item_rg = [&](int t) -> int64_t {
    return (hit && t == g.nfull) ? (int64_t)g.nfull * gdim + (bid >> 1) : (int64_t)bid + (int64_t)t * gdim;
  };

  // ---- 0. the scales of the workgroup's rows go to LDS ahead of everything
  // else, so the epilogue reads them there: dword v holds rows 2 (v % 8) and
  // 2 (v % 8) + 1 of item v / 8 (gate/up: dwords 0-3 the gate rows, 4-7 the
  // up rows).  A pair that reaches past the matrix is not copied (a ragged
  // last row group; an odd R leaves its last row to the epilogue's global
  // read), nor are scales whose pointer is not 4-byte aligned.
  bool sc_ok =
      ((reinterpret_cast<uintptr_t>(scales0) | (GATEUP ? reinterpret_cast<uintptr_t>(scales1) : 0u)) & 3u) == 0;
  if constexpr (GROUP) {
#pragma unroll
    for (int j = 1; j < kMaxGroup; ++j)
      if (j < g.ngroup) sc_ok = sc_ok && (reinterpret_cast<uintptr_t>(g.gscales[j]) & 3u) == 0;
  }
  if (sc_ok) {
    for (int v0 = wave * 64; v0 < nmine * 8; v0 += kThreads) {   // wave-uniform
      const int v = v0 + lane, t = min(v >> 3, nmine - 1), d = v & 7;
      int gi;
      int64_t lrg;
      locate(item_rg(t), gi, lrg);
      const int64_t Rm = pick(R, g.gR, gi);
      const int64_t row = GATEUP ? lrg * ROWS + 2 * (d & 3) : lrg * ROWS + 2 * d;
      const uint16_t* sp = GATEUP ? (d < 4 ? scales0 : scales1) : pick(scales0, g.gscales, gi);
      if (v < nmine * 8 && row + 1 < Rm)
        __builtin_amdgcn_global_load_lds(sp + row, smem + g.sc_off + (uint32_t)v0 * 4u, 4, 0, 0);
    }
  }

  // ---- this wave's slice: runs [rb, re) of 32 columns, held in packed
  // blocks [b0, b1]; a tile row of the wave's window is those blocks
  const int per = g.per;
  const int rb = wave * per, re = rb + per;
  const int b0 = rb >> 3, b1 = (re - 1) >> 3;
  const int gwr = (b1 - b0 + 1) * (BLK / 16);  // granules of the window per row (< gsw)

  // ---- 1. the wave's slice of x (M vectors) goes out first, into its last
  // ring slots (the first tiles follow once their descriptors are ready)
  const int gx = per * 4;                      // 16-byte granules of one vector's slice
  const int nxg = M * gx;
  const int nxw = (nxg + 63) / 64;
  uint8_t* xsl = ring + (size_t)(NS - g.xslots) * g.slot_bytes;                  // [n][slice], then x'
  for (int j = 0; j < nxw; ++j) {              // every issued copy has an active lane
    const int p = j * 64 + lane;
    if (p < nxg) {
      const int n = (p >= gx) + (p >= 2 * gx) + (p >= 3 * gx), jj = p - n * gx;
      __builtin_amdgcn_global_load_lds(x + (int64_t)n * g.ldx + (int64_t)rb * 32 + jj * 8, xsl + (size_t)j * 1024,
                                       16, 0, 0);
    }
  }

  // copy descriptors.  A tile is ROWS rows of each matrix it reads (16 of
  // one, or 8 gate rows then 8 up rows), row r of the tile r * gsw granules
  // into the slot.  Copy j moves granules p = 64 (j mod nh) + lane of its
  // matrix's rows; granule p is granule p % gsw of row p / gsw.  Lanes whose
  // granule is a row's pad granule copy the row's first block into that pad
  // (which nothing reads), so only the last copy of each matrix masks lanes:
  // those past its ROWS rows, whose LDS would belong to the next rows or
  // slot.  dd = the lane's byte offset from the tile's first row, computed
  // once.
  const int nh = GATEUP ? nwd / 2 : nwd;
  const uint32_t row_bytes = (uint32_t)g.row_bytes;
  constexpr int NDMA = max_dma(K);
  uint32_t dd[NDMA];
#pragma unroll
  for (int j = 0; j < NDMA; ++j) {
    const int jh = (GATEUP && j >= nh) ? j - nh : j;
    const uint32_t p = (uint32_t)(jh * 64 + lane);
    const uint32_t r = (uint32_t)(((uint64_t)p * g.gsw_magic) >> 24), jj = p - r * (uint32_t)gsw;
    dd[j] = (uint32_t)b0 * BLK + ((p < (uint32_t)(ROWS * gsw) && jj < (uint32_t)gwr) ? r * row_bytes + jj * 16u : 0u);
  }
  const bool tail_ok = (uint32_t)((nh - 1) * 64 + lane) < (uint32_t)(ROWS * gsw);   // lane of a last copy in use
  const uint32_t up_lds = (uint32_t)(ROWS * gsw * 16);   // LDS byte offset of the up rows in a tile
  const int ncp = nwd;                         // copies per tile (wave-uniform)
  const uint8_t* cb0 = reinterpret_cast<const uint8_t*>(codes0);
  const uint8_t* cb1 = reinterpret_cast<const uint8_t*>(GATEUP ? codes1 : codes0);
  auto issue_tile = [&](int t) {
    int gi;
    int64_t rg;
    locate(item_rg(t), gi, rg);
    const int64_t Rm = pick(R, g.gR, gi);
    const uint8_t* cbm = GATEUP ? cb0 : reinterpret_cast<const uint8_t*>(pick(codes0, g.gcodes, gi));
    uint8_t* slot = ring + (size_t)(t % NS) * g.slot_bytes;
    // the tile's rows of each matrix as one buffer: rows past the matrix
    // (a ragged last row group) or past a half's ROWS / 2 rows fall outside
    // it and read as zeros
    const bool hf = hit && t == g.nfull;
    const int64_t r0 = rg * ROWS + (hf ? (bid & 1) * (ROWS / 2) : 0);
    const int64_t nrow = hf ? ROWS / 2 : ROWS;
    const int64_t left = Rm - r0;
    const int nbytes = (int)((left < nrow ? (left > 0 ? left : 0) : nrow) * (int64_t)row_bytes);
    const __amdgpu_buffer_rsrc_t rs0 =
        __builtin_amdgcn_make_buffer_rsrc((void*)(cbm + r0 * g.row_bytes), (short)0, nbytes, kRawBufferWord3);
    const __amdgpu_buffer_rsrc_t rs1 =
        GATEUP ? __builtin_amdgcn_make_buffer_rsrc((void*)(cb1 + r0 * g.row_bytes), (short)0, nbytes, kRawBufferWord3)
               : rs0;
#pragma unroll
    for (int j = 0; j < NDMA; ++j) {
      if (j < nwd) {
        const bool up = GATEUP && j >= nh;
        const int jh = up ? j - nh : j;
        if (jh < nh - 1 || tail_ok)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              up ? rs1 : rs0,
              (__attribute__((address_space(3))) void*)(slot + (up ? up_lds : 0u) + (uint32_t)jh * 1024u), 16,
              (int)dd[j], 0, 0, 0);
      }
    }
  };

  // the ring fills a little at a time: one tile now, in a slot the x slice
  // does not use, the second once the x slice is in registers (every
  // workgroup's first tiles share HBM; a second tile in that first burst
  // delays the first, most for k = 4)
  int next = 0;                                // next tile to copy; tiles go out in order
  const int t0 = min(nmine, min(1, NS - g.xslots));
  for (; next < t0; ++next) issue_tile(next);
  wait_vmcnt(ncp * t0);                        // the x slice has landed

  // ---- 2. exponent of the slice per vector: its largest |x[n]| * 2^e lands
  // in [2^14, 2^15); then x' = f16(x 2^e) in place.  Each vector's granules
  // belong to one group of G = 64 / M' lanes (M' = M rounded up to a power
  // of two): lane (n, j) = (lane / G, lane % G) takes granules j, j + G, ...
  // of vector n, so the maximum is one short DPP reduction over the group
  // and each lane scales by its own vector's exponent.
  static_assert(kXPer == 5, "x granules are read five at a time");
  const int lgG = M == 1 ? 6 : (M == 2 ? 5 : 4);
  const int G = 1 << lgG;
  const int xn = lane >> lgG, xj = lane & (G - 1);
  const int nxu = (gx + G - 1) >> lgG;         // granules per lane (<= kXPer: gx <= 80)
  uint4 xr[kXPer];
  uint32_t xa[kXPer];
  bool xok[kXPer];
  {
#pragma unroll
    for (int u = 0; u < kXPer; ++u) {          // granules past the slice read granule 0 and are zeroed
      const int jj = u * G + xj;
      xok[u] = xn < M && u < nxu && jj < gx;
      xa[u] = lds_addr(xsl) + (uint32_t)(xok[u] ? xn * gx + jj : 0) * 16u;
    }
    lds_u32x4 xv[kXPer];
    lds_read_b128x5(xa, xv);
#pragma unroll
    for (int u = 0; u < kXPer; ++u)
      xr[u] = xok[u] ? make_uint4(xv[u][0], xv[u][1], xv[u][2], xv[u][3]) : make_uint4(0u, 0u, 0u, 0u);
  }
  u16x2 mxp = {0, 0};
#pragma unroll
  for (int u = 0; u < kXPer; ++u) {
    if (u >= nxu) break;                       // wave-uniform
    mxp = max_abs8(xr[u], mxp);                // zero past the slice
  }
  uint32_t mx = max((uint32_t)mxp.x, (uint32_t)mxp.y);
  // maximum over the lane's group: within rows of 16 by rotation (every
  // lane of a row ends with the row's maximum), then across rows
  mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x121, 0xF, 0xF, false));   // row_ror:1
  mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x122, 0xF, 0xF, false));   // row_ror:2
  mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x124, 0xF, 0xF, false));   // row_ror:4
  mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x128, 0xF, 0xF, false));   // row_ror:8
  if (lgG >= 5) {                              // rows 1 and 3 take the maxima of rows 0-1 and 2-3
    mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x142, 0xA, 0xF, false));   // row_bcast:15
    if (lgG == 6) {                            // rows 2 and 3 take the maximum of rows 0-1: row 3 has all
      mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)mx, 0x143, 0xC, 0xF, false));   // row_bcast:31
      mx = (uint32_t)__builtin_amdgcn_readlane((int)mx, 63);
    } else {
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)mx, 31);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)mx, 63);
      mx = lane < 32 ? lo : hi;
    }
  }
  auto exponent = [](uint32_t v) {
    int e = 0;
    if (v != 0u && v < 0x7F80u) {              // finite, non-zero maximum
      int ex;
      frexpf(bf16_bits_to_f32(v), &ex);        // max in [2^(ex-1), 2^ex)
      e = 15 - ex;
    }
    return e;
  };
  const int xe = exponent(mx);                 // the exponent of this lane's vector
  // per-vector exponents for the epilogue's scaling (vectors past M: 0)
  const int e0 = __builtin_amdgcn_readlane(xe, 0);
  const int e1 = M > 1 ? __builtin_amdgcn_readlane(xe, 1 * (M == 2 ? 32 : 16)) : 0;
  const int e2 = M > 2 ? __builtin_amdgcn_readlane(xe, 32) : 0;
  const int e3 = M > 3 ? __builtin_amdgcn_readlane(xe, 48) : 0;
#pragma unroll
  for (int u = 0; u < kXPer; ++u) {
    if (u >= nxu) break;
    const uint32_t u4[4] = {xr[u].x, xr[u].y, xr[u].z, xr[u].w};
    uint32_t o[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      o[h] = pack_f16x2(ldexpf(bf16_bits_to_f32(u4[h] & 0xFFFFu), xe), ldexpf(bf16_bits_to_f32(u4[h] >> 16), xe));
    }
    if (xok[u]) lds_write_b128(xa[u], lds_u32x4{o[0], o[1], o[2], o[3]});
  }

  // ---- 3. B operand in registers: lane (n, q) of group gg holds
  // x'[n, run * 32 + 8u .. +7] for run = rb + 4 gg + q (zero past the M
  // vectors or past the slice, whose A lanes then decode run rb): those
  // lanes read 64 zero bytes written after the slice's x'.
  const uint32_t zero_lds = lds_addr(xsl) + (uint32_t)nxg * 16u;
  if (lane < 4) lds_write_b128(zero_lds + (uint32_t)lane * 16u, lds_u32x4{0u, 0u, 0u, 0u});
  half8 B[NG][4];
  int wo[NG], so[NG];
  const int ngw = (per + 3) >> 2;              // groups of four runs (<= NG)
  uint32_t ba[NG];
#pragma unroll
  for (int gg = 0; gg < NG; ++gg) {
    const int run = rb + 4 * gg + q;
    const bool valid = run < re;
    const int runc = valid ? run : rb;
    const int w0 = (7 - (runc & 7)) * K;
    const int blk = (runc >> 3) - b0;          // block within the window
    wo[gg] = blk * WPB + w0;
    so[gg] = blk * WPB + (w0 + K == WPB ? 0 : w0 + K);   // word after the run, wrapping in the block
    ba[gg] = (valid && i < M) ? lds_addr(xsl + ((size_t)i * gx * 8 + (size_t)(runc - rb) * 32) * 2) : zero_lds;
  }
  {
    lds_u32x4 bv[NG][4];
    lds_read_b128x4n<NG>(ba, bv);              // in-slice address for every lane
#pragma unroll
    for (int gg = 0; gg < NG; ++gg)
#pragma unroll
      for (int u = 0; u < 4; ++u) B[gg][u] = __builtin_bit_cast(half8, bv[gg][u]);
  }
  const int my_e = i == 0 ? e0 : i == 1 ? e1 : i == 2 ? e2 : e3;     // scale of column n = i

  __atomic_signal_fence(__ATOMIC_SEQ_CST);     // the x' reads above stay before any later copy
  for (; next < min(nmine, 2); ++next) issue_tile(next);   // the x slots are free now

  const uint32_t mul = kMul;
  const uint64_t add64 = kAdd;
  for (int t = 0; t < nwhole; ++t) {
    wait_vmcnt(ncp * (next - 1 - t));          // tile t has landed (tiles after it may be in flight)
    const uint8_t* trow = ring + (size_t)(t % NS) * g.slot_bytes + (size_t)i * gsw * 16;
    f32x4 acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto consume = [&](const uint32_t (&W)[K + 1], const half8 (&Bg)[4]) {
      u32x4 A[4];
      if constexpr (DECODE) {
        decode_run_codes<K>(W, mul, add64, A);
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) A[u] = u32x4{W[u % (K + 1)], W[(u + 1) % (K + 1)], W[(u + 2) % (K + 1)], W[0]};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, A[u]), Bg[u], acc[u], 0, 0, 0);
    };
    // the words of every group of the tile in one read block; groups past
    // the B capacity re-read group 0 (their words are not used)
    static_assert(NG <= 5, "at most five run groups per tile row");
    uint32_t aw[5], as[5];
    const uint32_t tb = lds_addr(trow);
#pragma unroll
    for (int gg = 0; gg < 5; ++gg) {
      aw[gg] = tb + (uint32_t)wo[gg < NG ? gg : 0] * 4u;
      as[gg] = tb + (uint32_t)so[gg < NG ? gg : 0] * 4u;
    }
    // the same read block fetches the partner wave's progress.  The two waves
    // of a SIMD (w, w ^ 4) share its VALU: the one that has finished more row
    // groups drops to the lower issue priority, so neither runs ahead and
    // leaves the other to finish alone (the hardware breaks ties by age, so
    // on a tie the younger wave takes the higher priority)
    uint32_t W[5][K + 1];
    uint32_t other_v;
    lds_read_runs5<K>(aw, as, W, prog_other, other_v);
    {
      const uint32_t other = (uint32_t)__builtin_amdgcn_readfirstlane((int)other_v);
      if ((uint32_t)t < other || ((uint32_t)t == other && wave >= 4)) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
    }
#pragma unroll
    for (int gg = 0; gg < NG; ++gg)
      if (gg < ngw) consume(W[gg], B[gg]);
    // partial D tile of this slice: lane (n, q) holds rows 4q .. 4q+3 of
    // column n; scaled back by 2^-e_n (exact) into common units
    const f32x4 sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    f32x4 pv;
#pragma unroll
    for (int e = 0; e < 4; ++e) pv[e] = ldexpf(sum[e], -my_e);
    if (i < M) *reinterpret_cast<f32x4*>(part + ((size_t)(t * kWaves + wave) * 4 + i) * 16 + 4 * q) = pv;
    lds_write_b32(prog_mine, (uint32_t)t + 1u);
    // refill: one tile per row group, so the ring stays as far ahead as the
    // prologue put it (tile t + 2 goes out when row group t ends).  More
    // copies in flight only lengthened the issue of each copy: two per row
    // group (up to t + NS) ran gate/up 0.35 us slower per call.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (next < nmine && next <= t + NS) issue_tile(next++);
  }

  // ---- 4b. the half row group (always the last item): ROWS / 2 output
  // rows.  MFMA row i < 8 carries output row i & 7 (gate/up: gate rows 0-3,
  // up rows 4-7) at run positions 0-15, row 8 + i the same output row at
  // positions 16-31; B columns 0-3 hold x' of positions 0-15 (the lane's
  // own B[gg][0..1]) and columns 4-7 x' of positions 16-31 (B[gg][2..3] of
  // lane n - 4, one DPP row shift).  D rows 0-7 x columns 0-3 and rows 8-15
  // x columns 4-7 are the two halves of each sum; the epilogue adds them.
  if (hit) {
    const int t = g.nfull;
    wait_vmcnt(0);
    const int hr = GATEUP ? ((i & 7) < 4 ? (i & 3) : 8 + (i & 3)) : (i & 7);   // tile row of the lane
    const uint32_t tbh = lds_addr(ring + (size_t)(t % NS) * g.slot_bytes + (size_t)hr * gsw * 16);
    uint32_t aw[5], as[5];
#pragma unroll
    for (int gg = 0; gg < 5; ++gg) {
      aw[gg] = tbh + (uint32_t)wo[gg < NG ? gg : 0] * 4u;
      as[gg] = tbh + (uint32_t)so[gg < NG ? gg : 0] * 4u;
    }
    uint32_t W[5][K + 1];
    uint32_t other_v;
    lds_read_runs5<K>(aw, as, W, prog_other, other_v);
    asm volatile("" : : "v"(other_v));         // (the progress word is not needed here)
    f32x4 hacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int gg = 0; gg < NG; ++gg) {
      if (gg < ngw) {
        u32x4 A2[2];
        if constexpr (DECODE) {
          decode_half_codes<K>(W[gg], i >= 8, mul, add64, A2);
        } else {
#pragma unroll
          for (int u = 0; u < 2; ++u) A2[u] = u32x4{W[gg][u % (K + 1)], W[gg][(u + 1) % (K + 1)], W[gg][0], W[gg][K]};
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const u32x4 own = __builtin_bit_cast(u32x4, B[gg][u]);
          const u32x4 hi = __builtin_bit_cast(u32x4, B[gg][u + 2]);
          // lanes 4-7 of each row take lane n - 4's upper x' (row_shr:4,
          // bank 1 only); every other lane keeps its own B, which is zero for
          // n >= M (so for n >= 4)
          u32x4 bh;
#pragma unroll
          for (int c = 0; c < 4; ++c)
            bh[c] = (uint32_t)__builtin_amdgcn_update_dpp((int)own[c], (int)hi[c], 0x114, 0xF, 0x2, false);
          hacc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, A2[u]),
                                                           __builtin_bit_cast(half8, bh), hacc[u], 0, 0, 0);
        }
      }
    }
    // lane (n, q) holds D rows 4q .. 4q+3 of column n: n < 4, q < 2 the
    // first halves of vector n, 4 <= n < 8, q >= 2 the second halves of
    // vector n - 4; both go to the partial tile of that vector, rows 4q ..
    const f32x4 hsum = hacc[0] + hacc[1];
    const int m = i & 3;
    const int me = m == 0 ? e0 : m == 1 ? e1 : m == 2 ? e2 : e3;
    f32x4 hv;
#pragma unroll
    for (int e = 0; e < 4; ++e) hv[e] = ldexpf(hsum[e], -me);
    if (m < M && ((i < 4 && q < 2) || (i >= 4 && i < 8 && q >= 2)))
      *reinterpret_cast<f32x4*>(part + ((size_t)(t * kWaves + wave) * 4 + m) * 16 + 4 * q) = hv;
  }

  // ---- 5. one barrier, then every output: the eight slices' partials in a
  // fixed order, times scale / d, and the epilogue
  lds_barrier();
  // thread idx takes output row idx % ROWS of vector (idx / ROWS) % 4 of
  // item idx / (4 ROWS) (shifts only; vectors past M skip)
  constexpr int kRowsLog = GATEUP ? 3 : 4;
  for (int idx = tid; idx < nmine * 4 * ROWS; idx += kThreads) {
    const int t = idx >> (kRowsLog + 2), m = (idx >> kRowsLog) & 3, row = idx & (ROWS - 1);
    if (m >= M) continue;
    int gi;
    int64_t lrg;
    locate(item_rg(t), gi, lrg);
    const bool hf = hit && t == g.nfull;
    if (hf && row >= ROWS / 2) continue;
    const int64_t Rm = pick(R, g.gR, gi);
    const int64_t orow = lrg * ROWS + (hf ? (bid & 1) * (ROWS / 2) : 0) + row;
    if (orow >= Rm) continue;
    const int64_t o = (int64_t)m * Rm + orow;
    const float* pp = part + ((size_t)t * kWaves * 4 + m) * 16;
    // partial-tile rows of this output: whole row groups row (gate/up: gate
    // row, up row + 8); a half its two position halves, rows row and row + 8
    // (gate/up: gate row and row + 8, up 4 + row and 12 + row).  Both reads
    // are made either way (the second repeats the first for a whole row
    // group), so the sum needs no branch.
    const int b0h = hf ? row + 8 : row;
    float d0 = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float lo = pp[w * 64 + row], hi = pp[w * 64 + b0h];
      d0 += hf ? lo + hi : lo;
    }
    // the row's scale from LDS (scale row srow of item t), or from global
    // memory where its pair was not copied
    const int srow = (int)(orow - lrg * ROWS);
    const bool sl = sc_ok && (orow | 1) < Rm;
    const uint8_t* sct = smem + g.sc_off + (size_t)t * kScaleBytes;
    const uint16_t sg = sl ? *reinterpret_cast<const uint16_t*>(sct + srow * 2) : pick(scales0, g.gscales, gi)[orow];
    const float v0 = d0 * (half_bits_to_f32(sg) * kRcp);
    if constexpr (GATEUP) {
      const int a1 = hf ? 4 + row : 8 + row, b1 = hf ? 12 + row : 8 + row;
      float d1 = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float lo = pp[w * 64 + a1], hi = pp[w * 64 + b1];
        d1 += hf ? lo + hi : lo;
      }
      const uint16_t su = sl ? *reinterpret_cast<const uint16_t*>(sct + 16 + srow * 2) : scales1[orow];
      const float v1 = d1 * (half_bits_to_f32(su) * kRcp);
      if (gate_f32) gate_f32[o] = v0;
      if (up_f32) up_f32[o] = v1;
      if (out) reinterpret_cast<uint16_t*>(out)[o] = swiglu_bf16(v0, v1);   // no out: a column chunk
    } else {
      void* om = pick(out, g.gout, gi);
      if (out_f32) reinterpret_cast<float*>(om)[o] = v0;
      else reinterpret_cast<uint16_t*>(om)[o] = f32_to_bf16_bits(v0);
    }
  }
}


// Column chunks of a row: at most kChunkBlocks 256-column blocks each (x of
// a chunk stays in registers), the blocks dealt out evenly.
constexpr int64_t kChunkBlocks = 20;

int64_t axis1_nchunks(int64_t C) {
  const int64_t nb = C / 256;
  return nb < 1 ? 1 : (nb + kChunkBlocks - 1) / kChunkBlocks;
}

// first block of chunk j of n over nb blocks (chunk j is [first(j), first(j + 1)))
int64_t axis1_chunk_first(int64_t nb, int64_t n, int64_t j) { return j * nb / n; }

// MFMA groups of four runs per wave -> the register-resident B capacity
// instantiated for it (2 or 5 groups: C <= 2048 or C <= 5120); 0 if C is too
// wide for B to stay in registers.
int axis1_ng(int64_t C) {
  const int64_t per = C / 256;                 // runs per wave
  const int64_t ngw = (per + 3) / 4;
  return ngw <= 2 ? 2 : ngw <= 5 ? 5 : 0;
}

// Host geometry; returns false if the shape does not fit (LDS or registers).
// nrg_total: row groups of the launch (0: those of R; a grouped call passes
// the sum over its matrices).
bool axis1_geom(int64_t R, int64_t C, int M, int k, bool gateup, int64_t grid, Axis1Geom& g,
                int64_t nrg_total = 0) {
  const int rows = gateup ? 8 : 16;
  if (M < 1 || M > 4 || C % 256 != 0 || axis1_ng(C) == 0) return false;
  const int blk = 256 * k / 8;                 // bytes per block
  g = Axis1Geom{};
  g.R = R;
  g.C = C;
  g.ldx = C;
  g.M = M;
  g.nrg = nrg_total > 0 ? nrg_total : (R + rows - 1) / rows;
  g.ngroup = 1;
  g.gend[0] = g.nrg;
  g.gR[0] = R;
  g.row_bytes = C * k / 8;
  g.per = (int)(C / 256);
  int nb = 0;                                  // widest wave window in blocks
  for (int w = 0; w < kWaves; ++w) {
    const int rb = w * g.per, re = rb + g.per;
    const int b = ((re - 1) >> 3) - (rb >> 3) + 1;
    nb = b > nb ? b : nb;
  }
  g.gsw = nb * blk / 16 + 1;
  const int nh = (rows * g.gsw + 63) / 64;     // copies per matrix of a tile
  g.nwd = gateup ? 2 * nh : nh;
  if (g.nwd > max_dma(k)) return false;
  g.gsw_magic = (uint32_t)(((1u << 24) + g.gsw - 1) / g.gsw);
  g.nmine_max = (int)((g.nrg + grid - 1) / grid);
  g.nfull = (int)(g.nrg / grid);
  g.nrem = (int)(g.nrg % grid);
  // the last round in halves when its row groups fill at most half the grid.
  // A half computes its outputs bit for bit as the whole row group would:
  // its two MFMAs per run group see, per output element, the same operands
  // as the whole row group's MFMAs 0/1 and 2/3, and the epilogue adds the
  // two position halves in the same order.
  g.half = (g.nrem > 0 && 2 * (int64_t)g.nrem <= grid) ? 1 : 0;
  g.slot_bytes = (uint32_t)((16 * g.gsw * 16 + 255) / 256 * 256);
  const uint64_t parts = (uint64_t)g.nmine_max * kPartBytes;
  if (parts >= kAxis1MaxLdsBytes) return false;
  const uint64_t fixed = parts + kProgBytes + (uint64_t)g.nmine_max * kScaleBytes;
  if (fixed >= kAxis1MaxLdsBytes) return false;
  const uint64_t nsl = (kAxis1MaxLdsBytes - fixed) / ((uint64_t)kWaves * g.slot_bytes);
  g.nslots = (int)(nsl < (uint64_t)kMaxSlots ? nsl : kMaxSlots);
  const uint64_t xbytes = (uint64_t)M * g.per * 64 + 64;   // one wave's x slice and 64 zero bytes
  g.xslots = (int)((xbytes + g.slot_bytes - 1) / g.slot_bytes);
  if (g.nslots < 2 || g.nslots < g.xslots + 1) return false;
  g.part_off = (uint32_t)kWaves * g.nslots * g.slot_bytes;
  g.prog_off = (uint32_t)(g.part_off + parts);
  g.sc_off = g.prog_off + kProgBytes;
  g.total = g.sc_off + (uint32_t)g.nmine_max * kScaleBytes;
  return g.total <= kAxis1MaxLdsBytes;
}

// One workgroup per CU, or per row group when there are fewer; a plain or
// gate/up call with at most half as many row groups as CUs runs each of
// them as two halves on twice as many workgroups.
int64_t axis1_grid(int64_t R, bool gateup, int64_t nrg_total = 0) {
  const int64_t rows = gateup ? 8 : 16;
  const int64_t nrg = nrg_total > 0 ? nrg_total : (R + rows - 1) / rows;
  const int64_t cus = device_cus();
  if (nrg >= cus) return cus;
  return (nrg_total == 0 && 2 * nrg <= cus) ? 2 * nrg : nrg;
}

}  // namespace a1
using namespace a1;
}  // namespace
}  // namespace trellis
