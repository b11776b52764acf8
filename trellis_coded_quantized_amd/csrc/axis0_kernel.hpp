// axis0_kernel.hpp -- device body of the axis-0 (down projection) matvec for
// M <= 4 on gfx950, and its host geometry (the launchers are in axis0.hip).
//
// The stored matrix is W^T [R_in, C_out], coded along C_out; the output is
// out[m, c] = sum_r w(r, c) x[m, r] with w(r, c) = value(s(r, c)) * scale[r].
// Source: mlx-bun 0.2.0 -> 0.4.0 diff (page 55), trellis-linear.ts SCATTER
// kernel and #scatter (split-K over the stored rows, one fold, cast to the
// activation dtype); page 56, trellis-vector-expand.ts (four weights from one
// window).
//
// The sum runs on v_mfma_f32_16x16x32_f16 with the 32 stored rows of a block
// as the contraction dimension:
//   A (16 columns x 32 rows): lane (i, q) decodes output columns 4i .. 4i+3
//     of a 64-column chunk (one 32-bit funnel window holds their four states)
//     for stored rows 8q .. 8q+7; each code y becomes an exact f16 integer,
//     two rows per register (code_pair_y: the byte sums of two 1MAD words
//     as f16 1026 + b, then one packed add of -1536).  Column 4i + j of the
//     chunk is row i of MFMA j.
//   B (32 rows x 16 n): x~[n, r] = scale[r] * x[n, r] (exact in f32) times a
//     per-wave 2^e_n, split into f16 hi (column n) and lo (column 4 + n)
//     halves; hi + lo is exact for every |x~| down to 2^-21 of the wave's
//     largest (below that, lo falls into f16 subnormals).
//   D: f32 sums of signed products (no offset to cancel).
// Work: workgroup (column group g of 256 columns, row split s) with 8 waves;
// wave w takes the split's 32-row blocks w, w + 8, ... through its own LDS
// ring (buffer_load ... lds copies, explicit vmcnt waits, no barrier in the
// loop).  The waves' D tiles meet in LDS at the end; the workgroup writes its
// f32 partial [s][m][c], scaled back by 2^-e_n; a fold kernel adds the splits.
#pragma once
#include "copy_ring.hpp"
#include "internal.hpp"
#include "mfma_common.hpp"

namespace trellis {
namespace {
namespace a0 {


constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kCols = 256;                // output columns per workgroup (one block)
constexpr int kXcds = 8;                  // workgroup b runs on XCD b % 8
constexpr int kChunks = kCols / 64;       // 64-column chunks: four MFMAs each
constexpr int kMaxSlots = 3;
constexpr int kMaxDma = 5;                // copies per wave per 32-row tile (k = 4: 32 rows x 9 granules)
constexpr int kMaxRowsPerSplit = 2048;
constexpr size_t kLdsBudget = 160 * 1024;
constexpr uint32_t kProgBytes = 64;       // blocks each wave has finished: u32 [wave]
// Pad granules after every 8 tile rows.  Lane group q reads tile rows 8q ..
// 8q+7; with rows gsr granules apart alone (a multiple of 4 dwords), rows 8
// apart fall in the same LDS banks and the four groups' reads would conflict
// four ways.  Two extra granules shift group q by 8q dwords: the words one
// read instruction touches (at most 8 per group) then lie in disjoint banks.
constexpr int kQuadPad = 2;

struct Axis0Geom {
  int64_t R, C;
  int M, ncg, S, rps;     // column groups, row splits, rows per split (multiple of 32)
  int64_t row_bytes;       // stride between stored rows (2 blocks when interleaved)
  int interleave;          // codes in the block-interleaved layout [C/512, R, 2 wpb]
  int gsr;                // granules per tile row in LDS (the group's block + one pad granule)
  int gq;                 // granules per 8 tile rows: 8 gsr + kQuadPad
  int nwd;                // copies per wave per tile
  int nslots;
  int scales16;           // scales 16-byte aligned: 16-byte loads in the prologue
  int x16;                // every row of x 16-byte aligned (x aligned, R % 8 == 0)
  uint32_t slot_bytes, xt_off, scr_off, prog_off, total;
  uint32_t scr_wave;      // bytes per wave in the scratch area: its x / scale staging, then its D tiles
};

// Row pairs of one chunk word: ds_read2_b32 of tile rows (0,1), (2,3), (4,5),
// (6,7) from address operand A, rows S dwords apart.
#define TRELLIS_A0_ROWS(O0, O1, O2, O3, A, S0, S1, S2, S3, S4, S5, S6, S7)  \
  "ds_read2_b32 %" #O0 ", %" #A " offset0:" #S0 " offset1:" #S1 "\n\t"     \
  "ds_read2_b32 %" #O1 ", %" #A " offset0:" #S2 " offset1:" #S3 "\n\t"     \
  "ds_read2_b32 %" #O2 ", %" #A " offset0:" #S4 " offset1:" #S5 "\n\t"     \
  "ds_read2_b32 %" #O3 ", %" #A " offset0:" #S6 " offset1:" #S7 "\n\t"
#define TRELLIS_A0_BLOCK(...)                                                \
  TRELLIS_A0_ROWS(0, 1, 2, 3, 18, __VA_ARGS__)                               \
  TRELLIS_A0_ROWS(4, 5, 6, 7, 19, __VA_ARGS__)                               \
  TRELLIS_A0_ROWS(8, 9, 10, 11, 20, __VA_ARGS__)                             \
  TRELLIS_A0_ROWS(12, 13, 14, 15, 21, __VA_ARGS__)                           \
  "ds_read_b128 %16, %22\n\tds_read_b32 %17, %23\n\ts_waitcnt lgkmcnt(0)"
#define TRELLIS_A0_OPERANDS                                                  \
  : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]), "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]),  \
    "=&v"(o[7]), "=&v"(o[8]), "=&v"(o[9]), "=&v"(o[10]), "=&v"(o[11]), "=&v"(o[12]),           \
    "=&v"(o[13]), "=&v"(o[14]), "=&v"(o[15]), "=&v"(bv), "=&v"(xv)                              \
  : "v"(a0[0]), "v"(a1[0]), "v"(a0[1]), "v"(a1[1]), "v"(ab), "v"(ax)                           \
  : "memory"

// The words of two 64-column chunks for the lane's eight tile rows, read from
// the ring and waited for in one block: W[c][rr][0] at LDS byte address
// a0[c] and W[c][rr][1] at a1[c], row rr lying rr * (2K + 1) * 4 dwords
// further (one block plus one pad granule per row); also the 16 bytes at ab
// and the dword at ax (into xv).
template <int K>
__device__ __forceinline__ void lds_read_chunks2(const uint32_t (&a0)[2], const uint32_t (&a1)[2], uint32_t ab,
                                                 uint32_t (&W)[2][8][2], lds_u32x4& bv, uint32_t ax, uint32_t& xv) {
  static_assert(words_per_block(K) / 4 + 1 == 2 * K + 1, "tile rows are one block plus one granule");
  lds_u32x2 o[16];
  if constexpr (K == 2) {
    asm volatile(TRELLIS_A0_BLOCK(0, 20, 40, 60, 80, 100, 120, 140) TRELLIS_A0_OPERANDS);
  } else if constexpr (K == 3) {
    asm volatile(TRELLIS_A0_BLOCK(0, 28, 56, 84, 112, 140, 168, 196) TRELLIS_A0_OPERANDS);
  } else {
    asm volatile(TRELLIS_A0_BLOCK(0, 36, 72, 108, 144, 180, 216, 252) TRELLIS_A0_OPERANDS);
  }
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int pr = 0; pr < 4; ++pr) {
      W[c][2 * pr][0] = o[8 * c + pr][0];
      W[c][2 * pr + 1][0] = o[8 * c + pr][1];
      W[c][2 * pr][1] = o[8 * c + 4 + pr][0];
      W[c][2 * pr + 1][1] = o[8 * c + 4 + pr][1];
    }
}
#undef TRELLIS_A0_OPERANDS
#undef TRELLIS_A0_BLOCK
#undef TRELLIS_A0_ROWS

template <int K>
__device__ __forceinline__ void axis0_body(const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scales,
                                           const uint16_t* __restrict__ x, float* __restrict__ partial,
                                           const Axis0Geom g, const int bid) {
  constexpr int WPB = words_per_block(K);
  constexpr int BLK = WPB * 4;                 // bytes of one block of a row
  constexpr int GSR = BLK / 16 + 1;            // granules per tile row in LDS (one pad granule)
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // the arguments the prologue needs are read together at entry (one wait
  // instead of one per first use)
  asm volatile("" : : "s"(codes), "s"(scales), "s"(x), "s"(g.R), "s"(g.M), "s"(g.ncg), "s"(g.S), "s"(g.rps),
               "s"(g.row_bytes), "s"(g.interleave), "s"(g.nwd), "s"(g.nslots), "s"(g.scales16), "s"(g.x16),
               "s"(g.slot_bytes), "s"(g.xt_off), "s"(g.scr_off), "s"(g.prog_off), "s"(g.scr_wave));
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, q = lane >> 4;
  const int M = g.M;
  const int64_t R = g.R, C = g.C;
  // Workgroup order: a row's blocks of 4 consecutive column groups fill
  // exactly k 128-byte lines, and neighbouring groups share the lines
  // between them.  Each unit (quad of column groups, row split) therefore
  // runs its 4 workgroups on one XCD (workgroup b runs on XCD b % 8), so every
  // line is fetched into a single L2.
  const int xcd = (int)((unsigned)bid % kXcds), j = (int)((unsigned)bid / kXcds);
  const int unit = (j >> 2) * kXcds + xcd;
  const int nq = (g.ncg + 3) >> 2;
  if (unit >= nq * g.S) return;
  const int cgi = 4 * (unit % nq) + (j & 3), s = unit / nq;
  if (cgi >= g.ncg) return;
  const int64_t r0 = (int64_t)s * g.rps;
  const int nr = (int)((R - r0 < g.rps) ? R - r0 : g.rps);   // rows of this split (>= 1)
  const int nblk = (nr + 31) >> 5;
  const int NS = g.nslots, nwd = g.nwd;
  constexpr int gsr = GSR;
  constexpr int GQ = 8 * GSR + kQuadPad;       // granules per 8 tile rows
  uint8_t* ring = smem + (size_t)wave * NS * g.slot_bytes;
  uint16_t* xt = reinterpret_cast<uint16_t*>(smem + g.xt_off);        // f16 [8][rps]: hi n, lo n
  uint8_t* scr = smem + g.scr_off + (size_t)wave * g.scr_wave;        // this wave's staging, then its D tiles
  // progress of the two waves of a SIMD (w and w ^ 4): the one ahead yields
  const uint32_t prog_mine = lds_addr(smem + g.prog_off) + (uint32_t)wave * 4u;
  const uint32_t prog_other = lds_addr(smem + g.prog_off) + (uint32_t)(wave ^ 4) * 4u;
  lds_write_b32(prog_mine, 0u);

  // ---- 1. x~ staging: lane (t, g) of the wave will hold rows 8g .. 8g+7 of
  // its t-th block.  When x and scales are 16-byte aligned and the wave's
  // rows are whole, the copy engine brings its x and scale granules into the
  // wave's scratch first, ahead of the first tiles, so only they are waited
  // for; otherwise plain loads (which then wait behind the tiles).
  const int nmy = nblk > wave ? (nblk - 1 - wave) / kWaves + 1 : 0;   // this wave's 32-row blocks
  const int tb = lane >> 2, g8 = lane & 3;
  const bool hold = tb < nmy;
  const int rl = (wave + kWaves * tb) * 32 + 8 * g8;   // first row of the lane's eight, in the split
  const bool fast = g.x16 && g.scales16 && nmy > 0 && (wave + kWaves * (nmy - 1)) * 32 + 32 <= nr;
  uint8_t* stg = scr;                          // 1 KB each: x[0 .. M-1], then the scales
  if (fast) {
#pragma unroll
    for (int c = 0; c < 5; ++c) {
      if (c < M || c == 4) {                   // lane 0 holds rows of the wave's first block: active
        const uint16_t* src = c < 4 ? x + (int64_t)c * R + r0 + rl : scales + r0 + rl;
        if (hold) __builtin_amdgcn_global_load_lds(src, stg + (c < 4 ? c : M) * 1024, 16, 0, 0);
      }
    }
  }

  // ---- 2. copy descriptors: tile granule p = 64 j + lane lies in group p / gq
  // of 8 rows; within it, granule c = rem % gsr of row rem / gsr (rem = p % gq;
  // the last granule of a row and the group's last kQuadPad granules are
  // pad).  Then the first tiles.
  uint32_t dd[kMaxDma];                       // active bit | byte offset from the tile's first row
#pragma unroll
  for (int j = 0; j < kMaxDma; ++j) {
    const int p = j * 64 + lane;
    const int g8 = p / GQ, rem = p - g8 * GQ;
    const int rr = 8 * g8 + rem / gsr, gg = rem % gsr;
    dd[j] = (j < nwd && g8 < 4 && rem < 8 * gsr && gg < gsr - 1)
                ? (1u << 31) | ((uint32_t)rr * (uint32_t)g.row_bytes + (uint32_t)(gg * 16)) : 0u;
  }
  // this column group's block of row 0; rows follow at g.row_bytes
  const uint8_t* cb = reinterpret_cast<const uint8_t*>(codes) +
                      (g.interleave ? ((int64_t)(cgi >> 1) * R * 2 + (cgi & 1)) * BLK : (int64_t)cgi * BLK);
  // The tiles go through a buffer resource per tile (rows past R fall outside
  // it and read as zeros; their x~ is zero): buffer copies count only against
  // vmcnt, so the LDS reads of the loop, which wait for lgkmcnt(0), do not
  // wait for the tiles still in flight (global-address copies would count
  // against both).
  auto issue_tile = [&](int t) {             // t-th block of this wave
    const int64_t rowb = r0 + (int64_t)(wave + kWaves * t) * 32;
    const int64_t left = R - rowb;
    const int nbytes = (int)((left < 32 ? left : 32) * g.row_bytes);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(cb + rowb * g.row_bytes), (short)0, nbytes, kRawBufferWord3);
    uint8_t* slot = ring + (size_t)(t % NS) * g.slot_bytes;
#pragma unroll
    for (int j = 0; j < kMaxDma; ++j) {
      if (j < nwd) {                           // every issued copy has an active lane
        const uint32_t d = dd[j];
        if (d >> 31)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(slot + (size_t)j * 1024),
                                                   16, (int)(d & 0x7FFFFFFFu), 0, 0, 0);
      }
    }
  };

  // ---- 3. x~[n, r] = scale[r] * x[n, r] (exact in f32) for this wave's rows,
  // eight per lane as staged above.  The wave's largest |x~[n]| * 2^e lands in
  // [2^14, 2^15); x~ 2^e is split into f16 hi and lo halves in xt, and the
  // wave's partial sums are scaled back by 2^-e at the end.
  float xv[4][8];
  uint32_t mx0 = 0u, mx1 = 0u, mx2 = 0u, mx3 = 0u;
  int next0 = 0;
  {
    // Tile 0 streams while x is prepared.  Only one wave of each SIMD pair
    // (w < 4) puts its tile into the launch's first HBM burst, which every
    // workgroup shares: the smaller burst lands sooner, and that wave keeps
    // the SIMD busy while its partner's tile follows once x has landed.
    // (More tiles in the burst would delay it further.)
    for (; next0 < min(nmy, wave < 4 ? 1 : 0); ++next0) issue_tile(next0);
    uint4 xb[4];
    uint16_t sb[8];
    if (fast) {
      wait_vmcnt(nwd * next0);                 // the x and scale copies have landed
      uint32_t sa[5];
#pragma unroll
      for (int c = 0; c < 5; ++c) sa[c] = lds_addr(stg) + (uint32_t)((c < 4 ? (c < M ? c : 0) : M) * 1024 + lane * 16);
      lds_u32x4 sv[5];
      lds_read_b128x5(sa, sv);                 // lanes without copies read stale bytes, masked here
#pragma unroll
      for (int n = 0; n < 4; ++n)
        xb[n] = (hold && n < M) ? make_uint4(sv[n][0], sv[n][1], sv[n][2], sv[n][3]) : make_uint4(0u, 0u, 0u, 0u);
      const uint4 v = hold ? make_uint4(sv[4][0], sv[4][1], sv[4][2], sv[4][3]) : make_uint4(0u, 0u, 0u, 0u);
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int h = 0; h < 8; ++h) sb[h] = (uint16_t)(w4[h >> 1] >> (16 * (h & 1)));
    } else {
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        uint32_t w4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int h = 0; h < 8; ++h)
          if (hold && n < M && rl + h < nr) w4[h >> 1] |= (uint32_t)x[(int64_t)n * R + r0 + rl + h] << (16 * (h & 1));
        xb[n] = make_uint4(w4[0], w4[1], w4[2], w4[3]);
      }
#pragma unroll
      for (int h = 0; h < 8; ++h) sb[h] = (hold && rl + h < nr) ? scales[r0 + rl + h] : (uint16_t)0;
    }
    for (; next0 < min(nmy, 1); ++next0) issue_tile(next0);   // waves 4-7: tile 0 now
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const uint32_t w4[4] = {xb[n].x, xb[n].y, xb[n].z, xb[n].w};
      uint32_t m = 0u;
#pragma unroll
      for (int h = 0; h < 8; ++h) {
        xv[n][h] = bf16_bits_to_f32((w4[h >> 1] >> (16 * (h & 1))) & 0xFFFFu) * half_bits_to_f32(sb[h]);
        m = max(m, __float_as_uint(xv[n][h]) & 0x7FFFFFFFu);
      }
      if (n == 0) mx0 = m;
      if (n == 1) mx1 = m;
      if (n == 2) mx2 = m;
      if (n == 3) mx3 = m;
    }
  }
  mx0 = wave_max_u32(mx0);
  mx1 = wave_max_u32(mx1);
  mx2 = wave_max_u32(mx2);
  mx3 = wave_max_u32(mx3);
  auto exponent = [](uint32_t v) {
    int e = 0;
    if (v != 0u && v < 0x7F800000u) {          // finite, non-zero maximum
      int ex;
      frexpf(__uint_as_float(v), &ex);         // max in [2^(ex-1), 2^ex)
      e = 15 - ex;
    }
    return e;
  };
  const int e0 = exponent(mx0), e1 = exponent(mx1), e2 = exponent(mx2), e3 = exponent(mx3);
  if (hold) {
    const int ev[4] = {e0, e1, e2, e3};
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int h = 0; h < 8; h += 2) {
        const float v0 = ldexpf(xv[n][h], ev[n]), v1 = ldexpf(xv[n][h + 1], ev[n]);
        hw[h >> 1] = pack_f16x2(v0, v1);
        const half2v hp = __builtin_bit_cast(half2v, hw[h >> 1]);
        const _Float16 h0 = hp[0], h1 = hp[1];                 // by value
        lw[h >> 1] = pack_f16x2(v0 - (float)h0, v1 - (float)h1);
      }
      lds_write_b128(lds_addr(xt + n * g.rps + rl), lds_u32x4{hw[0], hw[1], hw[2], hw[3]});
      lds_write_b128(lds_addr(xt + (4 + n) * g.rps + rl), lds_u32x4{lw[0], lw[1], lw[2], lw[3]});
    }
  }

  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  int next = next0;
  for (; next < min(nmy, 2); ++next) issue_tile(next);    // tile 1; then one tile ahead (below)

  // ---- 4. per-lane decode geometry for the four chunks: the 32-bit window
  // of columns 4i .. 4i+3 starts at bit (252 - t) k of the block (t = the
  // chunk offset + 4i), in words wi and wn (wrapping within the block)
  int wia[kChunks], wna[kChunks], offa[kChunks];
#pragma unroll
  for (int ch = 0; ch < kChunks; ++ch) {
    const int t = ch * 64 + 4 * i;
    const int p0 = (252 - t) * K;
    wia[ch] = p0 >> 5;
    wna[ch] = (wia[ch] + 1 == WPB) ? 0 : wia[ch] + 1;
    offa[ch] = p0 & 31;
  }
  // B of a 32-row block: lane (n', q) holds xt[n'][8q .. 8q+7] (n' < 8), zero otherwise
  auto b_addr = [&](int blk) { return lds_addr(xt + (i < 8 ? i : 0) * g.rps + blk * 32 + 8 * q); };
  auto b_operand = [&](lds_u32x4 v) {
    return i < 8 ? __builtin_bit_cast(half8, v) : half8{0, 0, 0, 0, 0, 0, 0, 0};
  };

  const int my_e = i == 0 ? e0 : i == 1 ? e1 : i == 2 ? e2 : e3;   // partial-sum scale of column n = i
  f32x4 acc[kChunks][4];
#pragma unroll
  for (int ch = 0; ch < kChunks; ++ch)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[ch][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint32_t mul = kMul;
  const uint64_t add64 = kAdd;
  for (int t = 0; t < nmy; ++t) {
    wait_vmcnt(nwd * (next - 1 - t));          // tile t has landed
    const int blk = wave + kWaves * t;
    half8 Bv;
    const uint8_t* tile = ring + (size_t)(t % NS) * g.slot_bytes + (size_t)q * GQ * 16;
    // 8 rows x 4 columns: windows, then 1MAD words, then row-paired codes
    auto decode_chunk = [&](int ch, const uint32_t (&W)[8][2]) {
      uint32_t st[8][4];
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        const uint32_t v = __builtin_amdgcn_alignbit(W[rr][1], W[rr][0], offa[ch]);
#pragma unroll
        for (int j = 0; j < 4; ++j) st[rr][j] = __builtin_amdgcn_ubfe(v, (3 - j) * K, kL);
      }
      uint32_t xw[8][4];
#pragma unroll
      for (int rr = 0; rr < 8; ++rr)
#pragma unroll
        for (int j = 0; j < 4; ++j) xw[rr][j] = onemad_word_mad64(st[rr][j], mul, add64);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 A;
#pragma unroll
        for (int e = 0; e < 4; ++e) A[e] = code_pair_y(xw[2 * e][j], xw[2 * e + 1][j]);
        acc[ch][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, A), Bv, acc[ch][j], 0, 0, 0);
      }
    };
    // two chunks per read block (the first also brings this block's B)
    const uint32_t ta = lds_addr(tile), ab = b_addr(blk);
#pragma unroll
    for (int ch = 0; ch < kChunks; ch += 2) {
      const uint32_t a0[2] = {ta + (uint32_t)wia[ch] * 4u, ta + (uint32_t)wia[ch + 1] * 4u};
      const uint32_t a1[2] = {ta + (uint32_t)wna[ch] * 4u, ta + (uint32_t)wna[ch + 1] * 4u};
      uint32_t W[2][8][2];
      lds_u32x4 bv;
      uint32_t other_v;
      lds_read_chunks2<K>(a0, a1, ab, W, bv, prog_other, other_v);
      if (ch == 0) {
        Bv = b_operand(bv);
        // the two waves of a SIMD (w, w ^ 4) share its VALU: the one that has
        // finished more blocks drops to the lower issue priority (on a tie
        // the younger wave takes the higher one: the hardware favours the
        // older); the partner's count comes with the first read block
        const uint32_t other = (uint32_t)__builtin_amdgcn_readfirstlane((int)other_v);
        if ((uint32_t)t < other || ((uint32_t)t == other && wave >= 4)) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
      } else {
        asm volatile("" : : "v"(other_v));     // (not needed for the second read block)
      }
      if (ch == kChunks - 2) {
        // the tile's last words are in registers: its slot may be refilled
        // now, ahead of the decode (tile t + 2, one tile ahead of the next
        // block)
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (next < nmy && next <= t + 2) issue_tile(next++);
      }
      decode_chunk(ch, W[0]);
      decode_chunk(ch + 1, W[1]);
    }
    lds_write_b32(prog_mine, (uint32_t)t + 1u);
  }

  // ---- 5. hi + lo into LDS; the waves' tiles are added in a
  // fixed order and scaled by 1 / d * 2^-e_n into the partial of this split
  float* red = reinterpret_cast<float*>(scr);  // f32 [M][kCols] of this wave, scr_wave bytes apart
#pragma unroll
  for (int ch = 0; ch < kChunks; ++ch)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 d = acc[ch][j];
      f32x4 tot;
#pragma unroll
      for (int e = 0; e < 4; ++e) {            // lane n (< 4) adds lane n + 4 (the lo column)
        const float de = d[e];                 // by value: bit casts of vector-element lvalues read element 0
        tot[e] = de + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(de), 0x104, 0xF, 0xF, false));
      }
      if (i < M) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col = ch * 64 + 4 * (4 * q + e) + j;   // MFMA row 4q + e of chunk ch, MFMA j
          red[i * kCols + col] = ldexpf(tot[e], -my_e);   // exact: common units
        }
      }
    }
  lds_barrier();
  for (int idx = tid; idx < M * kCols; idx += kThreads) {
    const int n = idx / kCols, col = idx - n * kCols;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      v += reinterpret_cast<const float*>(smem + g.scr_off + (size_t)w * g.scr_wave)[n * kCols + col];
    partial[((int64_t)s * M + n) * C + (int64_t)cgi * kCols + col] = v * kRcp;
  }
}

// Host geometry; false if the shape does not fit.
bool axis0_geom(int64_t R, int64_t C, int M, int k, Axis0Geom& g) {
  if (M < 1 || M > 4 || C % kCols != 0) return false;
  const int blk = 256 * k / 8;
  g.R = R;
  g.C = C;
  g.M = M;
  g.ncg = (int)(C / kCols);
  int S = device_cus() / g.ncg;
  if (S < 1) S = 1;
  int64_t rps = (R + S - 1) / S;
  rps = (rps + 31) / 32 * 32;
  if (rps > kMaxRowsPerSplit) rps = kMaxRowsPerSplit;
  g.rps = (int)rps;
  g.S = (int)((R + rps - 1) / rps);
  g.row_bytes = C * k / 8;
  g.interleave = 0;
  g.gsr = blk / 16 + 1;
  g.gq = 8 * g.gsr + kQuadPad;
  g.nwd = (4 * g.gq + 63) / 64;
  if (g.nwd > kMaxDma) return false;
  g.slot_bytes = (uint32_t)((4 * g.gq * 16 + 255) / 256 * 256);
  const size_t xt = (size_t)8 * g.rps * 2;
  // per wave: its x and scale staging ((M + 1) KB), later its D tiles (M KB)
  g.scr_wave = (uint32_t)((size_t)(M + 1) * 1024);
  const size_t scr = (size_t)kWaves * g.scr_wave;
  const size_t fixed = ((xt + 255) / 256 + (scr + 255) / 256) * 256 + kProgBytes;
  if (fixed >= kLdsBudget) return false;
  size_t ns = (kLdsBudget - fixed) / ((size_t)kWaves * g.slot_bytes);
  if (ns > (size_t)kMaxSlots) ns = kMaxSlots;
  if (ns < 2) return false;
  g.nslots = (int)ns;
  g.xt_off = (uint32_t)kWaves * g.nslots * g.slot_bytes;
  g.scr_off = g.xt_off + (uint32_t)((xt + 255) / 256 * 256);
  g.prog_off = g.scr_off + (uint32_t)((scr + 255) / 256 * 256);
  g.total = g.prog_off + kProgBytes;
  g.scales16 = 0;
  g.x16 = 0;
  return g.total <= kLdsBudget;
}

}  // namespace a0
using namespace a0;
}  // namespace
}  // namespace trellis
