// prefill.hip -- fused axis-1 prefill on gfx950: packed codes are decoded
// into an LDS tile of bf16 weights that feeds bf16 MFMA directly, so no
// expanded weight matrix ever exists in HBM.
//
// out[m, r] = bf16( sum_c wb(r, c) * x[m, c] ),  wb = bf16(f32(value * scale))
// Source: mlx-bun 0.2.0 -> 0.4.0 diff (page 56), trellis-tiled-prefill.ts
// (x tile and reconstructed bf16 weight tile in threadgroup memory, matrix
// multiply-accumulate in f32; precise value before the bf16 weight rounding).
//
// Tiling.  A workgroup of 4 waves (one per SIMD) owns 512 rows of x and 128
// weight rows; each wave computes a 128 (x rows) x 128 (weight rows) block
// as 4 x 4 v_mfma_f32_32x32x16_bf16 tiles with 256 f32 accumulators per
// lane (the 32 x 32 form keeps each accumulator in place across the loop).
// Every decoded weight therefore serves 512 rows of x, which keeps the VALU
// decode (about nine operations per weight) under the MFMA time of a step.
// For M <= 256 the workgroup owns 128 rows of x instead (32 per wave, one
// MFMA tile along x, 64 accumulators), two workgroups share a CU, and the
// decode is the cost: a 512-row tile would spend most of its MFMA work on
// rows past M.
//
// x path.  Each wave's 128 rows of x are its own, so x needs no LDS: a
// first pass (prefill_xlayout_kernel) writes x once in the MFMA operand
// order, one 1 KB fragment per (32 rows, step, half step), and the main
// kernel loads every fragment it needs with one 16-byte load per lane, two
// steps' worth in a register ring.  LDS holds only the decoded weight tile,
// which all four waves share.
//
// Per step of 32 columns:
//   * each thread decodes 16 consecutive positions of one weight row for the
//     next step, between this step's MFMAs, into the other half of a
//     double-buffered LDS weight tile; its code words are loaded three
//     steps ahead;
//   * the x fragments of the next step are loaded during this one: half 0
//     at the start, half 1 once the previous step's half 1 has gone into the
//     MFMAs (it frees those registers);
//   * one workgroup barrier per step (for the weight tile), straddled by the
//     MFMAs: the interval between two barriers runs the second half of the
//     previous step from registers and then the first half of this step, so
//     the matrix core has work while the new step's operands leave LDS.
// Workgroups are mapped so that the 32 CUs of one XCD work on the same 512
// rows of x at the same time, which keeps that slice of x in the XCD's L2.
//
// Axis 0 (a matrix stored transposed, codes W^T [R_in, C_out k / 32], the
// down projection): the same kernel with the outputs C_out as the tile's
// weight rows and the stored rows R_in as the contraction.  A step is 32
// stored rows; each thread decodes 16 consecutive positions (output columns)
// of one stored row, the same 16 positions of the same block in every step,
// and writes them transposed into the weight tile (one 2-byte LDS write per
// weight).  The tile's 8-element chunks are swizzled per group of 16 rows so
// that those writes, and the 16-byte operand reads, spread over the banks.
#include <algorithm>
#include <type_traits>

#include "internal.hpp"
#include "mfma_common.hpp"
#include "trellis_device.hpp"

namespace trellis {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 4;
constexpr int kBMLarge = 512;            // x rows per workgroup, M > 256
constexpr int kBMSmall = 128;            // x rows per workgroup, M <= 256
constexpr int kBN = 128;                 // weight rows per workgroup
constexpr int kBK = 32;                  // columns per step
constexpr int kFN = kBN / 32;            // MFMA tiles along weight rows
constexpr int kRow = kBK + 8;            // padded LDS row (bf16): 80 bytes spread the 16-byte reads
constexpr int kFrag = 1024;              // bytes of one x operand fragment (64 lanes x 16 bytes)
constexpr int kXcds = 8;
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format

// Words holding the windows of 16 consecutive positions once the run is
// aligned to bit 0; odd k starts half the runs 16 bits into a word, so one
// more word is loaded and the run is shifted down.
template <int K>
struct Run16 {
  static constexpr int kAligned = (15 * K + kL + 31) / 32;
  static constexpr int kLoad = kAligned + (K & 1);
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two round-to-nearest-even bf16 conversions in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Decode positions q0 + 8 H .. q0 + 8 H + 7 of a run of 16 consecutive
// positions q0 .. q0 + 15 of one row (half H of the run).  Position q0 + i
// has its window at bit (15 - i) * K of the aligned run (the block stores
// position t at bit (T - 1 - t) * K, so later positions sit lower).
template <int K, int H>
__device__ __forceinline__ void decode_run8(const uint32_t (&w)[Run16<K>::kLoad], bool shift16,
                                           float sc, uint32_t mul, uint64_t add64,
                                           uint32_t (&pk)[4]) {
  constexpr int NA = Run16<K>::kAligned;
  uint32_t a[NA];
#pragma unroll
  for (int j = 0; j < NA; ++j) {
    if constexpr (K & 1)
      a[j] = shift16 ? __builtin_amdgcn_alignbit(w[j + 1], w[j], 16) : w[j];
    else
      a[j] = w[j];
  }
  float f[8];
#pragma unroll
  for (int ii = 0; ii < 8; ++ii) {
    const int rel = (15 - (8 * H + ii)) * K;
    const int wi = rel >> 5, ro = rel & 31;
    uint32_t s;
    if (ro + kL <= 32)
      s = (a[wi] >> ro) & kStateMask;
    else
      s = window(a[wi], a[wi + 1], (uint32_t)ro);
    // y = byte sum - 510: v_sad_u8 accumulates onto -510 (mod 2^32)
    const int y = (int)__builtin_amdgcn_sad_u8(onemad_word_mad64(s, mul, add64), 0u, (uint32_t)-kYOffset);
    f[ii] = code_value(y) * sc;
  }
#pragma unroll
  for (int p = 0; p < 4; ++p) pk[p] = pack_bf16x2(f[2 * p], f[2 * p + 1]);
}

// Work plan, in one of two modes.
//  * Rounds (stream == 0): the first nfull tiles run whole, in the XCD-aware
//    order below.  When the tiles left after the full rounds would fill at
//    most half of the CUs, each of those nsplit tiles is cut instead into S
//    segments of seg steps (a multiple of 4), one workgroup each, which leave
//    f32 partial tiles in slots unit = (tile - nfull) * S + segment.
//  * Stream (stream == 1, when the leftover tiles would fill more than half
//    of the CUs): the ntiles * nsteps steps are dealt out as G contiguous
//    ranges of U steps (U a multiple of 4), one persistent workgroup each.
//    A range crosses tile boundaries; whole tiles inside it are stored
//    directly, the piece of a tile at its start goes to slot 2 g and the
//    piece at its end to slot 2 g + 1.
// prefill_fold_kernel adds up the partial tiles of every split tile.
struct PrefillPlan {
  int nn;            // tiles along the weight rows
  int ntiles, nsteps;
  int stream;
  int nfull, per;    // rounds: whole tiles; per XCD
  int nsplit, S, seg;
  int U, G;          // stream: steps per workgroup, workgroups
  int il;            // axis 0: codes in the block-interleaved k = 3 layout [R/512, C, 48]
};

// Shapes that follow from the x rows BM of a workgroup tile.
template <int BM>
struct XTile {
  static constexpr int kWM = BM / kWaves;            // x rows per wave
  static constexpr int kFM = kWM / 32;               // MFMA tiles along x rows
  static constexpr int kPartFloats = BM * kBN;       // one partial tile (float4-interleaved per thread)
  static constexpr int kG4 = kFM * kFN * 4;          // float4 groups of one thread's accumulators
  static constexpr int kOcc = BM == kBMSmall ? 2 : 1;  // workgroups per CU (registers allow two at 128 rows)
};

// x rows per workgroup tile: M <= 256 takes 128-row tiles (a 512-row tile
// would spend half or more of its MFMA work on rows past M; measured
// crossover: 128-row tiles win at M = 256, lose at M = 512, where the decode
// they repeat per row tile costs more than the MFMA work they save).
constexpr int kSmallTileMaxM = 256;
int tile_rows(int64_t M) { return M <= kSmallTileMaxM ? kBMSmall : kBMLarge; }

// R: outputs per row of x (weight rows of the tile, the row stride of out);
// C: contraction length (columns of x).  Axis 1: codes [R, C k / 32].  Axis
// 0 (A0): codes [C, R k / 32], scales [C].
template <int K, int BM, bool A0>
__global__ __launch_bounds__(256, XTile<BM>::kOcc) void prefill_fused_kernel(
    const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ xf, uint16_t* __restrict__ out, float* __restrict__ part, int R,
    int C, int M, PrefillPlan plan) {
  constexpr int kBM = BM, kWM = XTile<BM>::kWM, kFM = XTile<BM>::kFM;
  constexpr int kPartFloats = XTile<BM>::kPartFloats;
  constexpr int WPB = words_per_block(K);
  constexpr int NL = Run16<K>::kLoad;
  // Separate LDS objects for the two weight tiles, so the compiler knows a
  // step's writes (the next tile) never alias its reads and can move the
  // decode in between the MFMAs.
  __shared__ __attribute__((aligned(16))) uint16_t Bs0[kBN * kRow];
  __shared__ __attribute__((aligned(16))) uint16_t Bs1[kBN * kRow];

  const int nsteps = C / kBK;

  // One piece: steps [t_begin, t_end) of `tile` (t_begin a multiple of 4);
  // its accumulators go to partial slot `unit`, or to out when unit < 0.
  auto piece = [&](const int tile, const int t_begin, const int t_end, const int unit) {
  const int mb = tile / plan.nn, nb = tile - mb * plan.nn;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: offsets stay in SGPRs
  const int m_wave = mb * kBM + wave * kWM;
  const int n0 = nb * kBN;

  // x fragments: fragment (b, t, h) of 32-row block b, step t and half h
  // sits at byte ((b * nsteps + t) * 2 + h) * kFrag of xf, lane l's 16 bytes
  // at l * 16 (row 32 b + l % 32, columns 16 (l / 32) + 8 h .. + 7 of the
  // step).  Blocks past the last row of x re-read the last block (their
  // results are never stored).
  const int nblk = (M + 31) / 32;
  const __amdgpu_buffer_rsrc_t xr =
      __builtin_amdgcn_make_buffer_rsrc((void*)xf, (short)0, nblk * nsteps * 2 * kFrag, kRsrcWord3);
  uint32_t xvo[kFM];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
    xvo[i] = (uint32_t)min(m_wave / 32 + i, nblk - 1) * (uint32_t)(nsteps * 2 * kFrag) + (uint32_t)lane * 16u;

  // Decode assignment.  Axis 1: weight row n0 + dr (clamped), positions
  // 16 dh .. + 15 of every step; dh is uniform over a wave.  Axis 0: stored
  // row 32 t + sr in step t, positions q0 .. q0 + 15 of block n0 / 256 (the
  // tile's columns 16 pg .. + 15) in every step.
  const int dr = lane + 64 * (wave >> 1), dh = wave & 1;
  const int sr = tid >> 3, pg = tid & 7;
  const int grow = min(n0 + dr, R - 1);
  const int row_bytes = ((A0 ? R : C) / kT) * WPB * 4;
  const __amdgpu_buffer_rsrc_t cr =
      __builtin_amdgcn_make_buffer_rsrc((void*)codes, (short)0, (A0 ? C : R) * row_bytes, kRsrcWord3);
  // axis 0: bytes between stored rows within the tile's block, and the
  // block's first byte (row-major: rows of R / 256 blocks; interleaved: block
  // pairs [R / 512][C][2 blocks], so a block's rows are 2 blocks apart)
  const int rstride = (A0 && plan.il) ? 2 * WPB * 4 : row_bytes;
  const int nblk0 = n0 / kT;
  const int bbase = (A0 && plan.il) ? ((nblk0 >> 1) * C * 2 + (nblk0 & 1)) * WPB * 4 : nblk0 * WPB * 4;
  const int cvo = grow * row_bytes;
  float sc = 0.f;
  if constexpr (!A0) sc = half_bits_to_f32(scales[grow]);
  const uint32_t mul = kMul;
  const uint64_t add64 = kAdd;
  // axis 0: the run's word offsets in its stored row (words wrap within the
  // block) and whether it starts 16 bits into a word; fixed for the piece
  uint32_t avo[NL];
  bool a0_shift = false;
  if constexpr (A0) {
    const int q0 = (n0 & (kT - 1)) + 16 * pg;
    const int rb = (kT - 16 - q0) * K;
    a0_shift = (rb & 31) != 0;
    const int w0 = rb >> 5;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int wj = (w0 + j >= WPB) ? w0 + j - WPB : w0 + j;
      avo[j] = (uint32_t)(sr * rstride + bbase + wj * 4);
    }
  }

  f32x16 acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j) acc[i][j] = f32x16{};

  // x operand ring: xh[h][slot][i] holds half h of the step with parity slot
  u32x4 xh[2][2][kFM];
  uint32_t cw[4][NL];       // code words of steps t + 1 .. t + 3
  uint32_t scw[4] = {0u, 0u, 0u, 0u};   // axis 0: fp16 scale bits of those steps' stored rows

  // Loads past the end re-read the last step (in bounds, unused), so the
  // loop body has no branches.
  auto load_x = [&](int t, int h, u32x4 (&dst)[kFM]) {
    const int soff = (min(t, nsteps - 1) * 2 + h) * kFrag;
#pragma unroll
    for (int i = 0; i < kFM; ++i) dst[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)xvo[i], soff, 0);
  };
  // Run of step t: block t / 8, first position q0 = 32 (t % 8) + 16 dh,
  // lowest window bit (240 - q0) K; words wrap within the block.
  auto run_bits = [&](int t) { return (kT - 16 - (kBK * (t & 7) + 16 * dh)) * K; };
  auto load_w = [&](uint32_t (&dst)[NL], uint32_t& sdst, int t) {
    t = min(t, nsteps - 1);
    if constexpr (A0) {
      const int so = t * kBK * rstride;          // stored row 32 t
#pragma unroll
      for (int j = 0; j < NL; ++j) dst[j] = __builtin_amdgcn_raw_buffer_load_b32(cr, (int)avo[j], so, 0);
      sdst = scales[t * kBK + sr];
    } else {
      const int w0 = run_bits(t) >> 5;
      const int base = (t >> 3) * WPB * 4;
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int wj = (w0 + j >= WPB) ? w0 + j - WPB : w0 + j;
        dst[j] = __builtin_amdgcn_raw_buffer_load_b32(cr, cvo, base + wj * 4, 0);
      }
    }
  };
  // Half H of the weights of step t (16 bytes per thread) into an LDS
  // buffer (past the last step: a buffer nobody reads again).
  auto decode_half = [&](const uint32_t (&w)[NL], uint32_t sbits, int t, uint32_t (&pk)[4], auto half) {
    if constexpr (A0)
      decode_run8<K, decltype(half)::value>(w, a0_shift, half_bits_to_f32((uint16_t)sbits), mul, add64, pk);
    else
      decode_run8<K, decltype(half)::value>(w, (run_bits(t) & 31) != 0, sc, mul, add64, pk);
  };
  // Axis 0: weight (tile row c, contraction index s) sits in 8-element chunk
  // (s / 8) ^ ((c / 16) % 4) of LDS row c; here c = 16 pg + 8 half + e.
  auto store_half = [&](const uint32_t (&pk)[4], uint16_t* buf, int half) {
    if constexpr (A0) {
      uint16_t* p = buf + (16 * pg + 8 * half) * kRow + 8 * ((sr >> 3) ^ (pg & 3)) + (sr & 7);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[(2 * e) * kRow] = (uint16_t)pk[e];
        p[(2 * e + 1) * kRow] = (uint16_t)(pk[e] >> 16);
      }
    } else {
      *reinterpret_cast<u32x4*>(&buf[dr * kRow + 16 * dh + 8 * half]) = u32x4{pk[0], pk[1], pk[2], pk[3]};
    }
  };
  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, 1>;

  // prologue (t_begin is a multiple of 4): words of the first three steps,
  // x of the first step, weights of the first step
  load_w(cw[0], scw[0], t_begin);
  load_w(cw[1], scw[1], t_begin + 1);
  load_w(cw[2], scw[2], t_begin + 2);
  load_x(t_begin, 0, xh[0][0]);
  load_x(t_begin, 1, xh[1][0]);
  {
    uint32_t pk[4];
    decode_half(cw[0], scw[0], t_begin, pk, H0{});
    store_half(pk, Bs0, 0);
    decode_half(cw[0], scw[0], t_begin, pk, H1{});
    store_half(pk, Bs0, 1);
  }
  __syncthreads();

  // weight operand of one half h of a step: b[j] holds rows 32 j + l % 32,
  // columns 16 (l / 32) + 8 h .. + 7 (the columns of the x fragments; any
  // assignment shared by both operands is a valid split of the contraction)
  const int bofs = (lane & 31) * kRow + 16 * (lane >> 5);
  // axis 0: logical chunk 2 (l / 32) + h of row 32 j + l % 32 is physical
  // chunk (2 (l / 32) + (l / 16) % 2) ^ (h + 2 (j % 2)); one offset per mask
  int bsw[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) bsw[q] = (lane & 31) * kRow + 8 * ((2 * (lane >> 5) + ((lane >> 4) & 1)) ^ q);
  auto read_b = [&](int h, const uint16_t* bbuf, bf16x8 (&b)[kFN]) {
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      const int off = A0 ? bsw[h + 2 * (j & 1)] : bofs + 8 * h;
      b[j] = *reinterpret_cast<const bf16x8*>(bbuf + off + 32 * j * kRow);
    }
  };
  auto mfma_half = [&](const bf16x8 (&b)[kFN], const u32x4 (&a)[kFM]) {
#pragma unroll
    for (int i = 0; i < kFM; ++i)
#pragma unroll
      for (int j = 0; j < kFN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[j], __builtin_bit_cast(bf16x8, a[i]), acc[i][j], 0, 0, 0);
  };

  // Software pipeline across the per-step barrier.  Interval t (between the
  // barriers of steps t - 1 and t) runs the second half of step t - 1 from
  // registers, then the first half of step t, while it reads the weights of
  // step t from LDS and decodes step t + 1.  After each barrier the wave has
  // MFMA work whose operands are already in registers, so the matrix core
  // does not wait for the LDS reads of the new step.
  bf16x8 bp[kFN];              // weights, second half of the previous step
  bf16x8 bc[kFN];              // weights, first half of the current step
#pragma unroll
  for (int j = 0; j < kFN; ++j) bp[j] = bf16x8{};
#pragma unroll
  for (int i = 0; i < kFM; ++i) xh[1][1][i] = u32x4{0u, 0u, 0u, 0u};   // "step t_begin - 1": adds zero

  // Four steps per iteration (the step count is a multiple of 8), so every
  // buffer and ring index below is a compile-time constant.
  for (int t0 = t_begin; t0 < t_end; t0 += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + u;
      const int sl = u & 1;                     // ring slot of step t (t0 is even)
      const uint16_t* bcur = (u & 1) ? Bs1 : Bs0;
      uint16_t* bnext = (u & 1) ? Bs0 : Bs1;
      uint32_t pk0[4], pk1[4];

      // first region: loads (words of step t + 3, x of step t + 1 half 0),
      // weights of step t (half 0), MFMAs of step t - 1 (half 1), decode of
      // step t + 1 (half 0)
      load_w(cw[(u + 3) & 3], scw[(u + 3) & 3], t + 3);
      load_x(t + 1, 0, xh[0][sl ^ 1]);
      read_b(0, bcur, bc);
      mfma_half(bp, xh[1][sl ^ 1]);
      decode_half(cw[(u + 1) & 3], scw[(u + 1) & 3], t + 1, pk0, H0{});
      __builtin_amdgcn_sched_group_barrier(0x020, kFM + NL + (A0 ? 1 : 0), 0);    // VMEM reads
      __builtin_amdgcn_sched_group_barrier(0x100, kFN, 0);                        // DS reads
#pragma unroll
      for (int g = 0; g < kFM * kFN; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                         // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);                         // VALU
      }
      __builtin_amdgcn_sched_barrier(0);

      // second region: x of step t + 1 half 1 (into the registers the MFMAs
      // above have read), weights of step t (half 1), MFMAs of step t (half
      // 0), decode of step t + 1 (half 1), LDS writes
      load_x(t + 1, 1, xh[1][sl ^ 1]);
      read_b(1, bcur, bp);
      mfma_half(bc, xh[0][sl]);
      decode_half(cw[(u + 1) & 3], scw[(u + 1) & 3], t + 1, pk1, H1{});
      store_half(pk0, bnext, 0);
      store_half(pk1, bnext, 1);
      __builtin_amdgcn_sched_group_barrier(0x020, kFM, 0);                        // VMEM reads
      __builtin_amdgcn_sched_group_barrier(0x100, kFN, 0);                        // DS reads
#pragma unroll
      for (int g = 0; g < kFM * kFN; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                         // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);                         // VALU
      }
      __builtin_amdgcn_sched_group_barrier(0x200, A0 ? 16 : 2, 0);                // DS writes
      __syncthreads();
      // MFMAs touch no memory, so without a fence the scheduler would move
      // them across the barrier.
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  mfma_half(bp, xh[1][1]);     // second half of the last step (t_end - 1 is odd: slot 1)

  if (unit >= 0) {
    // Split segment: the accumulators go to partial tile `unit`, float4 g4
    // (16 per MFMA tile (i, j)) of thread tid at float4 index g4 * 256 + tid.
    // Rows past M are neither stored nor folded.
    float4* dst = reinterpret_cast<float4*>(part) + (size_t)unit * (kPartFloats / 4);
#pragma unroll
    for (int i = 0; i < kFM; ++i) {
      if (m_wave + 32 * i + (lane & 31) >= M) continue;
#pragma unroll
      for (int j = 0; j < kFN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16 v = acc[i][j];
          dst[((i * kFN + j) * 4 + g) * 256 + tid] = make_float4(v[4 * g], v[4 * g + 1], v[4 * g + 2], v[4 * g + 3]);
        }
    }
    return;
  }

  // D of tile (i, j) (weights as the row operand): lane holds x row
  // m_wave + 32 i + lane % 32 and, for register group g, weight rows
  // n0 + 32 j + 8 g + 4 (lane / 32) + e, e = 0..3.
  if (m_wave >= M) return;
  const bool vec = (R & 3) == 0;
#pragma unroll
  for (int i = 0; i < kFM; ++i) {
    const int m = m_wave + 32 * i + (lane & 31);
    if (m >= M) continue;
    uint16_t* orow = out + (size_t)m * (size_t)R;
#pragma unroll
    for (int j = 0; j < kFN; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + 32 * j + 8 * g + 4 * (lane >> 5);
        const f32x16 v = acc[i][j];
        if (vec && n + 3 < R) {
          *reinterpret_cast<uint2*>(orow + n) =
              make_uint2(pack_bf16x2(v[4 * g], v[4 * g + 1]), pack_bf16x2(v[4 * g + 2], v[4 * g + 3]));
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < R) orow[n + e] = f32_to_bf16_bits(v[4 * g + e]);
        }
      }
  }
  };

  // Pieces of this workgroup.  Rounds: one (a whole tile in the XCD-aware
  // order -- workgroup b runs on XCD b % 8 and that XCD takes a contiguous
  // range of tiles, which share their 512 x rows -- or one split segment,
  // after all whole tiles).  Stream: the pieces of its range of steps.
  const int bid = blockIdx.x;
  int tile = 0, tb = 0, te = nsteps, unit = -1, pos = 0, start = 0, end = 0;
  if (!plan.stream) {
    if (bid < kXcds * plan.per) {
      tile = (bid % kXcds) * plan.per + bid / kXcds;
      if (tile >= plan.nfull) return;
    } else {
      unit = bid - kXcds * plan.per;               // split unit: tile nfull + unit / S, segment unit % S
      tile = plan.nfull + unit / plan.S;
      tb = (unit % plan.S) * plan.seg;
      te = min(nsteps, tb + plan.seg);
    }
  } else {
    start = bid * plan.U;
    end = min(plan.ntiles * nsteps, start + plan.U);
    pos = start;
  }
  for (;;) {
    if (plan.stream) {
      tile = pos / nsteps;
      tb = pos - tile * nsteps;
      te = min(nsteps, tb + (end - pos));
      unit = (tb == 0 && te == nsteps) ? -1 : 2 * bid + (pos == start ? 0 : 1);
    }
    piece(tile, tb, te, unit);
    if (!plan.stream) break;
    pos += te - tb;
    if (pos >= end) break;
    __syncthreads();                               // the next piece reuses the LDS buffers
  }
}

// x in MFMA operand order for the main kernel: 16-byte unit u of xf is lane
// u % 64 of fragment f = u / 64 = (b * nsteps + t) * 2 + h, i.e. row
// 32 b + u % 32 of x and columns 32 t + 16 ((u % 64) / 32) + 8 h .. + 7 (zero
// past the last row).
__global__ __launch_bounds__(256) void prefill_xlayout_kernel(const uint16_t* __restrict__ x,
                                                              uint4* __restrict__ xf, int M, int C,
                                                              int64_t nunits) {
  const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (u >= nunits) return;
  const int nsteps = C / kBK;
  const int l = (int)(u & 63);
  const int64_t f = u >> 6;
  const int h = (int)(f & 1);
  const int64_t bt = f >> 1;
  const int t = (int)(bt % nsteps), b = (int)(bt / nsteps);
  const int row = 32 * b + (l & 31), col = kBK * t + 16 * (l >> 5) + 8 * h;
  xf[u] = row < M ? *reinterpret_cast<const uint4*>(x + (int64_t)row * C + col) : make_uint4(0u, 0u, 0u, 0u);
}

// Sum the partial tiles of every split tile and store bf16: workgroup
// (tile, float4 group g4), thread tid; the element mapping is the one of the
// main kernel's epilogue.  Rounds: the split tiles are nfull + blockIdx / kG4,
// with slots ts * S .. ts * S + S - 1.  Stream: every tile has a workgroup;
// tile t is split when its steps span the ranges of workgroups ga < gb, and
// its piece of workgroup g sits in slot 2 g (g's first piece) or 2 g + 1 (ga,
// whose range began in an earlier tile).
template <int BM>
__global__ __launch_bounds__(256) void prefill_fold_kernel(const float* __restrict__ part,
                                                           uint16_t* __restrict__ out, int R, int M,
                                                           PrefillPlan plan) {
  constexpr int kWM = XTile<BM>::kWM, kG4 = XTile<BM>::kG4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ts = blockIdx.x / kG4, g4 = blockIdx.x % kG4;
  const float4* base = reinterpret_cast<const float4*>(part) + g4 * 256 + tid;
  constexpr size_t kSlot = XTile<BM>::kPartFloats / 4;
  const int i = g4 / (kFN * 4), j = (g4 / 4) % kFN, g = g4 % 4;
  const int tile = plan.stream ? ts : plan.nfull + ts;
  const int mb = tile / plan.nn, nb = tile - mb * plan.nn;
  const int m = mb * BM + wave * kWM + 32 * i + (lane & 31);
  const int n = nb * kBN + 32 * j + 8 * g + 4 * (lane >> 5);
  if (m >= M) return;                            // rows past M were not stored
  float4 v;
  if (!plan.stream) {
    const float4* src = base + (size_t)ts * plan.S * kSlot;
    v = src[0];
    for (int s = 1; s < plan.S; ++s) {
      const float4 w = src[(size_t)s * kSlot];
      v.x += w.x;
      v.y += w.y;
      v.z += w.z;
      v.w += w.w;
    }
  } else {
    const int ga = tile * plan.nsteps / plan.U, gb = ((tile + 1) * plan.nsteps - 1) / plan.U;
    if (ga == gb) return;                          // whole inside one range: stored by the main kernel
    const int first_of_ga = (ga * plan.U) / plan.nsteps == tile;
    v = base[(size_t)(2 * ga + (first_of_ga ? 0 : 1)) * kSlot];
    for (int gw = ga + 1; gw <= gb; ++gw) {
      const float4 w = base[(size_t)(2 * gw) * kSlot];
      v.x += w.x;
      v.y += w.y;
      v.z += w.z;
      v.w += w.w;
    }
  }
  uint16_t* orow = out + (size_t)m * (size_t)R;
  if ((R & 3) == 0 && n + 3 < R) {
    *reinterpret_cast<uint2*>(orow + n) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
  } else {
    const float e[4] = {v.x, v.y, v.z, v.w};
    for (int q = 0; q < 4; ++q)
      if (n + q < R) orow[n + q] = f32_to_bf16_bits(e[q]);
  }
}

// ---- register-direct prefill for M <= 64 -----------------------------------
//
// With few rows of x the tile kernel above is bound by its decode, and its
// per-step LDS round trip and barrier slow that decode down.  Here each lane
// decodes exactly the weights of its own MFMA operand: for step t (32
// columns) and half h, lane l holds weight row r0 + l % 32, positions
// 16 (l / 32) + 8 h .. + 7 of the step -- the same split of the contraction
// as the x fragments of prefill_xlayout_kernel -- so the 8 bf16 weights go
// straight from the decode into v_mfma_f32_32x32x16_bf16, with no LDS and no
// barrier in the loop.  A workgroup takes 32 weight rows and one of S chunks
// of the columns; its 4 waves split the chunk, meet once in LDS at the end,
// and store bf16 (S == 1) or an f32 partial [S][M][R] that
// prefill_direct_fold_kernel adds up.  Waves are many and independent, so the
// machine stays evenly loaded.  FM x tiles of 32 rows (M <= 64); from 65
// rows on, the tile kernel above shares each decoded weight among more rows.
constexpr int kDirectMaxM = 64;
// Up to this many rows the register-direct kernel reads x in place (no layout
// pass): per eager call at 17408 x 5120, k = 2, 30.0 vs 32.8 us (M = 2), 31.5
// vs 33.1 us (M = 8), 34.3 vs 34.7 us (M = 16), 43.0 vs 34.9 us (M = 32).
constexpr int kDirectXMaxM = 16;

// Two x tiles: registers capped for 4 waves per SIMD (a few spills outside
// the step loop) ran 3-4 % faster than 3 waves per SIMD without spills.
//
// XD: x is read in place (x [M, C] row-major) instead of from the operand-
// order copy, and the layout pass is not launched.  A lane's 16 bytes of a
// fragment are contiguous in its x row either way; in place, one load
// touches a line per row of the tile instead of 8 lines, so it pays only
// for few rows (M <= kDirectXMaxM): rows past M lie outside the buffer
// range and read as zeros without a memory access.
template <int K, int FM, bool XD = false>
__global__ __launch_bounds__(256, FM == 2 ? 4 : 1) void prefill_direct_kernel(
    const uint32_t* __restrict__ codes, const uint16_t* __restrict__ scales,
    const uint16_t* __restrict__ xf, uint16_t* __restrict__ out, float* __restrict__ part, int R, int C,
    int M, int S) {
  static_assert(!XD || FM == 1, "x read in place for one 32-row tile only");
  constexpr int WPB = words_per_block(K);
  constexpr int NL = Run16<K>::kLoad;
  __shared__ __attribute__((aligned(16))) float red[3][FM][16][64];   // waves 1..3's accumulators
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = (int)(blockIdx.x / (unsigned)S), s = (int)(blockIdx.x % (unsigned)S);
  const int r0 = tile * 32;
  const int nsteps = C / kBK;
  const int cs = (int)((int64_t)s * nsteps / S), ce = (int)((int64_t)(s + 1) * nsteps / S);
  const int t_begin = cs + (ce - cs) * wave / 4, t_end = cs + (ce - cs) * (wave + 1) / 4;

  const int row = min(r0 + (lane & 31), R - 1);   // rows past R decode row R - 1 (never stored)
  const int dh = lane >> 5;
  const int row_bytes = (C / kT) * WPB * 4;
  const __amdgpu_buffer_rsrc_t cr =
      __builtin_amdgcn_make_buffer_rsrc((void*)codes, (short)0, R * row_bytes, kRsrcWord3);
  const int cvo = row * row_bytes;
  const float sc = half_bits_to_f32(scales[row]);
  const int nblk = (M + 31) / 32;
  // fragment (tile i, step t, half h), lane u: x row 32 i + u % 32, columns
  // 32 t + 16 (u / 32) + 8 h .. + 7
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)xf, (short)0, XD ? M * C * 2 : nblk * nsteps * 2 * kFrag, kRsrcWord3);
  uint32_t xvo[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i)
    xvo[i] = XD ? (uint32_t)(lane & 31) * (uint32_t)(C * 2) + (uint32_t)dh * 32u
                : (uint32_t)min(i, nblk - 1) * (uint32_t)(nsteps * 2 * kFrag) + lane * 16u;

  auto load_x = [&](u32x4 (&dst)[2][FM], int t) {
    t = min(t, nsteps - 1);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < FM; ++i)
        dst[h][i] = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)xvo[i], XD ? t * 64 + h * 16 : (t * 2 + h) * kFrag,
                                                          0);
  };

  f32x16 acc[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) acc[i] = f32x16{};
  const uint32_t mul = kMul;
  const uint64_t add64 = kAdd;
  // The 8 steps of a block read only that block's WPB words: a lane loads its
  // row's block once, 16 bytes at a time, and takes each step's run from it
  // (word indices fixed per step; the two halves of a step, 16 positions
  // apart, differ by a select on lane / 32).  x of step t + 1 loads while
  // step t decodes.
  u32x4 xv[2][2][FM];
  if (t_begin & 1) load_x(xv[1], t_begin);
  else load_x(xv[0], t_begin);
  for (int blk = t_begin >> 3; blk <= (t_end - 1) >> 3; ++blk) {
    uint32_t W[WPB];
#pragma unroll
    for (int q = 0; q < WPB / 4; ++q) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(cr, cvo, (blk * WPB + 4 * q) * 4, 0);
      W[4 * q] = v[0];
      W[4 * q + 1] = v[1];
      W[4 * q + 2] = v[2];
      W[4 * q + 3] = v[3];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = blk * 8 + j;
      if (t < t_begin || t >= t_end) continue;
      load_x(xv[(j + 1) & 1], t + 1);
      // half-run dh: first position 32 j + 16 dh, lowest window bit (240 - 32 j - 16 dh) K
      const int rb0 = (kT - 16 - kBK * j) * K, rb1 = (kT - 32 - kBK * j) * K;
      uint32_t w[NL];
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int i0 = (rb0 >> 5) + i, i1 = (rb1 >> 5) + i;
        const uint32_t a0 = W[i0 >= WPB ? i0 - WPB : i0], a1 = W[i1 >= WPB ? i1 - WPB : i1];
        w[i] = dh ? a1 : a0;
      }
      const bool sh = dh ? (rb1 & 31) != 0 : (rb0 & 31) != 0;
      uint32_t pk[4];
      decode_run8<K, 0>(w, sh, sc, mul, add64, pk);
#pragma unroll
      for (int i = 0; i < FM; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]}),
                                                        __builtin_bit_cast(bf16x8, xv[j & 1][0][i]), acc[i], 0, 0, 0);
      decode_run8<K, 1>(w, sh, sc, mul, add64, pk);
#pragma unroll
      for (int i = 0; i < FM; ++i)
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]}),
                                                        __builtin_bit_cast(bf16x8, xv[j & 1][1][i]), acc[i], 0, 0, 0);
    }
  }

  // the four waves' sums, added in wave order by wave 0
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) red[wave - 1][i][e][lane] = acc[i][e];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][e] += red[w][i][e][lane];
  // D of tile i: lane holds x row 32 i + lane % 32 and weight rows
  // r0 + 8 g + 4 (lane / 32) + e
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = 32 * i + (lane & 31);
    if (m >= M) continue;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int n = r0 + 8 * g + 4 * dh + e;
        if (n >= R) continue;
        const float v = acc[i][4 * g + e];
        if (S == 1) out[(size_t)m * R + n] = f32_to_bf16_bits(v);
        else part[((size_t)s * M + m) * R + n] = v;
      }
  }
}

// out[e] = bf16(sum over s of part[s][e]), e over M * R, in split order.
__global__ __launch_bounds__(256) void prefill_direct_fold_kernel(const float* __restrict__ part,
                                                                  uint16_t* __restrict__ out, int S,
                                                                  int64_t n) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  float v = part[e];
  for (int s = 1; s < S; ++s) v += part[(size_t)s * n + e];
  out[e] = f32_to_bf16_bits(v);
}

// Column chunks per 32-row tile: enough workgroups for ~4 waves per SIMD
// (fewer, longer waves ran faster than ~8 per SIMD), at least 4 steps per
// chunk (one per wave).
int direct_splits(int64_t R, int64_t C) {
  const int64_t tiles = (R + 31) / 32, nsteps = C / kBK;
  const int64_t want = ((int64_t)device_cus() * 4 * 4 + tiles * 4 - 1) / (tiles * 4);
  return (int)std::max<int64_t>(1, std::min<int64_t>(want, nsteps / 4));
}

PrefillPlan make_plan(int64_t R, int64_t C, int64_t M) {
  PrefillPlan p{};
  const int bm = tile_rows(M);
  const int nm = (int)((M + bm - 1) / bm);
  const int occ = bm == kBMSmall ? XTile<kBMSmall>::kOcc : XTile<kBMLarge>::kOcc;
  p.nn = (int)((R + kBN - 1) / kBN);
  p.ntiles = nm * p.nn;
  const int cus = device_cus() * occ;          // workgroup slots
  const int nsteps = (int)(C / kBK), quads = nsteps / 4;
  const int rem = p.ntiles % cus;
  p.nsteps = nsteps;
  p.nfull = p.ntiles;
  p.nsplit = 0;
  p.S = 1;
  p.seg = nsteps;
  if (rem > 0 && 2 * rem <= cus && quads >= 2) {
    const int S0 = min(cus / rem, quads);
    p.seg = 4 * ((quads + S0 - 1) / S0);
    p.S = (nsteps + p.seg - 1) / p.seg;
    p.nsplit = rem;
    p.nfull = p.ntiles - rem;
  } else if (rem > 0 && quads >= 2) {
    const int64_t total = (int64_t)p.ntiles * nsteps;
    p.stream = 1;
    p.U = (int)(4 * ((total + 4 * (int64_t)cus - 1) / (4 * (int64_t)cus)));
    p.G = (int)((total + p.U - 1) / p.U);
  }
  p.per = (p.nfull + kXcds - 1) / kXcds;
  return p;
}

}  // namespace

// bytes of x in operand order: whole 32-row blocks
int64_t prefill_xf_bytes(int64_t C, int64_t M) { return (M + 31) / 32 * 32 * C * 2; }

bool prefill_fused_supported(int64_t R, int64_t C, int64_t M, int k) {
  // 32-bit buffer offsets (x in operand order and one weight matrix's codes
  // below 2 GiB) and 32-bit step counters over the whole problem
  const int64_t steps = ((M + tile_rows(M) - 1) / tile_rows(M)) * ((R + kBN - 1) / kBN) * (C / kBK);
  return k >= 2 && k <= 4 && C % (4 * kBK) == 0 && prefill_xf_bytes(C, M) < ((int64_t)1 << 31) &&
         R * C * k / 8 < ((int64_t)1 << 31) && steps < ((int64_t)1 << 30);
}

// workspace: x in operand order, then the f32 partial tiles of split tiles
// (register-direct path: the f32 partials [S][M][R] of its column chunks)
size_t prefill_fused_workspace_bytes(int64_t R, int64_t C, int64_t M, int axis0) {
  const size_t xfb0 = ((size_t)prefill_xf_bytes(C, M) + 255) / 256 * 256;
  if (!axis0 && M <= kDirectMaxM) {
    const int S = direct_splits(R, C);
    return xfb0 + (S > 1 ? (size_t)S * M * R * sizeof(float) : 0);
  }
  const PrefillPlan p = make_plan(R, C, M);
  const size_t slots = p.stream ? 2 * (size_t)p.G : (size_t)p.nsplit * (size_t)p.S;
  const size_t xfb = ((size_t)prefill_xf_bytes(C, M) + 255) / 256 * 256;
  const size_t tile_floats = (size_t)tile_rows(M) * kBN;
  return xfb + slots * tile_floats * sizeof(float);
}

hipError_t launch_prefill_fused(const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                                uint16_t* out, int64_t R, int64_t C, int64_t M, int k,
                                void* workspace, hipStream_t stream, int axis0, int interleave) {
  if (interleave && (!axis0 || k != 3 || R % 512 != 0)) return hipErrorInvalidValue;
  PrefillPlan p = make_plan(R, C, M);
  p.il = interleave;
  uint8_t* ws = reinterpret_cast<uint8_t*>(workspace);
  uint16_t* xf = reinterpret_cast<uint16_t*>(ws);
  float* part = reinterpret_cast<float*>(ws + ((size_t)prefill_xf_bytes(C, M) + 255) / 256 * 256);
  const int r = (int)R, c = (int)C, m = (int)M;
  const int64_t nunits = prefill_xf_bytes(C, M) / 16;
  hipError_t e = hipSuccess;
  const bool xd = !axis0 && M <= kDirectXMaxM;   // x read in place: no layout pass
  if (!xd) {
    hipLaunchKernelGGL(prefill_xlayout_kernel, dim3((unsigned)((nunits + 255) / 256)), dim3(256), 0, stream, x,
                       reinterpret_cast<uint4*>(xf), m, c, nunits);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!axis0 && M <= kDirectMaxM) {
    const int S = direct_splits(R, C);
    const dim3 dgrid((unsigned)(((R + 31) / 32) * S));
#define TRELLIS_DIRECT_LAUNCH(KK)                                                                                  \
  if (xd) hipLaunchKernelGGL((prefill_direct_kernel<KK, 1, true>), dgrid, dim3(256), 0, stream, codes, scales, x, out, \
                             part, r, c, m, S);                                                                    \
  else if (M > 32) hipLaunchKernelGGL((prefill_direct_kernel<KK, 2>), dgrid, dim3(256), 0, stream, codes, scales, xf,  \
                                      out, part, r, c, m, S);                                                      \
  else hipLaunchKernelGGL((prefill_direct_kernel<KK, 1>), dgrid, dim3(256), 0, stream, codes, scales, xf, out, part, r, \
                          c, m, S)
    switch (k) {
      case 2: TRELLIS_DIRECT_LAUNCH(2); break;
      case 3: TRELLIS_DIRECT_LAUNCH(3); break;
      case 4: TRELLIS_DIRECT_LAUNCH(4); break;
      default: return hipErrorInvalidValue;
    }
#undef TRELLIS_DIRECT_LAUNCH
    e = hipGetLastError();
    if (e != hipSuccess || S == 1) return e;
    const int64_t n = M * R;
    hipLaunchKernelGGL(prefill_direct_fold_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, part,
                       out, S, n);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)(p.stream ? p.G : kXcds * p.per + p.nsplit * p.S)), block(256);
  const bool small = tile_rows(M) == kBMSmall;
#define TRELLIS_PREFILL_LAUNCH(KK, BMM, AX0)                                                              \
  hipLaunchKernelGGL((prefill_fused_kernel<KK, BMM, AX0>), grid, block, 0, stream, codes, scales, xf, out, part, \
                     r, c, m, p)
  switch ((k * 2 + (small ? 1 : 0)) * 2 + (axis0 ? 1 : 0)) {
    case 8: TRELLIS_PREFILL_LAUNCH(2, kBMLarge, false); break;
    case 9: TRELLIS_PREFILL_LAUNCH(2, kBMLarge, true); break;
    case 10: TRELLIS_PREFILL_LAUNCH(2, kBMSmall, false); break;
    case 11: TRELLIS_PREFILL_LAUNCH(2, kBMSmall, true); break;
    case 12: TRELLIS_PREFILL_LAUNCH(3, kBMLarge, false); break;
    case 13: TRELLIS_PREFILL_LAUNCH(3, kBMLarge, true); break;
    case 14: TRELLIS_PREFILL_LAUNCH(3, kBMSmall, false); break;
    case 15: TRELLIS_PREFILL_LAUNCH(3, kBMSmall, true); break;
    case 16: TRELLIS_PREFILL_LAUNCH(4, kBMLarge, false); break;
    case 17: TRELLIS_PREFILL_LAUNCH(4, kBMLarge, true); break;
    case 18: TRELLIS_PREFILL_LAUNCH(4, kBMSmall, false); break;
    case 19: TRELLIS_PREFILL_LAUNCH(4, kBMSmall, true); break;
    default: return hipErrorInvalidValue;
  }
#undef TRELLIS_PREFILL_LAUNCH
  e = hipGetLastError();
  if (e != hipSuccess || (!p.stream && p.nsplit == 0)) return e;
  const unsigned ntile = (unsigned)(p.stream ? p.ntiles : p.nsplit);
  if (small)
    hipLaunchKernelGGL(prefill_fold_kernel<kBMSmall>, dim3(ntile * XTile<kBMSmall>::kG4), dim3(256), 0, stream,
                       part, out, r, m, p);
  else
    hipLaunchKernelGGL(prefill_fold_kernel<kBMLarge>, dim3(ntile * XTile<kBMLarge>::kG4), dim3(256), 0, stream,
                       part, out, r, m, p);
  return hipGetLastError();
}

}  // namespace trellis
