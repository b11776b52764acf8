// axis1.hip -- axis-1 matvec and fused gate/up + SwiGLU for M <= 4 on gfx950.
//
// y[m, r] = sum_c w(r, c) x[m, c],  w(r, c) = value(s(r, c)) * scale[r].
// Source: mlx-bun 0.2.0 -> 0.4.0 diff (page 55), trellis-linear.ts REDUCE and
// GATEUP kernels (one pass over x, gate/up never materialised, SwiGLU cast
// chain in the epilogue); page 56, trellis-shared-m.ts (decode once, reuse
// for every vector).
//
// The sum is refactored as y = (scale / d) * sum_c code(r, c) * x[m, c] so
// the inner product runs on v_mfma_f32_16x16x32_f16 with exact operands:
//   A (16 rows x 32 k): the integer code y = bytesum(1MAD word) - 510, exact
//     in f16; built two at a time from the byte sums (v_sad_u8 straight into
//     f16 bits, one packed subtract).
//   B (32 k x 16 n): x'[n, c] = f16(x[n, c] * 2^e_n), e_n chosen per vector so
//     the largest |x| lands in [2^14, 2^15); every bf16 value down to 2^-17 of
//     that maximum is exact in f16.
//   D: f32 accumulators; the epilogue applies scale/d and 2^-e_n.
//
// Persistent schedule: one workgroup of 8 waves per CU.
//  1. The workgroup finds e_n and stages x' for all vectors and columns in
//     LDS (no separate pass over x, no workspace).
//  2. It streams row groups b, b + grid, ... (16 A-rows each: 16 output rows,
//     or 8 gate + 8 up rows sharing B).  The 8 waves split a row group's runs
//     of 32 columns; each lane decodes one whole run per step: k words plus
//     the next one up (wrapping to word 0 at the block end) hold every window
//     of the run, and k extra funnel shifts make every window a single
//     v_bfe_u32 at a constant offset.  Code words ride a 4-deep register ring
//     that runs across row-group boundaries, so the HBM stream never drains;
//     B comes from LDS.  Partial D tiles meet in LDS (double buffered, one
//     barrier per row group) and one wave, rotating with the row group,
//     applies scale / d, 2^-e and the epilogue.
#include "internal.hpp"
#include "mfma_common.hpp"

namespace trellis {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPWaves = 8;                     // waves per workgroup (two per SIMD)
constexpr int kXPad = 16;                      // f16 elements of row padding (spreads LDS banks)
constexpr int kXRegs = 5;                      // 16-byte pieces of x held per thread while staging (M*C <= 20480 in one pass)

// Dynamic LDS layout of the persistent kernel.
struct Axis1Lds {
  int64_t ldx;          // padded x' row (elements)
  size_t tile_off;      // two code tiles of 16 rows, row stride rs bytes
  size_t rs;            // padded tile row (bytes): a row's packed words + 16 B
  size_t tile_bytes;
  size_t red_off;       // f32x4 [2][kPWaves][64] partial sums (double buffered)
  size_t exp_off;       // int [4] exponents, then uint32 [kPWaves][4] max staging
  size_t total;
};

__host__ __device__ inline Axis1Lds axis1_lds(int64_t C, int M, int k) {
  Axis1Lds l;
  l.ldx = C + kXPad;
  // x' f16 [M][ldx] followed by 64 zero bytes (B operand of ragged runs)
  l.tile_off = ((size_t)M * (size_t)l.ldx * 2 + 64 + 255) / 256 * 256;
  l.rs = (size_t)C * k / 8 + 16;
  l.tile_bytes = (16 * l.rs + 255) / 256 * 256;
  l.red_off = l.tile_off + 2 * l.tile_bytes;
  l.exp_off = l.red_off + 2 * kPWaves * 64 * sizeof(f32x4);
  l.total = l.exp_off + 4 * sizeof(int) + kPWaves * 4 * sizeof(uint32_t);
  return l;
}

__device__ __forceinline__ half8 load_half8(const uint16_t* p) {
  return __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(p));
}

// The 32 codes of one run as four MFMA A operands of 8 exact f16 values
// (A[u] element e = position 8u + e of the run).
template <int K>
__device__ __forceinline__ void decode_run_f16(const uint32_t (&w)[K + 1], uint32_t mul,
                                               uint64_t add64, uint32_t magic, u32x4 (&A)[4]) {
  uint32_t a[2 * K];                           // a[j] holds bits 16j .. 16j+31 of the run
#pragma unroll
  for (int m = 0; m < K; ++m) {
    a[2 * m] = w[m];
    a[2 * m + 1] = __builtin_amdgcn_alignbit(w[m + 1], w[m], 16);
  }
  // three phases, so no 1MAD result is consumed right after it is produced:
  // all 32 windows, all 32 1MAD words, then the 16 f16 pairs
  uint32_t st[32];
#pragma unroll
  for (int p = 0; p < 32; ++p) {
    const int b = (31 - p) * K;                 // window start of position p
    st[p] = __builtin_amdgcn_ubfe(a[b >> 4], b & 15, kL);
  }
  uint32_t xw[32];
#pragma unroll
  for (int p = 0; p < 32; ++p) xw[p] = onemad_word_mad64(st[p], mul, add64);
#pragma unroll
  for (int v = 0; v < 16; ++v) A[v >> 2][v & 3] = code_pair_f16(xw[2 * v], xw[2 * v + 1], magic);
}

template <int K, int M, bool GATEUP>
__global__ __launch_bounds__(512) void axis1_persistent_kernel(
    const uint32_t* __restrict__ codes0, const uint16_t* __restrict__ scales0,
    const uint32_t* __restrict__ codes1, const uint16_t* __restrict__ scales1,
    const uint16_t* __restrict__ x, void* __restrict__ out, int out_f32,
    float* __restrict__ gate_f32, float* __restrict__ up_f32, int64_t R, int64_t C) {
  constexpr int WPB = words_per_block(K);
  constexpr int ROWS = GATEUP ? 8 : 16;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const Axis1Lds lay = axis1_lds(C, M, K);
  uint16_t* xs = reinterpret_cast<uint16_t*>(smem);
  uint16_t* zpad = xs + (int64_t)M * lay.ldx;                  // 32 zero elements
  f32x4* red = reinterpret_cast<f32x4*>(smem + lay.red_off);
  int* sexp = reinterpret_cast<int*>(smem + lay.exp_off);
  uint32_t* smax = reinterpret_cast<uint32_t*>(sexp + 4);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar) index
  const int64_t n8 = C / 8;
  const int64_t nrg = (R + ROWS - 1) / ROWS;
  const int64_t nmine = (nrg > (int64_t)blockIdx.x) ? (nrg - 1 - blockIdx.x) / gridDim.x + 1 : 0;
  const int64_t row_words = (C / kT) * WPB;
  const int npieces = (int)(row_words / 4);      // 16-byte pieces per packed row
  uint8_t* tiles = smem + lay.tile_off;

  // HBM -> LDS copy of the 16 packed rows of local row group t into tile buf:
  // coalesced 16-byte pieces straight into LDS (global_load_lds_dwordx4);
  // wave w copies tile rows w and w + 8.
  auto dma_tile = [&](int64_t t, int buf) {
    const int64_t rg = (int64_t)blockIdx.x + t * gridDim.x;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int rr = wave + 8 * h;
      const int64_t row = rg * ROWS + (GATEUP ? (rr & 7) : rr);
      const uint32_t* src = ((GATEUP && rr >= 8) ? codes1 : codes0) + (row < R ? row : 0) * row_words;
      uint8_t* dst = tiles + (size_t)buf * lay.tile_bytes + (size_t)rr * lay.rs;
      for (int p0 = 0; p0 < npieces; p0 += 64) {
        if (p0 + lane < npieces)
          __builtin_amdgcn_global_load_lds(src + (int64_t)(p0 + lane) * 4, dst + (size_t)p0 * 16, 16, 0, 0);
      }
    }
  };

  // the first two tiles stream in while x is staged
  if (nmine > 0) dma_tile(0, 0);
  if (nmine > 1) dma_tile(1, 1);


  // ---- 1. per-vector exponent and the f16 copy of x in LDS.  One pass:
  // every thread loads its (up to kXRegs) 16-byte pieces of x at once, keeps
  // them in registers through the max reduction, then converts them.
  {
    const int64_t npc = (int64_t)M * n8;         // 16-byte pieces of x
    uint4 xv[kXRegs];
    uint32_t mx[M];
#pragma unroll
    for (int m = 0; m < M; ++m) mx[m] = 0u;
#pragma unroll
    for (int u = 0; u < kXRegs; ++u) {
      const int64_t j = tid + (int64_t)u * 512;
      xv[u] = (j < npc) ? reinterpret_cast<const uint4*>(x)[j] : make_uint4(0u, 0u, 0u, 0u);
    }
    for (int64_t j = tid + (int64_t)kXRegs * 512; j < npc; j += 512) {   // rows longer than the registers hold
      const uint4 v = reinterpret_cast<const uint4*>(x)[j];
      const int m = (int)((uint32_t)j / (uint32_t)n8);
      const uint32_t u4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int h = 0; h < 4; ++h)
#pragma unroll
        for (int mm = 0; mm < M; ++mm)
          if (mm == m) mx[mm] = max(mx[mm], max(u4[h] & 0x7FFFu, (u4[h] >> 16) & 0x7FFFu));
    }
#pragma unroll
    for (int u = 0; u < kXRegs; ++u) {
      const int64_t j = tid + (int64_t)u * 512;
      const int m = (int)((uint32_t)j / (uint32_t)n8);
      const uint32_t u4[4] = {xv[u].x, xv[u].y, xv[u].z, xv[u].w};
      uint32_t v = 0u;
#pragma unroll
      for (int h = 0; h < 4; ++h) v = max(v, max(u4[h] & 0x7FFFu, (u4[h] >> 16) & 0x7FFFu));
#pragma unroll
      for (int mm = 0; mm < M; ++mm)
        if (mm == m && j < npc) mx[mm] = max(mx[mm], v);
    }
#pragma unroll
    for (int m = 0; m < M; ++m) {
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) mx[m] = max(mx[m], (uint32_t)__shfl_xor((int)mx[m], o, 64));
      if (lane == 0) smax[wave * 4 + m] = mx[m];
    }
    if (tid < 4) reinterpret_cast<uint4*>(zpad)[tid] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    int e[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      uint32_t v = 0u;
#pragma unroll
      for (int w = 0; w < kPWaves; ++w) v = max(v, smax[w * 4 + m]);
      e[m] = 0;
      if (v != 0u && v < 0x7F80u) {             // finite, non-zero maximum
        int ex;
        frexpf(bf16_bits_to_f32(v), &ex);        // max in [2^(ex-1), 2^ex)
        e[m] = 15 - ex;                          // max * 2^e in [2^14, 2^15)
      }
      if (tid == 0) sexp[m] = e[m];
    }
    auto convert_store = [&](int64_t j, const uint4& v) {
      const int m = (int)((uint32_t)j / (uint32_t)n8);
      const int64_t c8 = j - (int64_t)m * n8;
      int em = e[0];
#pragma unroll
      for (int mm = 1; mm < M; ++mm) em = (mm == m) ? e[mm] : em;
      const uint32_t u4[4] = {v.x, v.y, v.z, v.w};
      uint32_t o[4];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const _Float16 lo = (_Float16)ldexpf(bf16_bits_to_f32(u4[h] & 0xFFFFu), em);
        const _Float16 hi = (_Float16)ldexpf(bf16_bits_to_f32(u4[h] >> 16), em);
        o[h] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
      }
      *reinterpret_cast<uint4*>(xs + (int64_t)m * lay.ldx + c8 * 8) = make_uint4(o[0], o[1], o[2], o[3]);
    };
#pragma unroll
    for (int u = 0; u < kXRegs; ++u) {
      const int64_t j = tid + (int64_t)u * 512;
      if (j < npc) convert_store(j, xv[u]);
    }
    for (int64_t j = tid + (int64_t)kXRegs * 512; j < npc; j += 512)
      convert_store(j, reinterpret_cast<const uint4*>(x)[j]);
  }
  // ---- 2. row groups
  const int i = lane & 15, q = lane >> 4;
  const int nruns = (int)(C / 32);
  const int per = (nruns + kPWaves - 1) / kPWaves;
  const int rb = min(nruns, wave * per), re = min(nruns, rb + per);
  const int nfull = (re - rb) >> 2;              // full groups of four runs (one per lane group q)
  const int ntail = (re - rb) & 3;               // runs of a ragged last group
  // word and spill-word offsets of this lane's run in groups 0 and 1 (run = rb + q + 4g)
  auto word_off = [&](int run) { return (run >> 3) * WPB + (7 - (run & 7)) * K; };
  auto spill_off = [&](int run) {
    const int w = (7 - (run & 7)) * K + K;      // word after the run, wrapping to word 0 of the block
    return (run >> 3) * WPB + (w == WPB ? 0 : w);
  };
  const int wo0 = word_off(rb + q), so0 = spill_off(rb + q);
  const int wo1 = word_off(rb + q + 4), so1 = spill_off(rb + q + 4);
  const uint16_t* xrow = xs + (int64_t)(i < M ? i : 0) * lay.ldx;
  // B operand of group g: x' columns of run rb + q + 4g (lanes past the M vectors read the zero pad)
  const uint16_t* bbase = (i < M) ? xrow + (int64_t)(rb + q) * 32 : zpad;
  const int bstep = (i < M) ? 128 : 0;
  const uint32_t mul = kMul, magic = kHalfMagic;
  const uint64_t add64 = kAdd;

  // epilogue: wave (t mod 8) finalises row group t; lane < ROWS * M owns one output
  const int on = lane / ROWS, orr = lane % ROWS;
  const bool oown = lane < ROWS * M;

  __builtin_amdgcn_s_waitcnt(0);              // this wave's part of tiles 0 and 1
  __syncthreads();

  for (int64_t t = 0; t < nmine; ++t) {
    const int buf = (int)(t & 1);
    const bool owner = (int)(t % kPWaves) == wave;
    const int64_t orow = ((int64_t)blockIdx.x + t * gridDim.x) * ROWS + orr;
    float osc0 = 0.f, osc1 = 0.f;
    if (owner && oown && orow < R) {
      osc0 = half_bits_to_f32(scales0[orow]);
      if constexpr (GATEUP) osc1 = half_bits_to_f32(scales1[orow]);
    }
    const uint32_t* trow = reinterpret_cast<const uint32_t*>(tiles + (size_t)buf * lay.tile_bytes + (size_t)i * lay.rs);
    // four independent accumulators: the MFMAs of a group do not wait on each other
    f32x4 acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint32_t Wa[K + 1], Wb[K + 1];
    half8 Ba[4], Bb[4];
    auto read_group = [&](int g, uint32_t (&W)[K + 1], half8 (&B)[4]) {
      const int j = g >> 1;                     // offsets repeat every two groups, one block apart
      const int wo = ((g & 1) ? wo1 : wo0) + j * WPB;
      const int so = ((g & 1) ? so1 : so0) + j * WPB;
#pragma unroll
      for (int m = 0; m < K; ++m) W[m] = trow[wo + m];
      W[K] = trow[so];
      const uint16_t* bp = bbase + (int64_t)g * bstep;
#pragma unroll
      for (int u = 0; u < 4; ++u) B[u] = load_half8(bp + 8 * u);
    };
    auto consume = [&](const uint32_t (&W)[K + 1], const half8 (&B)[4]) {
      u32x4 A[4];
      decode_run_f16<K>(W, mul, add64, magic, A);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        acc[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, A[u]), B[u], acc[u], 0, 0, 0);
    };
    // full groups: LDS reads run one group ahead of the decode (ping-pong)
    if (nfull > 0) read_group(0, Wa, Ba);
    for (int g = 0; g < nfull; g += 2) {
      if (g + 1 < nfull) read_group(g + 1, Wb, Bb);
      consume(Wa, Ba);
      if (g + 2 < nfull) read_group(g + 2, Wa, Ba);
      if (g + 1 < nfull) consume(Wb, Bb);
    }
    if (ntail) {                                // ragged last group: lanes past the range add zeros
      const int run = rb + 4 * nfull + q;
      const bool valid = run < re;
      const int runc = valid ? run : rb;
      const uint32_t* bw = trow + (runc >> 3) * WPB;
      const int w0 = (7 - (runc & 7)) * K;
#pragma unroll
      for (int m = 0; m < K; ++m) Wa[m] = bw[w0 + m];
      Wa[K] = bw[(w0 + K == WPB) ? 0 : w0 + K];
      const uint16_t* bp = (i < M && valid) ? xrow + (int64_t)run * 32 : zpad;
#pragma unroll
      for (int u = 0; u < 4; ++u) Ba[u] = load_half8(bp + 8 * u);
      consume(Wa, Ba);
    }
    // row group complete: the next tile's copy has landed (this wave's part),
    // partial D tiles go to LDS, one barrier, then the freed tile is refilled
    // two row groups ahead and one wave runs the epilogue.
    red[(buf * kPWaves + wave) * 64 + lane] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 2 < nmine) dma_tile(t + 2, buf);
    if (owner && oown && orow < R) {
      // D of a 16x16 tile: lane 16*(a/4) + n holds row a, column n in element a % 4
      const int e = sexp[on];
      float s0 = 0.f;
#pragma unroll
      for (int v = 0; v < kPWaves; ++v) s0 += red[(buf * kPWaves + v) * 64 + 16 * (orr >> 2) + on][orr & 3];
      const float v0 = ldexpf(s0 * (osc0 * kRcp), -e);
      const int64_t o = (int64_t)on * R + orow;
      if constexpr (GATEUP) {
        const int ju = orr + 8;
        float s1 = 0.f;
#pragma unroll
        for (int v = 0; v < kPWaves; ++v) s1 += red[(buf * kPWaves + v) * 64 + 16 * (ju >> 2) + on][ju & 3];
        const float v1 = ldexpf(s1 * (osc1 * kRcp), -e);
        if (gate_f32) gate_f32[o] = v0;
        if (up_f32) up_f32[o] = v1;
        const float gT = round_bf16(v0);
        const float uT = round_bf16(v1);
        const float sig = round_bf16(1.0f / (1.0f + expf(-gT)));
        const float silu = round_bf16(gT * sig);
        reinterpret_cast<uint16_t*>(out)[o] = f32_to_bf16_bits(silu * uT);
      } else {
        if (out_f32) reinterpret_cast<float*>(out)[o] = v0;
        else reinterpret_cast<uint16_t*>(out)[o] = f32_to_bf16_bits(v0);
      }
    }
  }
}

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

template <int K, int M, bool GU>
hipError_t axis1_launch_one(const uint32_t* c0, const uint16_t* s0, const uint32_t* c1,
                            const uint16_t* s1, const uint16_t* x, void* out, int out_f32,
                            float* gf, float* uf, int64_t R, int64_t C, hipStream_t stream) {
  const Axis1Lds lay = axis1_lds(C, M, K);
  static bool lds_attr = false;                 // raise the dynamic LDS limit once per instantiation
  if (!lds_attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&axis1_persistent_kernel<K, M, GU>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kAxis1MaxLdsBytes);
    if (e != hipSuccess) return e;
    lds_attr = true;
  }
  const int64_t rows = GU ? 8 : 16;
  const int64_t nrg = (R + rows - 1) / rows;
  const int64_t cus = device_cus();
  const unsigned grid = (unsigned)(nrg < cus ? nrg : cus);
  hipLaunchKernelGGL((axis1_persistent_kernel<K, M, GU>), dim3(grid), dim3(512), lay.total, stream,
                     c0, s0, c1, s1, x, out, out_f32, gf, uf, R, C);
  return hipGetLastError();
}

template <int K>
hipError_t axis1_main(const uint32_t* c0, const uint16_t* s0, const uint32_t* c1,
                      const uint16_t* s1, const uint16_t* x, void* out, int out_f32, float* gf,
                      float* uf, int64_t R, int64_t C, int M, hipStream_t stream) {
  const bool gu = c1 != nullptr;
#define TRELLIS_AXIS1_CASE(MM)                                                                      \
  case MM:                                                                                           \
    return gu ? axis1_launch_one<K, MM, true>(c0, s0, c1, s1, x, out, out_f32, gf, uf, R, C, stream) \
              : axis1_launch_one<K, MM, false>(c0, s0, c1, s1, x, out, out_f32, gf, uf, R, C, stream);
  switch (M) {
    TRELLIS_AXIS1_CASE(1)
    TRELLIS_AXIS1_CASE(2)
    TRELLIS_AXIS1_CASE(3)
    TRELLIS_AXIS1_CASE(4)
    default: return hipErrorInvalidValue;
  }
#undef TRELLIS_AXIS1_CASE
}

}  // namespace

size_t axis1_workspace_bytes(int64_t, int64_t, int, int) { return 0; }

size_t axis1_lds_bytes(int64_t C, int M, int k) { return axis1_lds(C, M, k).total; }

hipError_t launch_axis1(const uint32_t* codes0, const uint16_t* scales0, const uint32_t* codes1,
                        const uint16_t* scales1, const uint16_t* x, void* out, int out_f32,
                        float* gate_f32, float* up_f32, int64_t R, int64_t C, int M, int k,
                        void*, hipStream_t stream) {
  switch (k) {
    case 2: return axis1_main<2>(codes0, scales0, codes1, scales1, x, out, out_f32, gate_f32, up_f32, R, C, M, stream);
    case 3: return axis1_main<3>(codes0, scales0, codes1, scales1, x, out, out_f32, gate_f32, up_f32, R, C, M, stream);
    case 4: return axis1_main<4>(codes0, scales0, codes1, scales1, x, out, out_f32, gate_f32, up_f32, R, C, M, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace trellis
