/*
 * trellis_oracle.c -- slow, plain CPU oracle for the packed trellis-coded
 * linear layer.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or constant generator with the GPU library; neither side
 * includes or links the other.
 *
 * Source of every definition below (cited by page title and section):
 *   [TL]  mlx-bun 0.2.0 -> 0.4.0 diff, page 55, src/model/trellis-linear.ts:
 *         file header comment (packed format, axis convention) and the HEADER
 *         decode helpers (1MAD code, value, window/state), REDUCE / SCATTER /
 *         GATEUP / EXPAND kernel descriptions, TrellisLinear.forward.
 *   [TP]  mlx-bun 0.2.0 -> 0.4.0 diff, page 56, src/model/trellis-tiled-prefill.ts
 *         (prefill weight = bf16 of the precise value times the scale).
 *
 * Precision: every sum is taken in double over the terms in index order.
 * Products that are exact in double (f32 weight x bf16 activation,
 * bf16 x bf16) are formed exactly.  No blocking, no reordering, no tricks:
 * each function is the definition written out.
 *
 * Parity pins: see tests/test_oracle_pins.py (closed forms, brute force over
 * all 2^L states, shift-register writer/reader, one-hot metamorphic tests,
 * dense decode-then-dot via numpy, exact rational rounding via fractions).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* 1MAD constants and the divisor, as printed in [TL] HEADER (trellis_y /
 * trellis_val).  d = 147.800537109375 is exactly 605391 / 4096. */
#define TRO_MUL 34038481u
#define TRO_ADD 76625530u
#define TRO_DIV 147.800537109375

/* ------------------------------------------------------------------ */
/* scalar conversions                                                  */
/* ------------------------------------------------------------------ */

/* IEEE binary16 bits -> exact double. */
double tro_half_to_double(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 10) & 31;
  const int m = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)m, -24);                 /* subnormal */
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), e - 25);            /* (1.m) * 2^(e-15) */
  return sign ? -v : v;
}

/* bfloat16 bits -> exact double (bf16 is the top half of a binary32). */
double tro_bf16_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* Round a finite double to the nearest bfloat16, ties to even, and return
 * its bits.  Written from the definition: scale by the bf16 ulp of v's
 * binade, round the integer significand half-to-even, scale back. */
uint16_t tro_double_to_bf16(double v) {
  if (isnan(v)) return 0x7FC0;
  const int neg = signbit(v) ? 1 : 0;
  double a = fabs(v);
  float r;
  if (a == 0.0) {
    r = 0.0f;
  } else {
    int e;
    frexp(a, &e);                  /* a = f * 2^e, f in [0.5, 1) -> binade 2^(e-1) */
    int b = e - 1;                 /* 2^b <= a < 2^(b+1) */
    if (b < -126) b = -126;        /* subnormal bf16: fixed ulp 2^-133 */
    const double ulp = ldexp(1.0, b - 7);   /* 8 significant bits */
    double q = a / ulp;            /* exact: power-of-two scaling */
    double fl = floor(q);
    double rem = q - fl;
    double n = fl;
    if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) n = fl + 1.0;
    const double res = n * ulp;
    if (res > 3.3895313892515355e38) r = INFINITY;   /* beyond the largest finite bf16 */
    else r = (float)res;                             /* exact: <= 9 significant bits */
  }
  if (neg) r = -r;
  uint32_t u;
  memcpy(&u, &r, 4);
  return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------ */
/* decode primitive                                                    */
/* ------------------------------------------------------------------ */

/* Words per block: a block of T symbols of k bits is T*k/32 words. */
static int64_t tro_wpb(int k, int T) { return (int64_t)T * k / 32; }

/* Bit i of a block, bits counted LSB-first inside each 32-bit word and word
 * 0 first ([TL] HEADER trellis_state reads word wi >> off upward). */
static uint32_t tro_block_bit(const uint32_t* blk, int64_t i) {
  return (blk[i / 32] >> (i % 32)) & 1u;
}

/* State of block position t: the L-bit window whose lowest bit is bit
 * (T-1-t)*k of the block, read cyclically modulo the block's T*k bits
 * ([TL] file header: tail-biting window; HEADER trellis_state). */
uint32_t tro_state(const uint32_t* blk, int k, int L, int T, int t) {
  const int64_t nbits = (int64_t)T * k;
  const int64_t p = (int64_t)(T - 1 - t) * k;
  uint32_t s = 0;
  for (int j = 0; j < L; ++j) s |= tro_block_bit(blk, (p + j) % nbits) << j;
  return s;
}

/* 1MAD code of a state ([TL] HEADER trellis_y): x = s*34038481 + 76625530
 * modulo 2^32, then the sum of the four bytes of x, minus 510. */
int32_t tro_y(uint32_t s) {
  const uint32_t x = s * TRO_MUL + TRO_ADD;     /* unsigned arithmetic wraps mod 2^32 */
  const int32_t b0 = (int32_t)(x & 255u);
  const int32_t b1 = (int32_t)((x >> 8) & 255u);
  const int32_t b2 = (int32_t)((x >> 16) & 255u);
  const int32_t b3 = (int32_t)((x >> 24) & 255u);
  return b0 + b1 + b2 + b3 - 510;
}

/* Code value: y / d correctly rounded to binary32 ([TL] HEADER trellis_val,
 * the precise divide that matches the host table).  The candidate from a
 * double division is checked against both neighbours with exact residuals:
 * c*d is exact in double (24-bit by 20-bit significands). */
float tro_value(int32_t y) {
  const float f = (float)((double)y / TRO_DIV);
  const float cand[3] = {nextafterf(f, -INFINITY), f, nextafterf(f, INFINITY)};
  int best = 1;
  double best_err = fabs((double)cand[1] * TRO_DIV - (double)y);
  for (int i = 0; i < 3; i += 2) {
    const double err = fabs((double)cand[i] * TRO_DIV - (double)y);
    if (err < best_err) { best = i; best_err = err; }
  }
  /* No ties exist: y/d = 4096*y/605391 is never a binary32 midpoint for
   * 0 < |y| < 605391 (605391 is odd and does not divide y). */
  return cand[best];
}

/* Matvec weight ([TL] HEADER variant notes; default numerics): f32 product
 * of the code value and the row's fp16 scale, no bf16 rounding. */
static float tro_weight_f32(uint32_t s, double scale) {
  return (float)((double)tro_value(tro_y(s)) * scale);   /* product exact in double, one rounding */
}

/* Expansion / prefill weight ([TL] EXPAND kernel, [TP] tiled prefill):
 * bf16 (round to nearest even) of the f32 product value * scale. */
static double tro_weight_bf16(uint32_t s, double scale) {
  return tro_bf16_to_double(tro_double_to_bf16((double)tro_weight_f32(s, scale)));
}

/* Pointer to block b of stored row r ([TL] file header: row-major
 * [rows, cols*k/32]; C/T blocks of wpb words per row). */
static const uint32_t* tro_block(const uint32_t* codes, int64_t r, int64_t b, int64_t C, int k, int T) {
  const int64_t wpb = tro_wpb(k, T);
  return codes + r * (C / T) * wpb + b * wpb;
}

static uint32_t tro_state_rc(const uint32_t* codes, int64_t r, int64_t c, int64_t C, int k, int L, int T) {
  return tro_state(tro_block(codes, r, c / T, C, k, T), k, L, T, (int)(c % T));
}

/* Every weight of a stored [R, C] matrix: state, code y and value. */
void tro_decode(const uint32_t* codes, int64_t R, int64_t C, int k, int L, int T,
                uint16_t* states, int16_t* ys, float* values) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < R; ++r) {
    for (int64_t c = 0; c < C; ++c) {
      const uint32_t s = tro_state_rc(codes, r, c, C, k, L, T);
      const int32_t y = tro_y(s);
      if (states) states[r * C + c] = (uint16_t)s;
      if (ys) ys[r * C + c] = (int16_t)y;
      if (values) values[r * C + c] = tro_value(y);
    }
  }
}

/* ------------------------------------------------------------------ */
/* linear layer results                                                */
/* ------------------------------------------------------------------ */

/* Axis 1 ([TL] REDUCE): out[m, i] = sum_c w(row_i, c) * x[m, c] for the
 * selected stored rows (rows == NULL selects all R).  x: bf16 [M, C];
 * out: double [M, nrows].  abs_out (double [M, nrows], may be NULL)
 * receives sum_c |w(row_i, c) * x[m, c]|, the scale of the terms each sum
 * cancels (the parity criterion measures rounding error against it). */
void tro_matvec_axis1(const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                      int M, int64_t R, int64_t C, int k, int L, int T,
                      const int64_t* rows, int64_t nrows, double* out, double* abs_out) {
  if (!rows) nrows = R;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t i = 0; i < nrows; ++i) {
    const int64_t r = rows ? rows[i] : i;
    const double scale = tro_half_to_double(scales[r]);
    double* acc = (double*)calloc((size_t)M, sizeof(double));
    double* aacc = (double*)calloc((size_t)M, sizeof(double));
    for (int64_t c = 0; c < C; ++c) {
      const double w = (double)tro_weight_f32(tro_state_rc(codes, r, c, C, k, L, T), scale);
      for (int m = 0; m < M; ++m) {
        const double t = w * tro_bf16_to_double(x[(int64_t)m * C + c]);
        acc[m] += t;
        aacc[m] += fabs(t);
      }
    }
    for (int m = 0; m < M; ++m) {
      out[(int64_t)m * nrows + i] = acc[m];
      if (abs_out) abs_out[(int64_t)m * nrows + i] = aacc[m];
    }
    free(acc);
    free(aacc);
  }
}

/* Axis 0 ([TL] SCATTER + fold): stored matrix is W^T [R_in, C_out], coded
 * along C_out; out[m, j] = sum_r w(r, col_j) * x[m, r] over ALL stored rows,
 * with the stored row's scale.  x: bf16 [M, R]; out: double [M, ncols].
 * abs_out (may be NULL): sum_r |w(r, col_j) * x[m, r]|. */
void tro_matvec_axis0(const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                      int M, int64_t R, int64_t C, int k, int L, int T,
                      const int64_t* cols, int64_t ncols, double* out, double* abs_out) {
  if (!cols) ncols = C;
#pragma omp parallel for schedule(dynamic, 4)
  for (int64_t j = 0; j < ncols; ++j) {
    const int64_t c = cols ? cols[j] : j;
    double* acc = (double*)calloc((size_t)M, sizeof(double));
    double* aacc = (double*)calloc((size_t)M, sizeof(double));
    for (int64_t r = 0; r < R; ++r) {
      const double w = (double)tro_weight_f32(tro_state_rc(codes, r, c, C, k, L, T),
                                              tro_half_to_double(scales[r]));
      for (int m = 0; m < M; ++m) {
        const double t = w * tro_bf16_to_double(x[(int64_t)m * R + r]);
        acc[m] += t;
        aacc[m] += fabs(t);
      }
    }
    for (int m = 0; m < M; ++m) {
      out[(int64_t)m * ncols + j] = acc[m];
      if (abs_out) abs_out[(int64_t)m * ncols + j] = aacc[m];
    }
    free(acc);
    free(aacc);
  }
}

/* SwiGLU cast chain of the fused gate/up kernel ([TL] GATEUP kernel
 * comment): gate and up rounded to bf16, sigmoid of the rounded gate rounded
 * to bf16, silu = bf16(gate_bf16 * sigmoid_bf16), out = bf16(silu * up_bf16).
 * exp is evaluated in double.  Returns bf16 bits. */
uint16_t tro_swiglu(double gate, double up) {
  const double gT = tro_bf16_to_double(tro_double_to_bf16(gate));
  const double uT = tro_bf16_to_double(tro_double_to_bf16(up));
  const double sig = tro_bf16_to_double(tro_double_to_bf16(1.0 / (1.0 + exp(-gT))));
  const double silu = tro_bf16_to_double(tro_double_to_bf16(gT * sig));   /* exact product */
  return tro_double_to_bf16(silu * uT);                                    /* exact product */
}

/* Fused gate/up ([TL] fusedGateUpSwiglu): two axis-1 matvecs over the same
 * x, then the cast chain.  gate_out / up_out (double [M, nrows], may be
 * NULL) receive the raw sums, gate_abs / up_abs (may be NULL) their sums of
 * absolute terms; out receives bf16 bits [M, nrows]. */
void tro_gateup_swiglu(const uint32_t* gcodes, const uint16_t* gscales,
                       const uint32_t* ucodes, const uint16_t* uscales, const uint16_t* x,
                       int M, int64_t R, int64_t C, int k, int L, int T,
                       const int64_t* rows, int64_t nrows,
                       double* gate_out, double* up_out, uint16_t* out,
                       double* gate_abs, double* up_abs) {
  if (!rows) nrows = R;
  double* g = (double*)malloc(sizeof(double) * (size_t)M * (size_t)nrows);
  double* u = (double*)malloc(sizeof(double) * (size_t)M * (size_t)nrows);
  tro_matvec_axis1(gcodes, gscales, x, M, R, C, k, L, T, rows, nrows, g, gate_abs);
  tro_matvec_axis1(ucodes, uscales, x, M, R, C, k, L, T, rows, nrows, u, up_abs);
  for (int64_t i = 0; i < (int64_t)M * nrows; ++i) {
    if (gate_out) gate_out[i] = g[i];
    if (up_out) up_out[i] = u[i];
    if (out) out[i] = tro_swiglu(g[i], u[i]);
  }
  free(g);
  free(u);
}

/* Expansion of the stored matrix ([TL] EXPAND): out[r, c] = bf16 bits of
 * the expansion weight, stored orientation, rows [r0, r0 + nr). */
void tro_expand_bf16(const uint32_t* codes, const uint16_t* scales, int64_t R, int64_t C,
                     int k, int L, int T, int64_t r0, int64_t nr, uint16_t* out) {
  (void)R;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < nr; ++i) {
    const int64_t r = r0 + i;
    const double scale = tro_half_to_double(scales[r]);
    for (int64_t c = 0; c < C; ++c)
      out[i * C + c] = tro_double_to_bf16(tro_weight_bf16(tro_state_rc(codes, r, c, C, k, L, T), scale));
  }
}

/* Axis-1 prefill ([TP]; [TL] forward expand-then-matmul fallback):
 * sum[a, b] = sum_c wb(rows_b, c) * x[ms_a, c] with bf16 expansion weights,
 * each product exact in double.  x: bf16 [M, C]; sums: double [nm, nr].
 * The layer output is the bf16 rounding of each sum.  abs_sums (may be
 * NULL) receives sum_c |wb(rows_b, c) * x[ms_a, c]|. */
void tro_prefill(const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                 int64_t M, int64_t R, int64_t C, int k, int L, int T,
                 const int64_t* ms, int64_t nm, const int64_t* rows, int64_t nr, double* sums,
                 double* abs_sums) {
  (void)M;
  (void)R;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t b = 0; b < nr; ++b) {
    const int64_t r = rows[b];
    const double scale = tro_half_to_double(scales[r]);
    double* wrow = (double*)malloc(sizeof(double) * (size_t)C);
    for (int64_t c = 0; c < C; ++c) wrow[c] = tro_weight_bf16(tro_state_rc(codes, r, c, C, k, L, T), scale);
    for (int64_t a = 0; a < nm; ++a) {
      const uint16_t* xr = x + ms[a] * C;
      double acc = 0.0, aacc = 0.0;
      for (int64_t c = 0; c < C; ++c) {
        const double t = wrow[c] * tro_bf16_to_double(xr[c]);
        acc += t;
        aacc += fabs(t);
      }
      sums[a * nr + b] = acc;
      if (abs_sums) abs_sums[a * nr + b] = aacc;
    }
    free(wrow);
  }
}

/* Axis-0 prefill ([TL] forward expand-then-matmul fallback, for the stored
 * transpose of the SCATTER kernel's layout): sum[a, b] = sum_r wb(r, cols_b)
 * * x[ms_a, r] over ALL stored rows, wb the bf16 expansion weight of stored
 * row r (its own scale); each product exact in double.  x: bf16 [M, R];
 * sums: double [nm, nc].  The layer output is the bf16 rounding of each sum.
 * abs_sums (may be NULL) receives sum_r |wb(r, cols_b) * x[ms_a, r]|. */
void tro_prefill_axis0(const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                       int64_t M, int64_t R, int64_t C, int k, int L, int T,
                       const int64_t* ms, int64_t nm, const int64_t* cols, int64_t nc, double* sums,
                       double* abs_sums) {
  (void)M;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t b = 0; b < nc; ++b) {
    const int64_t c = cols[b];
    double* wcol = (double*)malloc(sizeof(double) * (size_t)R);
    for (int64_t r = 0; r < R; ++r)
      wcol[r] = tro_weight_bf16(tro_state_rc(codes, r, c, C, k, L, T), tro_half_to_double(scales[r]));
    for (int64_t a = 0; a < nm; ++a) {
      const uint16_t* xr = x + ms[a] * R;
      double acc = 0.0, aacc = 0.0;
      for (int64_t r = 0; r < R; ++r) {
        const double t = wcol[r] * tro_bf16_to_double(xr[r]);
        acc += t;
        aacc += fabs(t);
      }
      sums[a * nc + b] = acc;
      if (abs_sums) abs_sums[a * nc + b] = aacc;
    }
    free(wcol);
  }
}

/* Worker threads OpenMP will use (1 without OpenMP). */
int tro_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
