/*
 * trellis.h -- C ABI of the MI355X (gfx950) packed trellis-coded linear layer.
 *
 * Every weight of a stored matrix [R, C] (coded along C) is one k-bit symbol
 * of a uint32 bitstream, in blocks of T symbols.  The weight at block
 * position t is decoded from its L-bit state, the window that starts at bit
 * (T-1-t)*k of the block and wraps at the block end; the state goes through
 * the "1MAD" computed code to a value, which is scaled by the stored row's
 * fp16 scale.  Source: mlx-bun 0.2.0 -> 0.4.0 diff (page 55),
 * src/model/trellis-linear.ts, file header comment (format, axis
 * convention) and the HEADER decode helpers (trellis_y, trellis_val,
 * trellis_val_rcp, trellis_state).
 *
 * Conventions shared by every entry point
 *   - Buffers are DEVICE memory owned by the caller; the library never
 *     allocates on these calls and never keeps a pointer after returning.
 *   - Tensors are row-major and contiguous.  bf16 and fp16 values are passed
 *     as uint16_t bit patterns.  codes, x, out and workspace must be 16-byte
 *     aligned; scales 2-byte aligned.
 *   - Supported geometry: k in {2, 3, 4}, L = 12, T = 256, C % T == 0,
 *     R >= 1, C >= 1 (others: TRELLIS_EUNSUPPORTED or TRELLIS_EINVAL).
 *   - `stream` is a hipStream_t (NULL = the device's default stream).  Calls
 *     are asynchronous on that stream and never synchronise the host -- the
 *     two *_tune calls alone wait for their timing runs (they exist for
 *     that).
 *   - All checks run on the host before any launch.  On any non-zero return
 *     nothing was launched and nothing was written; trellis_last_error()
 *     then describes the problem (thread-local, valid until the next call on
 *     the same thread).
 *   - Calls that take a workspace use it as scratch that is fully rewritten
 *     by the call; concurrent calls must not share one workspace.
 */
#ifndef TRELLIS_H
#define TRELLIS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define TRELLIS_OK 0
#define TRELLIS_EINVAL (-1)        /* bad pointer, size, alignment or argument */
#define TRELLIS_EUNSUPPORTED (-2)  /* geometry outside k in {2,3,4}, L = 12, T = 256 */
#define TRELLIS_EWORKSPACE (-3)    /* workspace smaller than the queried size */
#define TRELLIS_EHIP (-4)          /* a HIP runtime or library call failed */

/* output element types for the plain matvecs */
#define TRELLIS_OUT_BF16 0
#define TRELLIS_OUT_F32 1

/* prefill algorithms */
#define TRELLIS_PREFILL_FUSED 0        /* decode into LDS tiles feeding bf16 MFMA */
#define TRELLIS_PREFILL_EXPAND_GEMM 1  /* trellis_expand_bf16 into the workspace, then a GEMM */
/* FUSED where it measured at least as fast on MI355X (axis 1: M <= 128;
 * axis 0: M <= 512) and the shape allows it, else EXPAND_GEMM; the workspace
 * size query answers for the algorithm chosen, with the same arguments. */
#define TRELLIS_PREFILL_AUTO 2

/* Largest M accepted by the packed matvecs (the pages' matvec/prefill
 * crossover, trellis-linear.ts MATVEC_MAX_M). */
#define TRELLIS_MATVEC_MAX_M 4

/* Most matrices in one trellis_matvec_axis1_group call. */
#define TRELLIS_GROUP_MAX 4

/*
 * trellis_matvec_axis1 -- y[m, r] = sum_c w(r, c) * x[m, c]   (axis = 1).
 * Source: trellis-linear.ts (page 55), REDUCE kernel comment and
 * TrellisLinear.forward; shared-M form in trellis-shared-m.ts (page 56).
 *   codes   uint32 [R, C*k/32]  coded along the input dim C
 *   scales  fp16   [R]          per output row
 *   x       bf16   [M, C]
 *   out     [M, R], bf16 (out_dtype = TRELLIS_OUT_BF16) or f32 (TRELLIS_OUT_F32)
 *   1 <= M <= TRELLIS_MATVEC_MAX_M.
 * w(r, c) is the f32 product of the code value and scales[r] (no bf16
 * rounding of weights: the pages' default numerics); sums accumulate in f32.
 * For the pages' variants 0-3 contract (weights rounded to bf16 first) see
 * trellis_prefill, which computes it for any M.
 * Workspace: none for C <= 5120.  Wider rows run as column chunks of at
 * most 5120 columns whose f32 partial outputs ([chunks][M][R]) the workspace
 * holds; trellis_matvec_axis1_workspace_bytes gives its size (0 when none is
 * needed).
 */
size_t trellis_matvec_axis1_workspace_bytes(int64_t R, int64_t C, int M, int k, int L, int T);
int trellis_matvec_axis1(const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                         void* out, int out_dtype, int64_t R, int64_t C, int M, int k, int L,
                         int T, void* workspace, size_t workspace_bytes, void* stream);

/*
 * trellis_matvec_axis1_group -- trellis_matvec_axis1 for n matrices that
 * share x, C and k (a layer's projections of one input), in one launch.
 * Source: the REDUCE kernel of trellis-linear.ts (page 55), per matrix;
 * running a projection set as one launch is this library's addition.
 *   codes[j]  uint32 [R[j], C*k/32];  scales[j] fp16 [R[j]]
 *   out[j]    [M, R[j]] in out_dtype;  x bf16 [M, C];  1 <= M <= 4
 *   1 <= n <= TRELLIS_GROUP_MAX
 * codes, scales, out and R are host arrays of n entries (read during the
 * call; the buffers they point to are device memory).  Each out[j] equals
 * what trellis_matvec_axis1 writes for matrix j, bit for bit.  The launch
 * spans the 16-row groups of all n matrices, so small projections share the
 * machine with the large ones instead of running alone.  No workspace, so
 * C <= 5120 (one launch holds x in registers); wider rows:
 * TRELLIS_EUNSUPPORTED.
 */
int trellis_matvec_axis1_group(const uint32_t* const* codes, const uint16_t* const* scales, void* const* out,
                               const int64_t* R, int n, const uint16_t* x, int out_dtype, int64_t C, int M,
                               int k, int L, int T, void* stream);

/*
 * trellis_gateup_swiglu -- out[m, r] = bf16(silu(bf16 g) * bf16 u), where
 * g = gate(x), u = up(x) are two axis-1 matvecs of identical geometry over
 * the same x.  Cast chain: gate and up to bf16, sigmoid of the bf16 gate to
 * bf16, silu = bf16(gate * sigmoid), out = bf16(silu * up).
 * Source: trellis-linear.ts (page 55), GATEUP kernel comment and
 * fusedGateUpSwiglu / fusedGateUpEligible.
 *   gcodes, ucodes  uint32 [R, C*k/32];  gscales, uscales fp16 [R]
 *   x               bf16 [M, C];  out bf16 [M, R];  1 <= M <= 4
 *   gate_f32, up_f32  optional f32 [M, R] copies of the raw sums (NULL = none)
 * Workspace as for trellis_matvec_axis1 (C > 5120 only), twice the size:
 * gate and up partials per column chunk.
 */
size_t trellis_gateup_swiglu_workspace_bytes(int64_t R, int64_t C, int M, int k, int L, int T);
int trellis_gateup_swiglu(const uint32_t* gcodes, const uint16_t* gscales, const uint32_t* ucodes,
                          const uint16_t* uscales, const uint16_t* x, uint16_t* out,
                          float* gate_f32, float* up_f32, int64_t R, int64_t C, int M, int k,
                          int L, int T, void* workspace, size_t workspace_bytes, void* stream);

/*
 * trellis_matvec_axis0 -- y[m, c] = sum_r w(r, c) * x[m, r]   (axis = 0).
 * The stored matrix is W^T [R_in, C_out], coded along C_out; w uses the
 * stored row's scale.  Split-K over stored rows into f32 partials in the
 * workspace, then a second pass folds them.
 * Source: trellis-linear.ts (page 55), SCATTER kernel comment and
 * TrellisLinear #scatter (partials, then one sum and a cast).
 *   codes   uint32 [R_in, C_out*k/32];  scales fp16 [R_in]
 *   x       bf16 [M, R_in];  out [M, C_out] bf16 or f32;  1 <= M <= 4
 */
size_t trellis_matvec_axis0_workspace_bytes(int64_t R_in, int64_t C_out, int M, int k, int L, int T);
int trellis_matvec_axis0(const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                         void* out, int out_dtype, int64_t R_in, int64_t C_out, int M, int k,
                         int L, int T, void* workspace, size_t workspace_bytes, void* stream);

/*
 * trellis_matvec_axis0_noalloc -- trellis_matvec_axis0 without a workspace
 * argument, for callers that cannot allocate device memory (code under
 * stream capture, tight serving loops, harnesses that forbid hipMalloc).
 * The split-K partials go to a static device array of 4 MiB that the
 * library holds on each device until the process ends; nothing is
 * allocated by the call.  Shapes whose partials (trellis_matvec_axis0_
 * workspace_bytes) exceed 4 MiB are rejected with TRELLIS_EUNSUPPORTED.
 * Every call on one device shares that device's array, so calls that
 * overlap in time on one device (other streams, other threads) race; calls
 * in one stream's order do not.  Outputs equal trellis_matvec_axis0's bit
 * for bit.  Arguments and errors otherwise as for trellis_matvec_axis0.
 */
int trellis_matvec_axis0_noalloc(const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                                 void* out, int out_dtype, int64_t R_in, int64_t C_out, int M, int k,
                                 int L, int T, void* stream);

/*
 * trellis_mlp_decode -- the MLP of a decoder layer for M <= 4 rows:
 *   hidden = silu(gate(x)) * up(x)        (trellis_gateup_swiglu, bf16)
 *   out    = down(hidden)                 (trellis_matvec_axis0, bf16)
 * on one stream with no host round trip; gate and up are axis-1 matrices
 * [R, C], down is stored transposed (axis 0) as W_down^T [R, C_out].
 * Source: mlx-bun 0.2.0 -> 0.3.0 diff (page 42), src/model/qwen3_5.ts,
 * Qwen3MLP (down of silu(gate) * up); the fused gate/up SwiGLU kernel it
 * runs for at most TRELLIS_MATVEC_MAX_M rows is the GATEUP kernel of
 * trellis-linear.ts on the mlx-bun 0.2.0 -> 0.4.0 diff (page 55).
 *   gcodes, ucodes uint32 [R, C*k_gu/32];  gscales, uscales fp16 [R]
 *   dcodes uint32 [R, C_out*k_down/32];   dscales fp16 [R]
 *   x bf16 [M, C];  out bf16 [M, C_out];  1 <= M <= 4
 *   hidden bf16 [M, R] (may be NULL): receives the hidden vectors, which
 *     otherwise live in the workspace
 * The workspace (trellis_mlp_decode_workspace_bytes) holds the hidden
 * vectors and the down projection's partials.  Errors as for the two calls
 * it makes; nothing is launched unless both would be accepted.
 */
size_t trellis_mlp_decode_workspace_bytes(int64_t R, int64_t C, int64_t C_out, int M, int k_gu,
                                          int k_down, int L, int T);
int trellis_mlp_decode(const uint32_t* gcodes, const uint16_t* gscales, const uint32_t* ucodes,
                       const uint16_t* uscales, const uint32_t* dcodes, const uint16_t* dscales,
                       const uint16_t* x, uint16_t* hidden, uint16_t* out, int64_t R, int64_t C, int64_t C_out,
                       int M, int k_gu, int k_down, int L, int T, void* workspace, size_t workspace_bytes,
                       void* stream);

/*
 * trellis_expand_bf16 -- out[r, c] = bf16(value(r, c) * scales[r]) for the
 * stored matrix (stored orientation; an axis-0 caller gets W^T).  value is
 * y/d correctly rounded to f32; the product is rounded to f32, then to bf16
 * (nearest even).
 * Source: trellis-linear.ts (page 55), EXPAND kernel and expandTrellis;
 * trellis-vector-expand.ts (page 56).
 *   codes uint32 [R, C*k/32];  scales fp16 [R];  out bf16 [R, C]
 */
int trellis_expand_bf16(const uint32_t* codes, const uint16_t* scales, uint16_t* out, int64_t R,
                        int64_t C, int k, int L, int T, void* stream);

/*
 * Block-interleaved layout of k = 3 axis-0 matrices: codes [C/512, R, 48]
 * uint32, i.e. for every pair of 256-column blocks (2g, 2g+1) the rows one
 * after another, each row's two 24-word blocks side by side.  Only k = 3,
 * L = 12, T = 256 and C % 512 == 0 (TRELLIS_EUNSUPPORTED / TRELLIS_EINVAL
 * otherwise).  The results equal those of the row-major calls on the same
 * symbols.
 * Source: mlx-bun 0.2.0 -> 0.4.0 diff (page 55), trellis-linear.ts file
 * header (the optional k3/axis0 layout) and trellisGeometry (3-D codes
 * [groups, rows, 48]); the SCATTER and EXPAND kernels' INTERLEAVE addressing.
 *
 * trellis_matvec_axis0_il -- trellis_matvec_axis0 on interleaved codes; the
 *   workspace size is trellis_matvec_axis0_workspace_bytes.
 * trellis_expand_bf16_il -- trellis_expand_bf16 on interleaved codes; out is
 *   bf16 [R, C] in stored orientation.
 */
int trellis_matvec_axis0_il(const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                            void* out, int out_dtype, int64_t R_in, int64_t C_out, int M, int k,
                            int L, int T, void* workspace, size_t workspace_bytes, void* stream);
int trellis_expand_bf16_il(const uint32_t* codes, const uint16_t* scales, uint16_t* out, int64_t R,
                           int64_t C, int k, int L, int T, void* stream);

/*
 * trellis_prefill -- out[m, r] = bf16(sum_c wb(r, c) * x[m, c]) for axis 1,
 * where wb is the expansion weight of trellis_expand_bf16; f32 accumulation.
 * Source: trellis-tiled-prefill.ts (page 56) and the expand-then-matmul
 * fallback of TrellisLinear.forward (page 55).
 * For M <= TRELLIS_MATVEC_MAX_M this is also the matvec contract of the
 * pages' decode variants 0-3 (trellis-linear.ts file header and HEADER
 * TRELLIS_ROUND, page 55): every weight rounded to bf16 (value * scale),
 * products with x summed in f32, the sum cast to bf16.  The matvec entry
 * points keep the default numerics (f32 weights); this call gives the
 * bf16-weight result of the same layer.
 *   codes uint32 [R, C*k/32];  scales fp16 [R];  x bf16 [M, C];  out bf16 [M, R]
 *   M >= 1;  algo = TRELLIS_PREFILL_FUSED, TRELLIS_PREFILL_EXPAND_GEMM or
 *   TRELLIS_PREFILL_AUTO.
 * The EXPAND_GEMM workspace holds the bf16 [R, C] expansion and the GEMM's
 * own scratch; the GEMM runs hipBLASLt's top heuristic for the shape until
 * trellis_prefill_tune picks the fastest candidate.  The GEMM plan is made
 * before the expansion is launched, so a GEMM that cannot be planned
 * launches nothing.  The FUSED
 * workspace holds x rewritten in the MFMA operand order (ceil(M/32)*32*C*2
 * bytes), then f32 partial sums: for M <= 64 those of the column chunks the
 * weight rows are split into ([S][M][R]); above, the partial tiles of output
 * tiles split along C when whole tiles would leave compute units idle (the
 * size of that part depends on the device's compute-unit count).
 * FUSED returns TRELLIS_EUNSUPPORTED when the rewritten x or the codes
 * (R*C*k/8 bytes) reach 2 GiB (its loads use 32-bit buffer offsets).
 */
size_t trellis_prefill_workspace_bytes(int64_t R, int64_t C, int64_t M, int k, int L, int T,
                                       int algo);
int trellis_prefill(const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                    uint16_t* out, int64_t R, int64_t C, int64_t M, int k, int L, int T, int algo,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * trellis_prefill_axis0 -- out[m, c] = bf16(sum_r wb(r, c) * x[m, r]) for a
 * matrix stored transposed (axis 0: codes W^T [R_in, C_out*k/32], coded
 * along the outputs), wb the expansion weight of trellis_expand_bf16; f32
 * accumulation.  The down projection of an MLP for more than
 * TRELLIS_MATVEC_MAX_M rows.
 * Source: mlx-bun 0.2.0 -> 0.4.0 diff (page 55), the expand-then-matmul
 * fallback of TrellisLinear.forward, here for the transposed layout of the
 * SCATTER kernel's matrices.
 *   codes uint32 [R_in, C_out*k/32];  scales fp16 [R_in]
 *   x bf16 [M, R_in];  out bf16 [M, C_out];  M >= 1
 * algo:
 *   TRELLIS_PREFILL_EXPAND_GEMM: the expansion (stored orientation,
 *     R_in*C_out*2 bytes) goes into the workspace, then one bf16 GEMM (the
 *     top heuristic until trellis_prefill_axis0_tune picks), planned before
 *     anything is launched, as in trellis_prefill.
 *   TRELLIS_PREFILL_FUSED: the fused kernel of trellis_prefill with the
 *     outputs C_out as the tile's weight rows and the stored rows R_in as
 *     the contraction; each weight is decoded once per 128 (M <= 256) or
 *     512 rows of x and written transposed into the LDS tile.  Needs R_in a
 *     multiple of 128 (else TRELLIS_EUNSUPPORTED; the workspace size query
 *     then returns 0).  Workspace: x in operand order, then f32 partial
 *     tiles, as for trellis_prefill.
 *   TRELLIS_PREFILL_AUTO: one of the two (see its definition).
 * At M <= TRELLIS_MATVEC_MAX_M: the variants 0-3 (bf16-weight) result of
 * the axis-0 matvec, as for trellis_prefill.
 */
size_t trellis_prefill_axis0_workspace_bytes(int64_t R_in, int64_t C_out, int64_t M, int k, int L, int T,
                                             int algo);
int trellis_prefill_axis0(const uint32_t* codes, const uint16_t* scales, const uint16_t* x, uint16_t* out,
                          int64_t R_in, int64_t C_out, int64_t M, int k, int L, int T, int algo,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * trellis_prefill_axis0_il -- trellis_prefill_axis0 on the block-interleaved
 * k = 3 layout (codes [C_out/512, R_in, 48], see trellis_matvec_axis0_il);
 * same algorithms, workspace (trellis_prefill_axis0_workspace_bytes) and
 * result bits as the row-major call on the same symbols.
 * Source: trellis-splitk-prefill.ts (page 56), the INTERLEAVE addressing of
 * its partial kernel; trellis-linear.ts (page 55) file header.
 */
int trellis_prefill_axis0_il(const uint32_t* codes, const uint16_t* scales, const uint16_t* x, uint16_t* out,
                             int64_t R_in, int64_t C_out, int64_t M, int k, int L, int T, int algo,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * trellis_prefill_tune / trellis_prefill_axis0_tune -- the EXPAND_GEMM
 * algorithm of trellis_prefill / trellis_prefill_axis0, once, after timing
 * every hipBLASLt candidate GEMM for this shape on the caller's buffers.
 * The fastest becomes the GEMM that later EXPAND_GEMM calls of the same
 * shape on this device enqueue (graph captures included).  These two calls
 * SYNCHRONISE the host (they wait for the timing runs) and are meant for
 * set-up, outside any stream capture.  Arguments, workspace and errors as
 * for the call they tune with algo = TRELLIS_PREFILL_EXPAND_GEMM; out
 * receives that call's result.  Which candidate wins can differ between
 * processes, and with it the GEMM's summation order: results stay within
 * the same contract, not bit-identical across tuned processes.
 */
int trellis_prefill_tune(const uint32_t* codes, const uint16_t* scales, const uint16_t* x, uint16_t* out,
                         int64_t R, int64_t C, int64_t M, int k, int L, int T, void* workspace,
                         size_t workspace_bytes, void* stream);
int trellis_prefill_axis0_tune(const uint32_t* codes, const uint16_t* scales, const uint16_t* x, uint16_t* out,
                               int64_t R_in, int64_t C_out, int64_t M, int k, int L, int T, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * trellis_decode_states -- test export of the decode primitive: for every
 * weight of the stored [R, C] matrix, its L-bit state, its 1MAD code y and
 * the f32 code value y/d (correctly rounded).  Any output may be NULL.
 * Source: trellis-linear.ts (page 55), HEADER (trellis_state, trellis_y,
 * trellis_val).
 *   states uint16 [R, C];  y int16 [R, C];  value f32 [R, C]
 */
int trellis_decode_states(const uint32_t* codes, int64_t R, int64_t C, int k, int L, int T,
                          uint16_t* states, int16_t* y, float* value, void* stream);

/*
 * Measurement probes: where the matvec kernels' time goes (the pages' decode
 * variant 4, "no decode, timing floor only", trellis-linear.ts HEADER, page
 * 55, and a decode without memory).  Not part of the layer's contract.
 *
 * trellis_probe_decode_only -- the matvec loop's decode and MFMAs with no
 * memory traffic.  Thread g of blocks * 512 threads decodes the 32-position
 * run held in runs[g][0 .. k] (k words and the word after them) `iters`
 * times, adding 1 to every word after each pass, and feeds each pass's codes
 * to the matvec kernels' MFMA against an all-ones operand.  wave_sums[w]
 * (blocks * 8 floats) receives 16 times the sum of the codes wave w decoded
 * (exact while each sum stays below 2^24).  Decoded weights per call:
 * blocks * 512 * iters * 32.  runs uint32 [blocks * 512][k + 1].
 *
 * trellis_probe_gateup_decode_free -- trellis_gateup_swiglu's kernel with
 * the raw code words in place of the decoded codes: the same copies,
 * MFMAs, prologue and epilogue, no decode.  out (bf16 [M, R]) receives
 * meaningless values.  One launch only (C <= 5120).
 */
int trellis_probe_decode_only(const uint32_t* runs, float* wave_sums, int blocks, int iters, int k,
                              void* stream);
int trellis_probe_gateup_decode_free(const uint32_t* gcodes, const uint16_t* gscales, const uint32_t* ucodes,
                                     const uint16_t* uscales, const uint16_t* x, uint16_t* out, int64_t R,
                                     int64_t C, int M, int k, int L, int T, void* stream);

/* Description of the last non-OK status on this thread ("" if none). */
const char* trellis_last_error(void);

/* Library version string. */
const char* trellis_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TRELLIS_H */
