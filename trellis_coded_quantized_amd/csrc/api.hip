// api.hip -- the C ABI (include/trellis.h): host-side validation, workspace
// sizing and dispatch onto the caller's stream.  Validation mirrors the
// pages' geometry checks before any launch (mlx-bun 0.2.0 -> 0.4.0 diff,
// page 55, trellis-linear.ts trellisGeometry and fusedGateUpEligible; page 56,
// the prefill eligibility predicates): nothing is launched or written unless
// every check passes.
#include <hipblaslt/hipblaslt.h>

#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <tuple>

#include "trellis.h"
#include "internal.hpp"

namespace trellis {

// Compute units of the current device, queried once per device.
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

}  // namespace trellis

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return TRELLIS_OK;
}

constexpr int64_t kMaxDim = (int64_t)1 << 31;      // R, C, M each below 2^31
constexpr int64_t kMaxElems = (int64_t)1 << 40;    // R * C, M * C, M * R

int check_geometry(const char* fn, int64_t R, int64_t C, int k, int L, int T) {
  if (k != 2 && k != 3 && k != 4) return fail(TRELLIS_EUNSUPPORTED, "%s: k=%d not in {2,3,4}", fn, k);
  if (L != 12) return fail(TRELLIS_EUNSUPPORTED, "%s: L=%d unsupported (L must be 12)", fn, L);
  if (T != 256) return fail(TRELLIS_EUNSUPPORTED, "%s: T=%d unsupported (T must be 256)", fn, T);
  if (R < 1 || C < 1) return fail(TRELLIS_EINVAL, "%s: empty matrix R=%lld C=%lld", fn, (long long)R, (long long)C);
  if (R >= kMaxDim || C >= kMaxDim || R * C >= kMaxElems)
    return fail(TRELLIS_EINVAL, "%s: matrix %lld x %lld too large", fn, (long long)R, (long long)C);
  if (C % T != 0)
    return fail(TRELLIS_EINVAL, "%s: C=%lld coded columns not a multiple of the block T=%d", fn, (long long)C, T);
  return TRELLIS_OK;
}

int check_ptr(const char* fn, const char* name, const void* p, size_t align) {
  if (!p) return fail(TRELLIS_EINVAL, "%s: %s is NULL", fn, name);
  if (reinterpret_cast<uintptr_t>(p) % align != 0)
    return fail(TRELLIS_EINVAL, "%s: %s not %zu-byte aligned", fn, name, align);
  return TRELLIS_OK;
}

int check_m(const char* fn, int64_t M, int64_t maxM) {
  if (M < 1 || M > maxM) return fail(TRELLIS_EINVAL, "%s: M=%lld outside 1..%lld", fn, (long long)M, (long long)maxM);
  return TRELLIS_OK;
}

int check_workspace(const char* fn, const void* ws, size_t have, size_t need) {
  if (need == 0) return TRELLIS_OK;
  if (have < need) return fail(TRELLIS_EWORKSPACE, "%s: workspace %zu bytes < required %zu", fn, have, need);
  return check_ptr(fn, "workspace", ws, 256);
}

// The axis-1 kernel keeps x in registers and a ring of 16-row code tiles in
// LDS, 5120 columns per launch; wider rows run as column chunks.
int check_axis1_shape(const char* fn, int64_t R, int64_t C, int M, int k, bool gateup) {
  if (!trellis::axis1_supported(R, C, M, k, gateup))
    return fail(TRELLIS_EUNSUPPORTED, "%s: C=%lld (M=%d, k=%d) does not fit the kernel's register / LDS plan",
                fn, (long long)C, M, k);
  return TRELLIS_OK;
}

// The block-interleaved k = 3 layout of axis-0 matrices: codes [C/512, R, 48].
int check_interleaved(const char* fn, int64_t C, int k) {
  if (k != 3) return fail(TRELLIS_EUNSUPPORTED, "%s: the interleaved layout is k=3 only (k=%d)", fn, k);
  if (C % 512 != 0)
    return fail(TRELLIS_EINVAL, "%s: C=%lld not a multiple of 512 (two blocks per group)", fn, (long long)C);
  return TRELLIS_OK;
}

int hip_status(const char* fn, hipError_t e) {
  if (e == hipSuccess) return ok();
  return fail(TRELLIS_EHIP, "%s: HIP error %d (%s)", fn, (int)e, hipGetErrorString(e));
}

#define TRY(expr)            \
  do {                       \
    int _rc = (expr);        \
    if (_rc != TRELLIS_OK) return _rc; \
  } while (0)

// ---- bf16 GEMM of the expand-then-GEMM prefill (hipBLASLt) --------------

constexpr size_t kGemmWorkspace = (size_t)64 << 20;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

constexpr int kGemmCandidates = 64;

struct GemmPlan {
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, lc = nullptr;
  hipblasLtMatmulAlgo_t algo;                                  // in use: cand[0] until a tune call picks
  hipblasLtMatmulHeuristicResult_t cand[kGemmCandidates];      // hipBLASLt's candidates, best first
  int ncand = 0;
};

std::mutex g_lt_mu;
std::map<int, hipblasLtHandle_t> g_lt_handles;
std::map<std::tuple<int, int64_t, int64_t, int64_t, int>, GemmPlan> g_lt_plans;

// Axis 1 (nn = false): out[M, R] (row-major) = x[M, C] * W[R, C]^T.
// Column-major view: D (R x M, ld R) = op_T(A: C x R, ld C) * op_N(B: C x M, ld C).
// Axis 0 (nn = true): out[M, R] = x[M, C] * W[C, R], W the stored [C, R]
// expansion.  Column-major view: D (R x M, ld R) = op_N(A: R x C, ld R) * op_N(B: C x M, ld C).
//
// The handle and plan of a shape are made before anything is launched, so
// a failure here leaves the stream untouched.  Caller holds g_lt_mu.
int gemm_plan_locked(const char* fn, int64_t R, int64_t C, int64_t M, bool nn, GemmPlan** plan,
                     hipblasLtHandle_t* handle) {
  int dev = 0;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return hip_status(fn, he);
  auto hit = g_lt_handles.find(dev);
  if (hit == g_lt_handles.end()) {
    hipblasLtHandle_t h = nullptr;
    if (hipblasLtCreate(&h) != HIPBLAS_STATUS_SUCCESS) return fail(TRELLIS_EHIP, "%s: hipblasLtCreate failed", fn);
    hit = g_lt_handles.emplace(dev, h).first;
  }
  hipblasLtHandle_t h = hit->second;
  auto key = std::make_tuple(dev, R, C, M, nn ? 1 : 0);
  auto pit = g_lt_plans.find(key);
  if (pit == g_lt_plans.end()) {
    GemmPlan p;
    hipblasOperation_t ta = nn ? HIPBLAS_OP_N : HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
    uint64_t wsb = kGemmWorkspace;
    hipblasLtMatmulPreference_t pref = nullptr;
    int returned = 0;
    bool good = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS &&
                hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)) == HIPBLAS_STATUS_SUCCESS &&
                hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)) == HIPBLAS_STATUS_SUCCESS &&
                (nn ? hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, (uint64_t)R, (uint64_t)C, R)
                    : hipblasLtMatrixLayoutCreate(&p.la, HIP_R_16BF, (uint64_t)C, (uint64_t)R, C)) == HIPBLAS_STATUS_SUCCESS &&
                hipblasLtMatrixLayoutCreate(&p.lb, HIP_R_16BF, (uint64_t)C, (uint64_t)M, C) == HIPBLAS_STATUS_SUCCESS &&
                hipblasLtMatrixLayoutCreate(&p.lc, HIP_R_16BF, (uint64_t)R, (uint64_t)M, R) == HIPBLAS_STATUS_SUCCESS &&
                hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
                hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb, sizeof(wsb)) == HIPBLAS_STATUS_SUCCESS &&
                hipblasLtMatmulAlgoGetHeuristic(h, p.desc, p.la, p.lb, p.lc, p.lc, pref, kGemmCandidates, p.cand, &returned) == HIPBLAS_STATUS_SUCCESS &&
                returned > 0;
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    if (!good) {
      if (p.la) hipblasLtMatrixLayoutDestroy(p.la);
      if (p.lb) hipblasLtMatrixLayoutDestroy(p.lb);
      if (p.lc) hipblasLtMatrixLayoutDestroy(p.lc);
      if (p.desc) hipblasLtMatmulDescDestroy(p.desc);
      return fail(TRELLIS_EHIP, "%s: no hipBLASLt bf16 GEMM for %lld x %lld x %lld", fn, (long long)M,
                  (long long)R, (long long)C);
    }
    p.algo = p.cand[0].algo;
    p.ncand = returned;
    pit = g_lt_plans.emplace(key, p).first;
  }
  *plan = &pit->second;
  *handle = h;
  return TRELLIS_OK;
}

// Enqueue the GEMM with the plan's algorithm (no host synchronisation).
// Caller holds g_lt_mu.
int gemm_run_locked(const char* fn, const GemmPlan& p, hipblasLtHandle_t h, const uint16_t* W, const uint16_t* x,
                    uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  const float alpha = 1.0f, beta = 0.0f;
  hipblasStatus_t st = hipblasLtMatmul(h, p.desc, &alpha, W, p.la, x, p.lb, &beta, out, p.lc, out,
                                       p.lc, &p.algo, ws, ws_bytes, stream);
  if (st != HIPBLAS_STATUS_SUCCESS) return fail(TRELLIS_EHIP, "%s: hipblasLtMatmul status %d", fn, (int)st);
  return ok();
}

// Time every candidate on the caller's buffers (each writes the same
// product into out) and keep the fastest in the plan.  Synchronises the
// host; only the explicit tune calls come here.  Caller holds g_lt_mu.
int gemm_tune_locked(const char* fn, GemmPlan& tp, hipblasLtHandle_t h, const uint16_t* W, const uint16_t* x,
                     uint16_t* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    return fail(TRELLIS_EHIP, "%s: hipEventCreate failed", fn);
  }
  const float alpha = 1.0f, beta = 0.0f;
  float best = -1.0f;
  for (int i = 0; i < tp.ncand; ++i) {
    if (tp.cand[i].workspaceSize > ws_bytes) continue;
    bool run_ok = hipblasLtMatmul(h, tp.desc, &alpha, W, tp.la, x, tp.lb, &beta, out, tp.lc, out, tp.lc,
                                  &tp.cand[i].algo, ws, ws_bytes, stream) == HIPBLAS_STATUS_SUCCESS;
    run_ok = run_ok && hipEventRecord(e0, stream) == hipSuccess;
    for (int rep = 0; run_ok && rep < 3; ++rep)
      run_ok = hipblasLtMatmul(h, tp.desc, &alpha, W, tp.la, x, tp.lb, &beta, out, tp.lc, out, tp.lc,
                               &tp.cand[i].algo, ws, ws_bytes, stream) == HIPBLAS_STATUS_SUCCESS;
    run_ok = run_ok && hipEventRecord(e1, stream) == hipSuccess && hipEventSynchronize(e1) == hipSuccess;
    float ms = 0.0f;
    if (run_ok && hipEventElapsedTime(&ms, e0, e1) == hipSuccess && (best < 0.0f || ms < best)) {
      best = ms;
      tp.algo = tp.cand[i].algo;
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  const hipError_t le = hipGetLastError();
  if (best < 0.0f) return fail(TRELLIS_EHIP, "%s: no hipBLASLt candidate ran (%s)", fn, hipGetErrorString(le));
  return ok();
}

// Expansion into the workspace, then the GEMM: out = x times the expansion
// (axis 1: W [R_out, C_con]; axis 0: the stored W^T [C_con, R_out]).  The
// plan is made first, so a GEMM that cannot be planned launches nothing.
int expand_gemm(const char* fn, const uint32_t* codes, const uint16_t* scales, const uint16_t* x, uint16_t* out,
                int64_t R_out, int64_t C_con, int64_t M, int k, bool axis0, int interleave, bool tune,
                void* workspace, size_t workspace_bytes, hipStream_t s) {
  std::lock_guard<std::mutex> lock(g_lt_mu);
  GemmPlan* plan = nullptr;
  hipblasLtHandle_t h = nullptr;
  TRY(gemm_plan_locked(fn, R_out, C_con, M, axis0, &plan, &h));
  uint16_t* wexp = reinterpret_cast<uint16_t*>(workspace);
  const size_t wexp_bytes = align_up((size_t)R_out * (size_t)C_con * 2, 256);
  const int64_t er = axis0 ? C_con : R_out, ec = axis0 ? R_out : C_con;   // stored orientation
  TRY(hip_status(fn, trellis::launch_expand(codes, scales, wexp, er, ec, k, s, interleave)));
  void* gws = reinterpret_cast<char*>(workspace) + wexp_bytes;
  const size_t gws_bytes = workspace_bytes - wexp_bytes;
  if (tune) TRY(gemm_tune_locked(fn, *plan, h, wexp, x, out, gws, gws_bytes, s));
  return gemm_run_locked(fn, *plan, h, wexp, x, out, gws, gws_bytes, s);
}

}  // namespace

extern "C" {

const char* trellis_last_error(void) { return g_err; }

const char* trellis_version(void) { return "trellis-mi355x 0.1.0 (gfx950)"; }

size_t trellis_matvec_axis1_workspace_bytes(int64_t R, int64_t C, int M, int k, int L, int T) {
  if (check_geometry("trellis_matvec_axis1_workspace_bytes", R, C, k, L, T) != TRELLIS_OK) return 0;
  if (M < 1 || M > TRELLIS_MATVEC_MAX_M) return 0;
  return trellis::axis1_workspace_bytes(R, C, M, k, false);
}

int trellis_matvec_axis1(const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                         void* out, int out_dtype, int64_t R, int64_t C, int M, int k, int L,
                         int T, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "trellis_matvec_axis1";
  TRY(check_geometry(fn, R, C, k, L, T));
  TRY(check_m(fn, M, TRELLIS_MATVEC_MAX_M));
  if (out_dtype != TRELLIS_OUT_BF16 && out_dtype != TRELLIS_OUT_F32)
    return fail(TRELLIS_EINVAL, "%s: out_dtype=%d unknown", fn, out_dtype);
  TRY(check_ptr(fn, "codes", codes, 16));
  TRY(check_ptr(fn, "scales", scales, 2));
  TRY(check_ptr(fn, "x", x, 16));
  TRY(check_ptr(fn, "out", out, 16));
  TRY(check_workspace(fn, workspace, workspace_bytes, trellis::axis1_workspace_bytes(R, C, M, k, false)));
  TRY(check_axis1_shape(fn, R, C, M, k, false));
  return hip_status(fn, trellis::launch_axis1(codes, scales, nullptr, nullptr, x, out,
                                              out_dtype == TRELLIS_OUT_F32, nullptr, nullptr, R, C,
                                              M, k, workspace, (hipStream_t)stream));
}

int trellis_matvec_axis1_group(const uint32_t* const* codes, const uint16_t* const* scales, void* const* out,
                               const int64_t* R, int n, const uint16_t* x, int out_dtype, int64_t C, int M,
                               int k, int L, int T, void* stream) {
  const char* fn = "trellis_matvec_axis1_group";
  if (n < 1 || n > TRELLIS_GROUP_MAX)
    return fail(TRELLIS_EINVAL, "%s: n=%d matrices, must be 1..%d", fn, n, TRELLIS_GROUP_MAX);
  if (!codes || !scales || !out || !R) return fail(TRELLIS_EINVAL, "%s: NULL pointer array", fn);
  TRY(check_m(fn, M, TRELLIS_MATVEC_MAX_M));
  if (out_dtype != TRELLIS_OUT_BF16 && out_dtype != TRELLIS_OUT_F32)
    return fail(TRELLIS_EINVAL, "%s: out_dtype=%d unknown", fn, out_dtype);
  TRY(check_ptr(fn, "x", x, 16));
  for (int j = 0; j < n; ++j) {
    TRY(check_geometry(fn, R[j], C, k, L, T));
    TRY(check_ptr(fn, "codes[j]", codes[j], 16));
    TRY(check_ptr(fn, "scales[j]", scales[j], 2));
    TRY(check_ptr(fn, "out[j]", out[j], 16));
  }
  if (!trellis::axis1_group_supported(R, n, C, M, k))
    return fail(TRELLIS_EUNSUPPORTED, "%s: %d matrices of C=%lld do not fit one launch (C <= 5120)", fn, n,
                (long long)C);
  return hip_status(fn, trellis::launch_axis1_group(codes, scales, out, R, n, x, out_dtype == TRELLIS_OUT_F32,
                                                    C, M, k, (hipStream_t)stream));
}

size_t trellis_gateup_swiglu_workspace_bytes(int64_t R, int64_t C, int M, int k, int L, int T) {
  if (check_geometry("trellis_gateup_swiglu_workspace_bytes", R, C, k, L, T) != TRELLIS_OK) return 0;
  if (M < 1 || M > TRELLIS_MATVEC_MAX_M) return 0;
  return trellis::axis1_workspace_bytes(R, C, M, k, true);
}

int trellis_gateup_swiglu(const uint32_t* gcodes, const uint16_t* gscales, const uint32_t* ucodes,
                          const uint16_t* uscales, const uint16_t* x, uint16_t* out,
                          float* gate_f32, float* up_f32, int64_t R, int64_t C, int M, int k,
                          int L, int T, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "trellis_gateup_swiglu";
  TRY(check_geometry(fn, R, C, k, L, T));
  TRY(check_m(fn, M, TRELLIS_MATVEC_MAX_M));
  TRY(check_ptr(fn, "gcodes", gcodes, 16));
  TRY(check_ptr(fn, "gscales", gscales, 2));
  TRY(check_ptr(fn, "ucodes", ucodes, 16));
  TRY(check_ptr(fn, "uscales", uscales, 2));
  TRY(check_ptr(fn, "x", x, 16));
  TRY(check_ptr(fn, "out", out, 16));
  if (gate_f32) TRY(check_ptr(fn, "gate_f32", gate_f32, 4));
  if (up_f32) TRY(check_ptr(fn, "up_f32", up_f32, 4));
  TRY(check_workspace(fn, workspace, workspace_bytes, trellis::axis1_workspace_bytes(R, C, M, k, true)));
  TRY(check_axis1_shape(fn, R, C, M, k, true));
  return hip_status(fn, trellis::launch_axis1(gcodes, gscales, ucodes, uscales, x, out, 0, gate_f32,
                                              up_f32, R, C, M, k, workspace, (hipStream_t)stream));
}

size_t trellis_matvec_axis0_workspace_bytes(int64_t R_in, int64_t C_out, int M, int k, int L, int T) {
  if (check_geometry("trellis_matvec_axis0_workspace_bytes", R_in, C_out, k, L, T) != TRELLIS_OK) return 0;
  if (M < 1 || M > TRELLIS_MATVEC_MAX_M) return 0;
  return trellis::axis0_workspace_bytes(R_in, C_out, M, k);
}

int trellis_matvec_axis0(const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                         void* out, int out_dtype, int64_t R_in, int64_t C_out, int M, int k,
                         int L, int T, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "trellis_matvec_axis0";
  TRY(check_geometry(fn, R_in, C_out, k, L, T));
  TRY(check_m(fn, M, TRELLIS_MATVEC_MAX_M));
  if (out_dtype != TRELLIS_OUT_BF16 && out_dtype != TRELLIS_OUT_F32)
    return fail(TRELLIS_EINVAL, "%s: out_dtype=%d unknown", fn, out_dtype);
  TRY(check_ptr(fn, "codes", codes, 16));
  TRY(check_ptr(fn, "scales", scales, 2));
  TRY(check_ptr(fn, "x", x, 16));
  TRY(check_ptr(fn, "out", out, 16));
  if (!trellis::axis0_supported(R_in, C_out, M, k))
    return fail(TRELLIS_EUNSUPPORTED, "%s: shape R=%lld C=%lld M=%d k=%d does not fit the kernel's LDS plan", fn,
                (long long)R_in, (long long)C_out, M, k);
  TRY(check_workspace(fn, workspace, workspace_bytes, trellis::axis0_workspace_bytes(R_in, C_out, M, k)));
  return hip_status(fn, trellis::launch_axis0(codes, scales, x, out, out_dtype == TRELLIS_OUT_F32,
                                              R_in, C_out, M, k, workspace, (hipStream_t)stream));
}

int trellis_matvec_axis0_noalloc(const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                                 void* out, int out_dtype, int64_t R_in, int64_t C_out, int M, int k,
                                 int L, int T, void* stream) {
  const char* fn = "trellis_matvec_axis0_noalloc";
  TRY(check_geometry(fn, R_in, C_out, k, L, T));
  TRY(check_m(fn, M, TRELLIS_MATVEC_MAX_M));
  if (out_dtype != TRELLIS_OUT_BF16 && out_dtype != TRELLIS_OUT_F32)
    return fail(TRELLIS_EINVAL, "%s: out_dtype=%d unknown", fn, out_dtype);
  TRY(check_ptr(fn, "codes", codes, 16));
  TRY(check_ptr(fn, "scales", scales, 2));
  TRY(check_ptr(fn, "x", x, 16));
  TRY(check_ptr(fn, "out", out, 16));
  if (!trellis::axis0_supported(R_in, C_out, M, k))
    return fail(TRELLIS_EUNSUPPORTED, "%s: shape R=%lld C=%lld M=%d k=%d does not fit the kernel's LDS plan", fn,
                (long long)R_in, (long long)C_out, M, k);
  const size_t need = trellis::axis0_workspace_bytes(R_in, C_out, M, k);
  if (need > trellis::kAxis0ScratchBytes)
    return fail(TRELLIS_EUNSUPPORTED, "%s: the split partials need %zu bytes, beyond the %zu-byte static scratch "
                "(use trellis_matvec_axis0 with a workspace)", fn, need, trellis::kAxis0ScratchBytes);
  void* scratch = nullptr;
  TRY(hip_status(fn, trellis::axis0_scratch(&scratch)));
  return hip_status(fn, trellis::launch_axis0(codes, scales, x, out, out_dtype == TRELLIS_OUT_F32, R_in, C_out, M,
                                              k, scratch, (hipStream_t)stream));
}

size_t trellis_mlp_decode_workspace_bytes(int64_t R, int64_t C, int64_t C_out, int M, int k_gu,
                                          int k_down, int L, int T) {
  if (check_geometry("trellis_mlp_decode_workspace_bytes", R, C, k_gu, L, T) != TRELLIS_OK) return 0;
  if (check_geometry("trellis_mlp_decode_workspace_bytes", R, C_out, k_down, L, T) != TRELLIS_OK) return 0;
  if (M < 1 || M > TRELLIS_MATVEC_MAX_M) return 0;
  // the bf16 hidden vectors [M, R], then the down projection's own workspace
  return align_up((size_t)M * (size_t)R * 2, 256) + align_up(trellis::axis1_workspace_bytes(R, C, M, k_gu, true), 256) +
         trellis::axis0_workspace_bytes(R, C_out, M, k_down);
}

int trellis_mlp_decode(const uint32_t* gcodes, const uint16_t* gscales, const uint32_t* ucodes,
                       const uint16_t* uscales, const uint32_t* dcodes, const uint16_t* dscales,
                       const uint16_t* x, uint16_t* hidden, uint16_t* out, int64_t R, int64_t C, int64_t C_out,
                       int M, int k_gu, int k_down, int L, int T, void* workspace, size_t workspace_bytes,
                       void* stream) {
  const char* fn = "trellis_mlp_decode";
  TRY(check_geometry(fn, R, C, k_gu, L, T));
  TRY(check_geometry(fn, R, C_out, k_down, L, T));
  TRY(check_m(fn, M, TRELLIS_MATVEC_MAX_M));
  TRY(check_ptr(fn, "gcodes", gcodes, 16));
  TRY(check_ptr(fn, "gscales", gscales, 2));
  TRY(check_ptr(fn, "ucodes", ucodes, 16));
  TRY(check_ptr(fn, "uscales", uscales, 2));
  TRY(check_ptr(fn, "dcodes", dcodes, 16));
  TRY(check_ptr(fn, "dscales", dscales, 2));
  TRY(check_ptr(fn, "x", x, 16));
  TRY(check_ptr(fn, "out", out, 16));
  if (hidden) TRY(check_ptr(fn, "hidden", hidden, 16));
  TRY(check_axis1_shape(fn, R, C, M, k_gu, true));
  if (!trellis::axis0_supported(R, C_out, M, k_down))
    return fail(TRELLIS_EUNSUPPORTED, "%s: down shape R=%lld C_out=%lld M=%d k=%d does not fit the kernel's LDS plan",
                fn, (long long)R, (long long)C_out, M, k_down);
  TRY(check_workspace(fn, workspace, workspace_bytes,
                      trellis_mlp_decode_workspace_bytes(R, C, C_out, M, k_gu, k_down, L, T)));
  char* ws = reinterpret_cast<char*>(workspace);
  const size_t hb = align_up((size_t)M * (size_t)R * 2, 256);
  const size_t w1 = align_up(trellis::axis1_workspace_bytes(R, C, M, k_gu, true), 256);
  uint16_t* mid = hidden ? hidden : reinterpret_cast<uint16_t*>(ws);
  hipStream_t s = (hipStream_t)stream;
  TRY(hip_status(fn, trellis::launch_axis1(gcodes, gscales, ucodes, uscales, x, mid, 0, nullptr, nullptr, R, C,
                                           M, k_gu, w1 ? ws + hb : nullptr, s)));
  return hip_status(fn, trellis::launch_axis0(dcodes, dscales, mid, out, 0, R, C_out, M, k_down, ws + hb + w1, s));
}

int trellis_matvec_axis0_il(const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                            void* out, int out_dtype, int64_t R_in, int64_t C_out, int M, int k,
                            int L, int T, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "trellis_matvec_axis0_il";
  TRY(check_geometry(fn, R_in, C_out, k, L, T));
  TRY(check_interleaved(fn, C_out, k));
  TRY(check_m(fn, M, TRELLIS_MATVEC_MAX_M));
  if (out_dtype != TRELLIS_OUT_BF16 && out_dtype != TRELLIS_OUT_F32)
    return fail(TRELLIS_EINVAL, "%s: out_dtype=%d unknown", fn, out_dtype);
  TRY(check_ptr(fn, "codes", codes, 16));
  TRY(check_ptr(fn, "scales", scales, 2));
  TRY(check_ptr(fn, "x", x, 16));
  TRY(check_ptr(fn, "out", out, 16));
  if (!trellis::axis0_supported(R_in, C_out, M, k))
    return fail(TRELLIS_EUNSUPPORTED, "%s: shape R=%lld C=%lld M=%d k=%d does not fit the kernel's LDS plan", fn,
                (long long)R_in, (long long)C_out, M, k);
  TRY(check_workspace(fn, workspace, workspace_bytes, trellis::axis0_workspace_bytes(R_in, C_out, M, k)));
  return hip_status(fn, trellis::launch_axis0(codes, scales, x, out, out_dtype == TRELLIS_OUT_F32, R_in, C_out,
                                              M, k, workspace, (hipStream_t)stream, 1));
}

int trellis_expand_bf16_il(const uint32_t* codes, const uint16_t* scales, uint16_t* out, int64_t R,
                           int64_t C, int k, int L, int T, void* stream) {
  const char* fn = "trellis_expand_bf16_il";
  TRY(check_geometry(fn, R, C, k, L, T));
  TRY(check_interleaved(fn, C, k));
  TRY(check_ptr(fn, "codes", codes, 16));
  TRY(check_ptr(fn, "scales", scales, 2));
  TRY(check_ptr(fn, "out", out, 16));
  return hip_status(fn, trellis::launch_expand(codes, scales, out, R, C, k, (hipStream_t)stream, 1));
}

int trellis_expand_bf16(const uint32_t* codes, const uint16_t* scales, uint16_t* out, int64_t R,
                        int64_t C, int k, int L, int T, void* stream) {
  const char* fn = "trellis_expand_bf16";
  TRY(check_geometry(fn, R, C, k, L, T));
  TRY(check_ptr(fn, "codes", codes, 16));
  TRY(check_ptr(fn, "scales", scales, 2));
  TRY(check_ptr(fn, "out", out, 16));
  return hip_status(fn, trellis::launch_expand(codes, scales, out, R, C, k, (hipStream_t)stream));
}

namespace {

// TRELLIS_PREFILL_AUTO: the fused kernel up to the M where it measured at
// least as fast as expansion + GEMM on 17408 x 5120, else expansion + GEMM.
// Axis 1: one 128-row x tile, M <= 128 (at M = 256 the weights are decoded
// twice and the GEMM is faster).  Axis 0: M <= 512 (the transposed GEMM is
// slower there; from M = 768 it wins).  R_out: outputs, C_con: contraction.
constexpr int64_t kAutoFusedMaxM = 128;
constexpr int64_t kAutoFusedMaxMAxis0 = 512;

int resolve_prefill_algo(int algo, int64_t R_out, int64_t C_con, int64_t M, int k, bool axis0) {
  if (algo != TRELLIS_PREFILL_AUTO) return algo;
  const int64_t max_m = axis0 ? kAutoFusedMaxMAxis0 : kAutoFusedMaxM;
  return M <= max_m && trellis::prefill_fused_supported(R_out, C_con, M, k) ? TRELLIS_PREFILL_FUSED
                                                                            : TRELLIS_PREFILL_EXPAND_GEMM;
}

}  // namespace

size_t trellis_prefill_workspace_bytes(int64_t R, int64_t C, int64_t M, int k, int L, int T,
                                       int algo) {
  if (check_geometry("trellis_prefill_workspace_bytes", R, C, k, L, T) != TRELLIS_OK) return 0;
  if (M < 1) return 0;
  algo = resolve_prefill_algo(algo, R, C, M, k, false);
  if (algo == TRELLIS_PREFILL_EXPAND_GEMM) return align_up((size_t)R * (size_t)C * 2, 256) + kGemmWorkspace;
  if (algo != TRELLIS_PREFILL_FUSED || !trellis::prefill_fused_supported(R, C, M, k)) return 0;
  return trellis::prefill_fused_workspace_bytes(R, C, M);
}

namespace {

int prefill_common(const char* fn, const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                   uint16_t* out, int64_t R, int64_t C, int64_t M, int k, int L, int T, int& algo, bool tune,
                   void* workspace, size_t workspace_bytes) {
  TRY(check_geometry(fn, R, C, k, L, T));
  TRY(check_m(fn, M, kMaxDim - 1));
  if (M * C >= kMaxElems || M * R >= kMaxElems)
    return fail(TRELLIS_EINVAL, "%s: M=%lld too large", fn, (long long)M);
  if (M > (int64_t)65535 * 128) return fail(TRELLIS_EINVAL, "%s: M=%lld too large", fn, (long long)M);
  if (tune) algo = TRELLIS_PREFILL_EXPAND_GEMM;
  if (algo != TRELLIS_PREFILL_FUSED && algo != TRELLIS_PREFILL_EXPAND_GEMM && algo != TRELLIS_PREFILL_AUTO)
    return fail(TRELLIS_EINVAL, "%s: algo=%d unknown", fn, algo);
  algo = resolve_prefill_algo(algo, R, C, M, k, false);
  TRY(check_ptr(fn, "codes", codes, 16));
  TRY(check_ptr(fn, "scales", scales, 2));
  TRY(check_ptr(fn, "x", x, 16));
  TRY(check_ptr(fn, "out", out, 16));
  if (algo == TRELLIS_PREFILL_FUSED && !trellis::prefill_fused_supported(R, C, M, k))
    return fail(TRELLIS_EUNSUPPORTED, "%s: fused kernel needs x and codes below 2 GiB (M=%lld R=%lld C=%lld)",
                fn, (long long)M, (long long)R, (long long)C);
  return check_workspace(fn, workspace, workspace_bytes, trellis_prefill_workspace_bytes(R, C, M, k, L, T, algo));
}

}  // namespace

int trellis_prefill(const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                    uint16_t* out, int64_t R, int64_t C, int64_t M, int k, int L, int T, int algo,
                    void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "trellis_prefill";
  TRY(prefill_common(fn, codes, scales, x, out, R, C, M, k, L, T, algo, false, workspace, workspace_bytes));
  hipStream_t s = (hipStream_t)stream;
  if (algo == TRELLIS_PREFILL_FUSED)
    return hip_status(fn, trellis::launch_prefill_fused(codes, scales, x, out, R, C, M, k, workspace, s));
  return expand_gemm(fn, codes, scales, x, out, R, C, M, k, false, 0, false, workspace, workspace_bytes, s);
}

int trellis_prefill_tune(const uint32_t* codes, const uint16_t* scales, const uint16_t* x, uint16_t* out,
                         int64_t R, int64_t C, int64_t M, int k, int L, int T, void* workspace,
                         size_t workspace_bytes, void* stream) {
  const char* fn = "trellis_prefill_tune";
  int algo = TRELLIS_PREFILL_EXPAND_GEMM;
  TRY(prefill_common(fn, codes, scales, x, out, R, C, M, k, L, T, algo, true, workspace, workspace_bytes));
  return expand_gemm(fn, codes, scales, x, out, R, C, M, k, false, 0, true, workspace, workspace_bytes,
                     (hipStream_t)stream);
}

size_t trellis_prefill_axis0_workspace_bytes(int64_t R_in, int64_t C_out, int64_t M, int k, int L, int T,
                                             int algo) {
  if (check_geometry("trellis_prefill_axis0_workspace_bytes", R_in, C_out, k, L, T) != TRELLIS_OK) return 0;
  if (M < 1) return 0;
  algo = resolve_prefill_algo(algo, C_out, R_in, M, k, true);
  if (algo == TRELLIS_PREFILL_FUSED)   // outputs C_out, contraction R_in
    return trellis::prefill_fused_supported(C_out, R_in, M, k) ? trellis::prefill_fused_workspace_bytes(C_out, R_in, M, 1)
                                                                 : 0;
  if (algo != TRELLIS_PREFILL_EXPAND_GEMM) return 0;
  return align_up((size_t)R_in * (size_t)C_out * 2, 256) + kGemmWorkspace;
}

namespace {

int prefill_axis0_common(const char* fn, const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                         uint16_t* out, int64_t R_in, int64_t C_out, int64_t M, int k, int L, int T, int& algo,
                         bool tune, int interleave, void* workspace, size_t workspace_bytes) {
  TRY(check_geometry(fn, R_in, C_out, k, L, T));
  if (interleave) TRY(check_interleaved(fn, C_out, k));
  TRY(check_m(fn, M, kMaxDim - 1));
  if (M * C_out >= kMaxElems || M * R_in >= kMaxElems)
    return fail(TRELLIS_EINVAL, "%s: M=%lld too large", fn, (long long)M);
  if (M > (int64_t)65535 * 128) return fail(TRELLIS_EINVAL, "%s: M=%lld too large", fn, (long long)M);
  if (tune) algo = TRELLIS_PREFILL_EXPAND_GEMM;
  if (algo != TRELLIS_PREFILL_FUSED && algo != TRELLIS_PREFILL_EXPAND_GEMM && algo != TRELLIS_PREFILL_AUTO)
    return fail(TRELLIS_EINVAL, "%s: algo=%d unknown", fn, algo);
  algo = resolve_prefill_algo(algo, C_out, R_in, M, k, true);
  if (algo == TRELLIS_PREFILL_FUSED && !trellis::prefill_fused_supported(C_out, R_in, M, k))
    return fail(TRELLIS_EUNSUPPORTED,
                "%s: fused kernel needs R_in a multiple of 128 and x and codes below 2 GiB (M=%lld R_in=%lld "
                "C_out=%lld)",
                fn, (long long)M, (long long)R_in, (long long)C_out);
  TRY(check_ptr(fn, "codes", codes, 16));
  TRY(check_ptr(fn, "scales", scales, 2));
  TRY(check_ptr(fn, "x", x, 16));
  TRY(check_ptr(fn, "out", out, 16));
  return check_workspace(fn, workspace, workspace_bytes,
                         trellis_prefill_axis0_workspace_bytes(R_in, C_out, M, k, L, T, algo));
}

int prefill_axis0_run(const char* fn, const uint32_t* codes, const uint16_t* scales, const uint16_t* x,
                      uint16_t* out, int64_t R_in, int64_t C_out, int64_t M, int k, int algo, bool tune,
                      int interleave, void* workspace, size_t workspace_bytes, hipStream_t s) {
  if (algo == TRELLIS_PREFILL_FUSED)
    return hip_status(fn, trellis::launch_prefill_fused(codes, scales, x, out, C_out, R_in, M, k, workspace, s, 1,
                                                        interleave));
  return expand_gemm(fn, codes, scales, x, out, C_out, R_in, M, k, true, interleave, tune, workspace,
                     workspace_bytes, s);
}

}  // namespace

int trellis_prefill_axis0(const uint32_t* codes, const uint16_t* scales, const uint16_t* x, uint16_t* out,
                          int64_t R_in, int64_t C_out, int64_t M, int k, int L, int T, int algo,
                          void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "trellis_prefill_axis0";
  TRY(prefill_axis0_common(fn, codes, scales, x, out, R_in, C_out, M, k, L, T, algo, false, 0, workspace,
                           workspace_bytes));
  return prefill_axis0_run(fn, codes, scales, x, out, R_in, C_out, M, k, algo, false, 0, workspace, workspace_bytes,
                           (hipStream_t)stream);
}

int trellis_prefill_axis0_il(const uint32_t* codes, const uint16_t* scales, const uint16_t* x, uint16_t* out,
                             int64_t R_in, int64_t C_out, int64_t M, int k, int L, int T, int algo,
                             void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "trellis_prefill_axis0_il";
  TRY(prefill_axis0_common(fn, codes, scales, x, out, R_in, C_out, M, k, L, T, algo, false, 1, workspace,
                           workspace_bytes));
  return prefill_axis0_run(fn, codes, scales, x, out, R_in, C_out, M, k, algo, false, 1, workspace, workspace_bytes,
                           (hipStream_t)stream);
}

int trellis_prefill_axis0_tune(const uint32_t* codes, const uint16_t* scales, const uint16_t* x, uint16_t* out,
                               int64_t R_in, int64_t C_out, int64_t M, int k, int L, int T, void* workspace,
                               size_t workspace_bytes, void* stream) {
  const char* fn = "trellis_prefill_axis0_tune";
  int algo = TRELLIS_PREFILL_EXPAND_GEMM;
  TRY(prefill_axis0_common(fn, codes, scales, x, out, R_in, C_out, M, k, L, T, algo, true, 0, workspace,
                           workspace_bytes));
  return prefill_axis0_run(fn, codes, scales, x, out, R_in, C_out, M, k, algo, true, 0, workspace, workspace_bytes,
                           (hipStream_t)stream);
}

int trellis_probe_decode_only(const uint32_t* runs, float* wave_sums, int blocks, int iters, int k,
                              void* stream) {
  const char* fn = "trellis_probe_decode_only";
  if (k != 2 && k != 3 && k != 4) return fail(TRELLIS_EUNSUPPORTED, "%s: k=%d not in {2,3,4}", fn, k);
  if (blocks < 1 || blocks > 65535) return fail(TRELLIS_EINVAL, "%s: blocks=%d outside 1..65535", fn, blocks);
  if (iters < 1) return fail(TRELLIS_EINVAL, "%s: iters=%d < 1", fn, iters);
  TRY(check_ptr(fn, "runs", runs, 4));
  TRY(check_ptr(fn, "wave_sums", wave_sums, 4));
  return hip_status(fn, trellis::launch_decode_only(runs, wave_sums, blocks, iters, k, (hipStream_t)stream));
}

int trellis_probe_gateup_decode_free(const uint32_t* gcodes, const uint16_t* gscales, const uint32_t* ucodes,
                                     const uint16_t* uscales, const uint16_t* x, uint16_t* out, int64_t R,
                                     int64_t C, int M, int k, int L, int T, void* stream) {
  const char* fn = "trellis_probe_gateup_decode_free";
  TRY(check_geometry(fn, R, C, k, L, T));
  TRY(check_m(fn, M, TRELLIS_MATVEC_MAX_M));
  TRY(check_ptr(fn, "gcodes", gcodes, 16));
  TRY(check_ptr(fn, "gscales", gscales, 2));
  TRY(check_ptr(fn, "ucodes", ucodes, 16));
  TRY(check_ptr(fn, "uscales", uscales, 2));
  TRY(check_ptr(fn, "x", x, 16));
  TRY(check_ptr(fn, "out", out, 16));
  if (trellis::axis1_workspace_bytes(R, C, M, k, true) != 0 || !trellis::axis1_supported(R, C, M, k, true))
    return fail(TRELLIS_EUNSUPPORTED, "%s: one launch only (C <= 5120), C=%lld", fn, (long long)C);
  return hip_status(fn, trellis::launch_gateup_decode_free(gcodes, gscales, ucodes, uscales, x, out, R, C, M, k,
                                                           (hipStream_t)stream));
}

int trellis_decode_states(const uint32_t* codes, int64_t R, int64_t C, int k, int L, int T,
                          uint16_t* states, int16_t* y, float* value, void* stream) {
  const char* fn = "trellis_decode_states";
  TRY(check_geometry(fn, R, C, k, L, T));
  TRY(check_ptr(fn, "codes", codes, 16));
  if (states) TRY(check_ptr(fn, "states", states, 2));
  if (y) TRY(check_ptr(fn, "y", y, 2));
  if (value) TRY(check_ptr(fn, "value", value, 4));
  return hip_status(fn, trellis::launch_decode_states(codes, R, C, k, states, y, value, (hipStream_t)stream));
}

}  // extern "C"
