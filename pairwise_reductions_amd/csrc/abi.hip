// C-ABI entry points: argument validation, workspace layout, dispatch and error reporting.
// Nothing here allocates device memory; every launch goes to the caller's stream.
#include "../../include/keops_mi355x.h"
#include "internal.h"

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return KEOPS_OK;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(KEOPS_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr int64_t kMaxExtent = 0x7fffffff;  // row and column counts must fit int32 indices

struct Range {
  const void* p;
  size_t bytes;
};

bool overlaps(Range a, Range b) {
  if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, a1 = a0 + a.bytes;
  const uintptr_t b0 = (uintptr_t)b.p, b1 = b0 + b.bytes;
  return a0 < b1 && b0 < a1;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// An empty array may be passed as NULL; a non-empty one must be a valid, aligned pointer.
int check_ptr(const void* p, const char* name, size_t align, size_t bytes) {
  if (bytes == 0) return KEOPS_OK;
  if (!p) return fail(KEOPS_ERR_INVALID_ARG, "%s must not be NULL", name);
  if (!aligned(p, align)) return fail(KEOPS_ERR_INVALID_ARG, "%s must be %zu-byte aligned", name, align);
  return KEOPS_OK;
}

int check_extent(int64_t v, const char* name) {
  if (v < 0) return fail(KEOPS_ERR_INVALID_ARG, "%s must be >= 0 (got %lld)", name, (long long)v);
  if (v > kMaxExtent) return fail(KEOPS_ERR_UNSUPPORTED, "%s = %lld exceeds 2^31-1", name, (long long)v);
  return KEOPS_OK;
}

int check_sigma(float sigma) {
  if (!std::isfinite(sigma) || !(sigma > 0.0f))
    return fail(KEOPS_ERR_INVALID_ARG, "sigma must be finite and > 0 (got %g)", (double)sigma);
  return KEOPS_OK;
}

// base-2 exponent scale: exp(-d2 / (2 sigma^2)) = 2^(-c2 d2)
double c2_of(float sigma) {
  const double s = (double)sigma;
  return 1.4426950408889634 / (2.0 * s * s);
}

// ---- workspace layouts ------------------------------------------------------------------
struct LowdLayout {
  keops::Plan plan;
  size_t cols_off, cols_bytes;  // column table
  size_t aux_off;               // one double: the largest column norm (argKmin screening)
  size_t part_off, part_bytes;  // per-split partials (argKmin lists for ops 2 and 6)
  size_t lse_off;               // per-split (m, l) pairs of the fused argKmin + LSE (op 6)
  size_t total;
};

LowdLayout lowd_layout(int op, int64_t M, int64_t N, int D, int C, int K) {
  LowdLayout L;
  L.plan = keops::plan_lowd(op, M, N, D, C, K, keops::device_cus());
  const bool needs_cols = (op != KEOPS_OP_GAUSS_SUM_GRAD_X);
  const bool knn = (op == KEOPS_OP_ARGKMIN || op == KEOPS_OP_ARGKMIN_LSE);
  const size_t S = (size_t)L.plan.splits, Mz = (size_t)M;
  L.cols_off = 0;
  L.cols_bytes = needs_cols ? keops::align_up((size_t)N * keops::col_stride(D) * sizeof(double)) : 0;
  L.aux_off = L.cols_bytes;
  const size_t aux_bytes = knn ? keops::kAlign : 0;
  L.part_off = L.aux_off + aux_bytes;
  size_t lse_bytes = 0;
  if (S > 1) {
    if (knn) {
      L.part_bytes = keops::align_up(S * Mz * keops::partial_bytes_per_row(KEOPS_OP_ARGKMIN, D, C, K));
      if (op == KEOPS_OP_ARGKMIN_LSE) lse_bytes = keops::align_up(S * Mz * keops::partial_bytes_per_row(KEOPS_OP_LSE, D, C, K));
    } else {
      L.part_bytes = keops::align_up(S * Mz * keops::partial_bytes_per_row(op, D, C, K));
    }
  } else {
    L.part_bytes = 0;
  }
  L.lse_off = L.part_off + L.part_bytes;
  L.total = L.lse_off + lse_bytes;
  if (M == 0 || N == 0) L.total = 0;
  return L;
}

int check_workspace(void* ws, size_t have, size_t need) {
  if (need == 0) return KEOPS_OK;
  if (!ws) return fail(KEOPS_ERR_INVALID_ARG, "workspace is NULL but %zu bytes are needed", need);
  if (!aligned(ws, 16)) return fail(KEOPS_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (have < need)
    return fail(KEOPS_ERR_INVALID_ARG, "workspace too small: %zu bytes given, %zu needed", have, need);
  return KEOPS_OK;
}

#define KEOPS_TRY(expr)          \
  do {                           \
    int st_ = (expr);            \
    if (st_ != KEOPS_OK) return st_; \
  } while (0)

#define KEOPS_HIP(expr, where)                 \
  do {                                         \
    hipError_t e_ = (expr);                    \
    if (e_ != hipSuccess) return hip_fail(e_, where); \
  } while (0)

}  // namespace

namespace keops {

int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace keops

extern "C" {

const char* keops_version(void) { return "keops_mi355x 0.1.0 (gfx950)"; }

const char* keops_status_string(int status) {
  switch (status) {
    case KEOPS_OK: return "ok";
    case KEOPS_ERR_INVALID_ARG: return "invalid argument";
    case KEOPS_ERR_UNSUPPORTED: return "unsupported configuration";
    case KEOPS_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* keops_last_error(void) { return g_last_error.c_str(); }

size_t keops_workspace_bytes(int op, int64_t B, int64_t M, int64_t N, int32_t D, int32_t C, int32_t K,
                             keops_dtype dtype) {
  if (B < 0 || M < 0 || N < 0 || M > kMaxExtent || N > kMaxExtent) return 0;
  switch (op) {
    case KEOPS_OP_GAUSS_SUM:
      if (dtype == KEOPS_F16) {
        if (!keops::highd_supported(D, C)) return 0;
        return keops::highd_workspace_bytes(B, M, N, D, C);
      }
      if (dtype != KEOPS_F32 || B != 1 || D < 1 || D > keops::kMaxLowD || C < 1 || C > keops::kMaxLowC) return 0;
      return lowd_layout(op, M, N, D, C, 0).total;
    case KEOPS_OP_LSE:
      if (D < 1 || D > keops::kMaxLowD) return 0;
      return lowd_layout(op, M, N, D, 1, 0).total;
    case KEOPS_OP_ARGKMIN:
    case KEOPS_OP_ARGKMIN_LSE:
      if (D < 1 || D > keops::kMaxLowD || K < 1 || K > keops::kMaxK || K > N) return 0;
      return lowd_layout(op, M, N, D, 1, K).total;
    case KEOPS_OP_GAUSS_SUM_GRAD_X:
      if (D < 1 || D > keops::kMaxLowD || C < 1 || C > keops::kMaxLowC) return 0;
      return lowd_layout(op, M, N, D, C, 0).total;
    case KEOPS_OP_GAUSS_SUM_GRAD_Y:  // the x-gradient kernel over the transposed pairs
      if (D < 1 || D > keops::kMaxLowD || C < 1 || C > keops::kMaxLowC) return 0;
      return lowd_layout(KEOPS_OP_GAUSS_SUM_GRAD_X, N, M, D, C, 0).total;
    case KEOPS_OP_GAUSS_SUM_GRAD_B:  // the Gauss sum over the transposed pairs
      if (D < 1 || D > keops::kMaxLowD || C < 1 || C > keops::kMaxLowC) return 0;
      return lowd_layout(KEOPS_OP_GAUSS_SUM, N, M, D, C, 0).total;
  }
  return 0;
}

int keops_gauss_sum(const void* x, const void* y, const void* b, float* out, int64_t B, int64_t M, int64_t N,
                    int32_t D, int32_t C, float sigma, keops_dtype dtype, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  KEOPS_TRY(check_extent(B, "B"));
  KEOPS_TRY(check_extent(M, "M"));
  KEOPS_TRY(check_extent(N, "N"));
  KEOPS_TRY(check_sigma(sigma));
  const bool half = (dtype == KEOPS_F16 || dtype == KEOPS_BF16);
  if (!half && dtype != KEOPS_F32) return fail(KEOPS_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (dtype == KEOPS_BF16) return fail(KEOPS_ERR_UNSUPPORTED, "the bf16 matrix-core path is not built (use KEOPS_F16)");
  if (half) {
    if (!keops::highd_supported(D, C))
      return fail(KEOPS_ERR_UNSUPPORTED, "fp16 path needs D in {32, 64} and 1 <= C <= 64 (got D=%d C=%d)", D, C);
  } else {
    if (B != 1) return fail(KEOPS_ERR_UNSUPPORTED, "float32 path needs B = 1 (got %lld)", (long long)B);
    if (D < 1 || D > keops::kMaxLowD || C < 1 || C > keops::kMaxLowC)
      return fail(KEOPS_ERR_UNSUPPORTED, "float32 path needs 1 <= D <= %d and 1 <= C <= %d (got D=%d C=%d)",
                  keops::kMaxLowD, keops::kMaxLowC, D, C);
  }
  const size_t es = half ? 2 : 4;
  const size_t al = half ? 16 : 4;
  const Range rx{x, (size_t)(B * M * D) * es}, ry{y, (size_t)(B * N * D) * es}, rb{b, (size_t)(B * N * C) * es};
  const Range ro{out, (size_t)(B * M * C) * sizeof(float)};
  KEOPS_TRY(check_ptr(x, "x", al, rx.bytes));
  KEOPS_TRY(check_ptr(y, "y", al, ry.bytes));
  KEOPS_TRY(check_ptr(b, "b", al, rb.bytes));
  KEOPS_TRY(check_ptr(out, "out", half ? 16 : 4, ro.bytes));
  if (overlaps(ro, rx) || overlaps(ro, ry) || overlaps(ro, rb))
    return fail(KEOPS_ERR_INVALID_ARG, "out overlaps an input");
  if (B == 0 || M == 0) return ok();
  if (half) {
    const size_t need = keops::highd_workspace_bytes(B, M, N, D, C);
    KEOPS_TRY(check_workspace(workspace, workspace_bytes, need));
    if (overlaps(Range{workspace, need}, ro)) return fail(KEOPS_ERR_INVALID_ARG, "workspace overlaps out");
    if (N == 0) {
      KEOPS_HIP(keops::launch_fill(out, B * M * C, 0.0f, stream), "fill");
      return ok();
    }
    KEOPS_HIP(keops::launch_gauss_sum_highd(x, y, b, out, workspace, B, M, N, D, C, sigma, dtype == KEOPS_BF16,
                                            stream),
              "gauss_sum_highd");
    return ok();
  }
  if (N == 0) {
    KEOPS_HIP(keops::launch_fill(out, M * C, 0.0f, stream), "fill");
    return ok();
  }
  const LowdLayout L = lowd_layout(KEOPS_OP_GAUSS_SUM, M, N, D, C, 0);
  KEOPS_TRY(check_workspace(workspace, workspace_bytes, L.total));
  if (overlaps(Range{workspace, L.total}, ro) || overlaps(Range{workspace, L.total}, rx) ||
      overlaps(Range{workspace, L.total}, ry) || overlaps(Range{workspace, L.total}, rb))
    return fail(KEOPS_ERR_INVALID_ARG, "workspace overlaps an input or the output");
  char* ws = static_cast<char*>(workspace);
  double* cols = reinterpret_cast<double*>(ws + L.cols_off);
  float* part = reinterpret_cast<float*>(ws + L.part_off);
  const double c2 = c2_of(sigma);
  KEOPS_HIP(keops::launch_prep_cols(static_cast<const float*>(y), cols, N, D, c2, true, stream), "prep_cols");
  KEOPS_HIP(keops::launch_gauss_sum_lowd(static_cast<const float*>(x), static_cast<const float*>(y), cols,
                                         static_cast<const float*>(b), out, part, M, N, D, C, c2, L.plan, stream),
            "gauss_sum_lowd");
  return ok();
}

int keops_lse(const float* x, const float* y, float* out, int64_t M, int64_t N, int32_t D, float sigma,
              void* workspace, size_t workspace_bytes, hipStream_t stream) {
  KEOPS_TRY(check_extent(M, "M"));
  KEOPS_TRY(check_extent(N, "N"));
  KEOPS_TRY(check_sigma(sigma));
  if (D < 1 || D > keops::kMaxLowD)
    return fail(KEOPS_ERR_UNSUPPORTED, "lse needs 1 <= D <= %d (got %d)", keops::kMaxLowD, D);
  const Range rx{x, (size_t)(M * D) * 4}, ry{y, (size_t)(N * D) * 4}, ro{out, (size_t)M * 4};
  KEOPS_TRY(check_ptr(x, "x", 4, rx.bytes));
  KEOPS_TRY(check_ptr(y, "y", 4, ry.bytes));
  KEOPS_TRY(check_ptr(out, "out", 4, ro.bytes));
  if (overlaps(ro, rx) || overlaps(ro, ry)) return fail(KEOPS_ERR_INVALID_ARG, "out overlaps an input");
  if (M == 0) return ok();
  if (N == 0) {
    KEOPS_HIP(keops::launch_fill(out, M, -INFINITY, stream), "fill");
    return ok();
  }
  const LowdLayout L = lowd_layout(KEOPS_OP_LSE, M, N, D, 1, 0);
  KEOPS_TRY(check_workspace(workspace, workspace_bytes, L.total));
  const Range rw{workspace, L.total};
  if (overlaps(rw, ro) || overlaps(rw, rx) || overlaps(rw, ry))
    return fail(KEOPS_ERR_INVALID_ARG, "workspace overlaps an input or the output");
  char* ws = static_cast<char*>(workspace);
  double* cols = reinterpret_cast<double*>(ws + L.cols_off);
  double* part = reinterpret_cast<double*>(ws + L.part_off);
  const double c2 = c2_of(sigma);
  KEOPS_HIP(keops::launch_prep_cols(y, cols, N, D, c2, true, stream), "prep_cols");
  KEOPS_HIP(keops::launch_lse_lowd(x, y, cols, out, part, M, N, D, c2, L.plan, stream), "lse_lowd");
  return ok();
}

namespace {

// Shared by keops_argkmin and keops_argkmin_lse (lse == NULL for the former).
int argkmin_impl(const float* x, const float* y, int32_t* idx, float* dist, float* lse, int64_t M, int64_t N,
                 int32_t D, int32_t K, float sigma, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const bool with_lse = (lse != nullptr);
  KEOPS_TRY(check_extent(M, "M"));
  KEOPS_TRY(check_extent(N, "N"));
  if (with_lse) KEOPS_TRY(check_sigma(sigma));
  if (D < 1 || D > keops::kMaxLowD)
    return fail(KEOPS_ERR_UNSUPPORTED, "argkmin needs 1 <= D <= %d (got %d)", keops::kMaxLowD, D);
  if (K < 1 || K > N) return fail(KEOPS_ERR_INVALID_ARG, "argkmin needs 1 <= K <= N (got K=%d N=%lld)", K, (long long)N);
  if (K > keops::kMaxK) return fail(KEOPS_ERR_UNSUPPORTED, "argkmin supports K <= %d (got %d)", keops::kMaxK, K);
  const Range rx{x, (size_t)(M * D) * 4}, ry{y, (size_t)(N * D) * 4};
  const Range ri{idx, (size_t)(M * K) * 4}, rd{dist, dist ? (size_t)(M * K) * 4 : 0};
  const Range rl{lse, with_lse ? (size_t)M * 4 : 0};
  KEOPS_TRY(check_ptr(x, "x", 4, rx.bytes));
  KEOPS_TRY(check_ptr(y, "y", 4, ry.bytes));
  KEOPS_TRY(check_ptr(idx, "idx", 4, ri.bytes));
  if (dist && !aligned(dist, 4)) return fail(KEOPS_ERR_INVALID_ARG, "dist must be 4-byte aligned");
  if (with_lse && !aligned(lse, 4)) return fail(KEOPS_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (overlaps(ri, rx) || overlaps(ri, ry) || overlaps(rd, rx) || overlaps(rd, ry) || overlaps(ri, rd) ||
      overlaps(rl, rx) || overlaps(rl, ry) || overlaps(rl, ri) || overlaps(rl, rd))
    return fail(KEOPS_ERR_INVALID_ARG, "idx/dist/lse overlap an input or each other");
  if (M == 0) return ok();
  const int op = with_lse ? KEOPS_OP_ARGKMIN_LSE : KEOPS_OP_ARGKMIN;
  const LowdLayout L = lowd_layout(op, M, N, D, 1, K);
  KEOPS_TRY(check_workspace(workspace, workspace_bytes, L.total));
  const Range rw{workspace, L.total};
  if (overlaps(rw, ri) || overlaps(rw, rd) || overlaps(rw, rl) || overlaps(rw, rx) || overlaps(rw, ry))
    return fail(KEOPS_ERR_INVALID_ARG, "workspace overlaps an input or an output");
  char* ws = static_cast<char*>(workspace);
  double* cols = reinterpret_cast<double*>(ws + L.cols_off);
  double* ymax = reinterpret_cast<double*>(ws + L.aux_off);
  double* lse_part = reinterpret_cast<double*>(ws + L.lse_off);
  const double c2 = with_lse ? c2_of(sigma) : 0.0;
  KEOPS_HIP(keops::launch_knn_lowd(x, y, cols, ymax, idx, dist, ws + L.part_off, lse, lse_part, M, N, D, K, c2,
                                   with_lse, L.plan, stream),
            "argkmin_lowd");
  return ok();
}

}  // namespace

int keops_argkmin(const float* x, const float* y, int32_t* idx, float* dist, int64_t M, int64_t N, int32_t D,
                  int32_t K, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return argkmin_impl(x, y, idx, dist, nullptr, M, N, D, K, 1.0f, workspace, workspace_bytes, stream);
}

int keops_argkmin_lse(const float* x, const float* y, int32_t* idx, float* dist, float* lse, int64_t M, int64_t N,
                      int32_t D, int32_t K, float sigma, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  if (!lse && M > 0) return fail(KEOPS_ERR_INVALID_ARG, "lse must not be NULL");
  return argkmin_impl(x, y, idx, dist, lse, M, N, D, K, sigma, workspace, workspace_bytes, stream);
}

int keops_gauss_sum_grad_x(const float* x, const float* y, const float* b, const float* g, float* grad,
                           int64_t M, int64_t N, int32_t D, int32_t C, float sigma, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  KEOPS_TRY(check_extent(M, "M"));
  KEOPS_TRY(check_extent(N, "N"));
  KEOPS_TRY(check_sigma(sigma));
  if (D < 1 || D > keops::kMaxLowD || C < 1 || C > keops::kMaxLowC)
    return fail(KEOPS_ERR_UNSUPPORTED, "grad_x needs 1 <= D <= %d and 1 <= C <= %d (got D=%d C=%d)",
                keops::kMaxLowD, keops::kMaxLowC, D, C);
  const Range rx{x, (size_t)(M * D) * 4}, ry{y, (size_t)(N * D) * 4}, rb{b, (size_t)(N * C) * 4};
  const Range rg{g, (size_t)(M * C) * 4}, ro{grad, (size_t)(M * D) * 4};
  KEOPS_TRY(check_ptr(x, "x", 4, rx.bytes));
  KEOPS_TRY(check_ptr(y, "y", 4, ry.bytes));
  KEOPS_TRY(check_ptr(b, "b", 4, rb.bytes));
  KEOPS_TRY(check_ptr(g, "g", 4, rg.bytes));
  KEOPS_TRY(check_ptr(grad, "grad", 4, ro.bytes));
  if (overlaps(ro, rx) || overlaps(ro, ry) || overlaps(ro, rb) || overlaps(ro, rg))
    return fail(KEOPS_ERR_INVALID_ARG, "grad overlaps an input");
  if (M == 0) return ok();
  if (N == 0) {
    KEOPS_HIP(keops::launch_fill(grad, M * D, 0.0f, stream), "fill");
    return ok();
  }
  const LowdLayout L = lowd_layout(KEOPS_OP_GAUSS_SUM_GRAD_X, M, N, D, C, 0);
  KEOPS_TRY(check_workspace(workspace, workspace_bytes, L.total));
  const Range rw{workspace, L.total};
  if (overlaps(rw, ro) || overlaps(rw, rx) || overlaps(rw, ry) || overlaps(rw, rb) || overlaps(rw, rg))
    return fail(KEOPS_ERR_INVALID_ARG, "workspace overlaps an input or the output");
  const double s = (double)sigma;
  const float c2f = (float)c2_of(sigma);
  const float inv_sigma2 = (float)(1.0 / (s * s));
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.part_off);
  KEOPS_HIP(keops::launch_grad_x_lowd(x, y, b, g, grad, part, M, N, D, C, c2f, inv_sigma2, L.plan, stream),
            "grad_x_lowd");
  return ok();
}

// d/dy: the x-gradient reduction with the roles of (x, g) and (y, b) exchanged, since
// -(1/s^2) sum_i k_ij (b_j . g_i)(y_j - x_i) = (1/s^2) sum_i k_ij (g_i . b_j)(x_i - y_j).
int keops_gauss_sum_grad_y(const float* x, const float* y, const float* b, const float* g, float* grad_y,
                           int64_t M, int64_t N, int32_t D, int32_t C, float sigma, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  KEOPS_TRY(check_extent(M, "M"));
  KEOPS_TRY(check_extent(N, "N"));
  KEOPS_TRY(check_sigma(sigma));
  if (D < 1 || D > keops::kMaxLowD || C < 1 || C > keops::kMaxLowC)
    return fail(KEOPS_ERR_UNSUPPORTED, "grad_y needs 1 <= D <= %d and 1 <= C <= %d (got D=%d C=%d)",
                keops::kMaxLowD, keops::kMaxLowC, D, C);
  const Range rx{x, (size_t)(M * D) * 4}, ry{y, (size_t)(N * D) * 4}, rb{b, (size_t)(N * C) * 4};
  const Range rg{g, (size_t)(M * C) * 4}, ro{grad_y, (size_t)(N * D) * 4};
  KEOPS_TRY(check_ptr(x, "x", 4, rx.bytes));
  KEOPS_TRY(check_ptr(y, "y", 4, ry.bytes));
  KEOPS_TRY(check_ptr(b, "b", 4, rb.bytes));
  KEOPS_TRY(check_ptr(g, "g", 4, rg.bytes));
  KEOPS_TRY(check_ptr(grad_y, "grad_y", 4, ro.bytes));
  if (overlaps(ro, rx) || overlaps(ro, ry) || overlaps(ro, rb) || overlaps(ro, rg))
    return fail(KEOPS_ERR_INVALID_ARG, "grad_y overlaps an input");
  if (N == 0) return ok();
  if (M == 0) {
    KEOPS_HIP(keops::launch_fill(grad_y, N * D, 0.0f, stream), "fill");
    return ok();
  }
  const LowdLayout L = lowd_layout(KEOPS_OP_GAUSS_SUM_GRAD_X, N, M, D, C, 0);
  KEOPS_TRY(check_workspace(workspace, workspace_bytes, L.total));
  const Range rw{workspace, L.total};
  if (overlaps(rw, ro) || overlaps(rw, rx) || overlaps(rw, ry) || overlaps(rw, rb) || overlaps(rw, rg))
    return fail(KEOPS_ERR_INVALID_ARG, "workspace overlaps an input or the output");
  const double s = (double)sigma;
  const float c2f = (float)c2_of(sigma);
  const float inv_sigma2 = (float)(1.0 / (s * s));
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + L.part_off);
  KEOPS_HIP(keops::launch_grad_x_lowd(y, x, g, b, grad_y, part, N, M, D, C, c2f, inv_sigma2, L.plan, stream),
            "grad_y_lowd");
  return ok();
}

// d/db: s is linear in b, so grad_b[j] = sum_i k_ij g_i, the Gauss sum over transposed pairs.
int keops_gauss_sum_grad_b(const float* x, const float* y, const float* g, float* grad_b, int64_t M, int64_t N,
                           int32_t D, int32_t C, float sigma, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  KEOPS_TRY(check_extent(M, "M"));
  KEOPS_TRY(check_extent(N, "N"));
  KEOPS_TRY(check_sigma(sigma));
  if (D < 1 || D > keops::kMaxLowD || C < 1 || C > keops::kMaxLowC)
    return fail(KEOPS_ERR_UNSUPPORTED, "grad_b needs 1 <= D <= %d and 1 <= C <= %d (got D=%d C=%d)",
                keops::kMaxLowD, keops::kMaxLowC, D, C);
  const Range rx{x, (size_t)(M * D) * 4}, ry{y, (size_t)(N * D) * 4}, rg{g, (size_t)(M * C) * 4};
  const Range ro{grad_b, (size_t)(N * C) * 4};
  KEOPS_TRY(check_ptr(x, "x", 4, rx.bytes));
  KEOPS_TRY(check_ptr(y, "y", 4, ry.bytes));
  KEOPS_TRY(check_ptr(g, "g", 4, rg.bytes));
  KEOPS_TRY(check_ptr(grad_b, "grad_b", 4, ro.bytes));
  if (overlaps(ro, rx) || overlaps(ro, ry) || overlaps(ro, rg)) return fail(KEOPS_ERR_INVALID_ARG, "grad_b overlaps an input");
  if (N == 0) return ok();
  if (M == 0) {
    KEOPS_HIP(keops::launch_fill(grad_b, N * C, 0.0f, stream), "fill");
    return ok();
  }
  const LowdLayout L = lowd_layout(KEOPS_OP_GAUSS_SUM, N, M, D, C, 0);
  KEOPS_TRY(check_workspace(workspace, workspace_bytes, L.total));
  const Range rw{workspace, L.total};
  if (overlaps(rw, ro) || overlaps(rw, rx) || overlaps(rw, ry) || overlaps(rw, rg))
    return fail(KEOPS_ERR_INVALID_ARG, "workspace overlaps an input or the output");
  char* ws = static_cast<char*>(workspace);
  double* cols = reinterpret_cast<double*>(ws + L.cols_off);
  float* part = reinterpret_cast<float*>(ws + L.part_off);
  const double c2 = c2_of(sigma);
  KEOPS_HIP(keops::launch_prep_cols(x, cols, M, D, c2, true, stream), "prep_cols");
  KEOPS_HIP(keops::launch_gauss_sum_lowd(y, x, cols, g, grad_b, part, N, M, D, C, c2, L.plan, stream),
            "grad_b_lowd");
  return ok();
}

}  // extern "C"
