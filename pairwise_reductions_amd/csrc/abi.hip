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
#include <utility>
#include <vector>

namespace {

thread_local std::string g_last_error;

// Event pairs recorded around main-sweep launches while timing is enabled on this thread.
struct SweepTiming {
  bool on = false;
  hipEvent_t open = nullptr;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pairs;
  void clear() {
    if (open) (void)hipEventDestroy(open);
    open = nullptr;
    for (auto& pr : pairs) {
      (void)hipEventDestroy(pr.first);
      (void)hipEventDestroy(pr.second);
    }
    pairs.clear();
  }
};
thread_local SweepTiming g_timing;

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
  size_t scr_off;               // argKmin: the float32 screening table
  size_t order_off;             // argKmin: spatial orders and starting thresholds
  size_t part_off, part_bytes;  // per-split partials (argKmin lists for ops 2 and 6)
  size_t lse_off;               // per-split (m, l) pairs of the fused argKmin + LSE (op 6)
  size_t mf_off;                // Gauss sum, LSE, one-channel gradient: the matrix-core operands
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
  L.scr_off = L.aux_off + aux_bytes;
  const size_t scr_bytes = knn ? keops::align_up(keops::knn_screen_bytes(N, D)) : 0;
  L.order_off = L.scr_off + scr_bytes;
  const size_t order_bytes = knn ? keops::align_up(keops::knn_order_bytes(M, N, D, K)) : 0;
  L.part_off = L.order_off + order_bytes;
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
  L.mf_off = L.lse_off + lse_bytes;
  size_t mf = 0;
  if (op == KEOPS_OP_GAUSS_SUM) mf = keops::mf_region_bytes(M, N, D, C);
  if (op == KEOPS_OP_LSE) mf = keops::mf_region_bytes(M, N, D, 0);
  if (op == KEOPS_OP_GAUSS_SUM_GRAD_X && C == 1) mf = keops::mf_region_bytes(M, N, D, 1 + D, true);
  L.total = L.mf_off + mf;
  if (M == 0 || N == 0) L.total = 0;
  return L;
}

// argKmin + LSE: the argKmin layout followed by a log-sum-exp layout whose matrix-core region
// and partials the matrix-core log-sum-exp sweep uses (the float64 column table of that layout
// stays unused: the fused sweep, which runs when the matrix cores decline, reads the
// argKmin one).
size_t argk_lse_bytes(int64_t M, int64_t N, int D, int K) {
  if (M == 0 || N == 0) return 0;
  return lowd_layout(KEOPS_OP_ARGKMIN_LSE, M, N, D, 1, K).total + lowd_layout(KEOPS_OP_LSE, M, N, D, 1, 0).total;
}

}  // namespace

namespace keops {
// Called around the main sweep's launch (begin, then end) on its stream; records an event
// pair while timing is enabled on this thread. Best effort: an event that cannot be created
// or recorded is skipped, and keops_sweep_timing_read then counts fewer pairs.
void sweep_event(hipStream_t s, bool begin) {
  if (!g_timing.on) return;
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return;
  if (hipEventRecord(e, s) != hipSuccess) {
    (void)hipEventDestroy(e);
    return;
  }
  if (begin) {
    if (g_timing.open) (void)hipEventDestroy(g_timing.open);
    g_timing.open = e;
  } else if (g_timing.open) {
    g_timing.pairs.emplace_back(g_timing.open, e);
    g_timing.open = nullptr;
  } else {
    (void)hipEventDestroy(e);
  }
}
}  // namespace keops

namespace {

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

int keops_sweep_timing(int enable) {
  g_timing.clear();
  g_timing.on = enable != 0;
  return ok();
}

int keops_sweep_timing_read(float* ms, int* count) {
  if (!ms || !count) return fail(KEOPS_ERR_INVALID_ARG, "ms and count must not be NULL");
  double total = 0.0;
  int n = 0;
  hipError_t err = hipSuccess;
  for (auto& pr : g_timing.pairs) {
    float t = 0.0f;
    err = hipEventSynchronize(pr.second);
    if (err == hipSuccess) err = hipEventElapsedTime(&t, pr.first, pr.second);
    if (err != hipSuccess) break;
    total += t;
    ++n;
  }
  g_timing.clear();
  if (err != hipSuccess) return hip_fail(err, "sweep timing");
  *ms = (float)total;
  *count = n;
  return ok();
}

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

}  // extern "C"

// ---- scratch of the allocation-free entry point -------------------------------------------
// A fixed device array that stands in for the caller's workspace in keops_gauss_sum_noalloc.
// Every device the library is loaded on holds its own copy until the process ends. Host code
// never uses this name as an address: the per-device address comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[KEOPS_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kScratchDevices = 64;
std::atomic<uintptr_t> g_scratch_addr[kScratchDevices];

// Device address of the current device's scratch array, looked up once per device (with that
// device current) and kept.
int scratch_address(void** addr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kScratchDevices)
    return fail(KEOPS_ERR_UNSUPPORTED, "gauss_sum_noalloc: device %d is beyond the %d it keeps scratch for", dev,
                kScratchDevices);
  uintptr_t a = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (a == 0) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(KEOPS_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    a = reinterpret_cast<uintptr_t>(p);
    g_scratch_addr[dev].store(a, std::memory_order_release);
  }
  *addr = reinterpret_cast<void*>(a);
  return KEOPS_OK;
}

}  // namespace

namespace {

// The two families of Gauss-sum kernels: float32 with D <= 8 runs the low-D VALU kernels
// (B = 1); fp16, bf16, and float32 with larger D run the matrix-core kernels (any B).
bool is_highd(keops_dtype dtype, int32_t D) { return dtype != KEOPS_F32 || D > keops::kMaxLowD; }

keops::ElemType elem_of(keops_dtype dtype) {
  return dtype == KEOPS_F16 ? keops::kElemF16 : (dtype == KEOPS_BF16 ? keops::kElemBF16 : keops::kElemF32);
}

size_t elem_size(keops_dtype dtype) { return dtype == KEOPS_F32 ? 4 : 2; }

// Shape checks shared by the Gauss-sum family.
int check_gauss_family(keops_dtype dtype, int64_t B, int32_t D, int32_t C, const char* what) {
  if (dtype != KEOPS_F32 && dtype != KEOPS_F16 && dtype != KEOPS_BF16)
    return fail(KEOPS_ERR_INVALID_ARG, "%s: unknown dtype %d", what, (int)dtype);
  if (is_highd(dtype, D)) {
    if (!keops::highd_supported(D, C))
      return fail(KEOPS_ERR_UNSUPPORTED, "%s: the matrix-core path needs 1 <= D <= 128 and 1 <= C <= 64 "
                  "(got D=%d C=%d)", what, D, C);
    return KEOPS_OK;
  }
  if (B != 1) return fail(KEOPS_ERR_UNSUPPORTED, "%s: the float32 path for D <= %d needs B = 1 (got %lld)", what,
                          keops::kMaxLowD, (long long)B);
  if (D < 1 || C < 1 || C > keops::kMaxLowC)
    return fail(KEOPS_ERR_UNSUPPORTED, "%s: float32 path needs 1 <= D <= %d and 1 <= C <= %d (got D=%d C=%d)", what,
                keops::kMaxLowD, keops::kMaxLowC, D, C);
  return KEOPS_OK;
}

// Points of a width the matrix-core kernels do not read directly (D not a multiple of 16) are
// first copied, zero-padded to highd_stored_features(D), to the front of the workspace.
size_t highd_pad_bytes(int64_t B, int64_t M, int64_t N, int D, size_t es) {
  const int Ds = keops::highd_stored_features(D);
  if (Ds == D) return 0;
  return keops::align_up((size_t)(B * M) * Ds * es) + keops::align_up((size_t)(B * N) * Ds * es);
}

// Workspace of a matrix-core Gauss sum: the padded points (if any), then the sweep's layout.
size_t highd_sum_bytes(int64_t B, int64_t M, int64_t N, int D, int C, keops_dtype dtype, bool general) {
  if (B == 0 || M == 0 || N == 0) return 0;
  return highd_pad_bytes(B, M, N, D, elem_size(dtype)) +
         keops::highd_workspace_bytes(B, M, N, keops::highd_stored_features(D), C, elem_of(dtype), general);
}

// Copies x and y into the workspace with zero features up to Ds = highd_stored_features(D) when
// D is not already a multiple of 16; on return x, y, D and ws describe what the kernels read.
hipError_t highd_pad_points(const void*& x, const void*& y, int64_t B, int64_t M, int64_t N, int& D, size_t es,
                            char*& ws, hipStream_t stream) {
  const int Ds = keops::highd_stored_features(D);
  if (Ds == D) return hipSuccess;
  void* xp = ws;
  ws += keops::align_up((size_t)(B * M) * Ds * es);
  void* yp = ws;
  ws += keops::align_up((size_t)(B * N) * Ds * es);
  hipError_t e = keops::launch_pad_rows(x, xp, B * M, D, Ds, (int)es, stream);
  if (e == hipSuccess) e = keops::launch_pad_rows(y, yp, B * N, D, Ds, (int)es, stream);
  x = xp;
  y = yp;
  D = Ds;
  return e;
}

// Workspace of the float32 scaled Gauss sum: the column-scaled weights, then the low-D layout.
size_t lowd_scaled_bytes(int64_t M, int64_t N, int D, int C, bool col_scaled) {
  const size_t tail = lowd_layout(KEOPS_OP_GAUSS_SUM, M, N, D, C, 0).total;
  if (M == 0 || N == 0) return 0;
  return (col_scaled ? keops::align_up((size_t)N * C * sizeof(float)) : 0) + tail;
}

// out = rscale . sum_j k_ij cscale_j b_j on either path; arguments already validated except
// for the workspace. b is of type bt (the low-D path takes float32 only). `ranges` lists the
// caller's buffers the workspace must not overlap.
// With use_scratch the device's scratch array replaces workspace (which is then ignored).
int gauss_sum_run(const void* x, const void* y, keops_dtype dtype, const void* b, keops::ElemType bt,
                  const float* rscale, const float* cscale, float* out, int64_t B, int64_t M, int64_t N, int32_t D,
                  int32_t C, float sigma, void* workspace, size_t workspace_bytes, const Range* ranges, int nranges,
                  hipStream_t stream, bool use_scratch = false) {
  if (B == 0 || M == 0) return ok();
  if (N == 0) {
    KEOPS_HIP(keops::launch_fill(out, B * M * C, 0.0f, stream), "fill");
    return ok();
  }
  const bool highd = is_highd(dtype, D);
  const keops::ElemType xy = elem_of(dtype);
  const size_t need = highd ? highd_sum_bytes(B, M, N, D, C, dtype, keops::highd_general(xy, bt, cscale != nullptr))
                            : lowd_scaled_bytes(M, N, D, C, cscale != nullptr);
  if (use_scratch) {
    if (need > KEOPS_NOALLOC_SCRATCH_BYTES)
      return fail(KEOPS_ERR_UNSUPPORTED, "gauss_sum_noalloc: these sizes need %zu bytes of scratch, more than the %zu "
                  "it holds (use keops_gauss_sum with a workspace)", need, (size_t)KEOPS_NOALLOC_SCRATCH_BYTES);
    workspace = nullptr;
    workspace_bytes = 0;
    if (need > 0) {
      KEOPS_TRY(scratch_address(&workspace));
      workspace_bytes = KEOPS_NOALLOC_SCRATCH_BYTES;
    }
  }
  KEOPS_TRY(check_workspace(workspace, workspace_bytes, need));
  for (int r = 0; r < nranges; ++r)
    if (overlaps(Range{workspace, need}, ranges[r]))
      return fail(KEOPS_ERR_INVALID_ARG, "workspace overlaps an input or an output");
  if (highd) {
    char* hws = static_cast<char*>(workspace);
    KEOPS_HIP(highd_pad_points(x, y, B, M, N, D, elem_size(dtype), hws, stream), "pad_features");
    KEOPS_HIP(keops::launch_gauss_sum_highd(x, y, xy, b, bt, rscale, cscale, out, hws, B, M, N, D, C, sigma, stream),
              "gauss_sum_highd");
    return ok();
  }
  char* ws = static_cast<char*>(workspace);
  const float* bw = static_cast<const float*>(b);
  if (cscale) {
    float* bs = reinterpret_cast<float*>(ws);
    KEOPS_HIP(keops::launch_scale_rows(bw, cscale, bs, N, C, stream), "scale_cols");
    bw = bs;
    ws += keops::align_up((size_t)N * C * sizeof(float));
  }
  const LowdLayout L = lowd_layout(KEOPS_OP_GAUSS_SUM, M, N, D, C, 0);
  double* cols = reinterpret_cast<double*>(ws + L.cols_off);
  float* part = reinterpret_cast<float*>(ws + L.part_off);
  const double c2 = c2_of(sigma);
  KEOPS_HIP(keops::launch_gauss_sum_lowd(static_cast<const float*>(x), static_cast<const float*>(y), cols, bw, rscale,
                                         out, part, ws + L.mf_off, M, N, D, C, c2, L.plan, stream),
            "gauss_sum_lowd");
  return ok();
}

int gauss_sum_impl(const void* x, const void* y, const void* b, const float* rscale, const float* cscale, float* out,
                   int64_t B, int64_t M, int64_t N, int32_t D, int32_t C, float sigma, keops_dtype dtype,
                   void* workspace, size_t workspace_bytes, hipStream_t stream, const char* what,
                   bool use_scratch = false) {
  KEOPS_TRY(check_extent(B, "B"));
  KEOPS_TRY(check_extent(M, "M"));
  KEOPS_TRY(check_extent(N, "N"));
  KEOPS_TRY(check_sigma(sigma));
  KEOPS_TRY(check_gauss_family(dtype, B, D, C, what));
  const bool highd = is_highd(dtype, D);
  const size_t es = elem_size(dtype);
  // the matrix-core kernels read rows of a multiple of 16 features as 16-byte vectors; other
  // widths are read element by element into a padded copy
  const size_t al = highd ? (D % 16 == 0 ? 16 : es) : 4;
  const Range rx{x, (size_t)(B * M * D) * es}, ry{y, (size_t)(B * N * D) * es}, rb{b, (size_t)(B * N * C) * es};
  const Range ro{out, (size_t)(B * M * C) * sizeof(float)};
  const Range rr{rscale, rscale ? (size_t)(B * M) * sizeof(float) : 0};
  const Range rc{cscale, cscale ? (size_t)(B * N) * sizeof(float) : 0};
  KEOPS_TRY(check_ptr(x, "x", al, rx.bytes));
  KEOPS_TRY(check_ptr(y, "y", al, ry.bytes));
  KEOPS_TRY(check_ptr(b, "b", highd ? es : 4, rb.bytes));
  KEOPS_TRY(check_ptr(out, "out", highd ? 16 : 4, ro.bytes));
  if (rscale && !aligned(rscale, 4)) return fail(KEOPS_ERR_INVALID_ARG, "row_scale must be 4-byte aligned");
  if (cscale && !aligned(cscale, 4)) return fail(KEOPS_ERR_INVALID_ARG, "col_scale must be 4-byte aligned");
  if (overlaps(ro, rx) || overlaps(ro, ry) || overlaps(ro, rb) || overlaps(ro, rr) || overlaps(ro, rc))
    return fail(KEOPS_ERR_INVALID_ARG, "out overlaps an input");
  const Range all[] = {rx, ry, rb, ro, rr, rc};
  return gauss_sum_run(x, y, dtype, b, elem_of(dtype), rscale, cscale, out, B, M, N, D, C, sigma, workspace,
                       workspace_bytes, all, 6, stream, use_scratch);
}

// Workspace of keops_gauss_sum_backward: the passes run one after another on the stream, so
// they share one region sized for the largest.
size_t backward_bytes(int64_t B, int64_t M, int64_t N, int D, int C, bool half, bool want_x, bool want_y,
                      bool want_b) {
  size_t need = 0;
  auto take = [&](size_t v) { need = v > need ? v : need; };
  if (half) {
    // the y-gradient sweep also yields the b-gradient when C is small enough
    const bool fuse_b = want_y && want_b && C <= keops::hd_fused_weight_channels();
    const int Ds = keops::highd_stored_features(D);
    if (want_x) take(keops::highd_grad_workspace_bytes(B, M, N, Ds, C, false));
    if (want_y) take(keops::highd_grad_workspace_bytes(B, N, M, Ds, C, fuse_b));
    if (want_b && !fuse_b) take(keops::highd_workspace_bytes(B, N, M, Ds, C, keops::kElemF16, true));
    // other widths: the padded points and Ds-wide gradients first, narrowed to D at the end
    if (Ds != D)
      need += highd_pad_bytes(B, M, N, D, 2) + (want_x ? keops::align_up((size_t)(B * M) * Ds * sizeof(float)) : 0) +
              (want_y ? keops::align_up((size_t)(B * N) * Ds * sizeof(float)) : 0);
  } else {
    if (want_x) take(lowd_layout(KEOPS_OP_GAUSS_SUM_GRAD_X, M, N, D, C, 0).total);
    if (want_y) take(lowd_layout(KEOPS_OP_GAUSS_SUM_GRAD_X, N, M, D, C, 0).total);
    if (want_b) take(lowd_layout(KEOPS_OP_GAUSS_SUM, N, M, D, C, 0).total);
  }
  return need;
}

// Workspace of keops_diffusion_scaling: ones, q, p and d (B N floats each), then the region of
// the two Gauss sums.
size_t diffusion_bytes(int64_t B, int64_t N, int D, keops_dtype dtype) {
  if (B == 0 || N == 0) return 0;
  const size_t vec = keops::align_up((size_t)(B * N) * sizeof(float));
  const size_t sums = is_highd(dtype, D) ? highd_sum_bytes(B, N, N, D, 1, dtype, true)
                                         : lowd_layout(KEOPS_OP_GAUSS_SUM, N, N, D, 1, 0).total;
  return 4 * vec + sums;
}

}  // namespace

extern "C" {

size_t keops_workspace_bytes(int op, int64_t B, int64_t M, int64_t N, int32_t D, int32_t C, int32_t K,
                             keops_dtype dtype) {
  if (B < 0 || M < 0 || N < 0 || M > kMaxExtent || N > kMaxExtent) return 0;
  switch (op) {
    case KEOPS_OP_GAUSS_SUM:
    case KEOPS_OP_GAUSS_SUM_SCALED: {
      if (dtype != KEOPS_F32 && dtype != KEOPS_F16 && dtype != KEOPS_BF16) return 0;
      const bool scaled = op == KEOPS_OP_GAUSS_SUM_SCALED;
      if (is_highd(dtype, D)) {
        if (!keops::highd_supported(D, C) || B == 0 || M == 0 || N == 0) return 0;
        const keops::ElemType xy = elem_of(dtype);
        return highd_sum_bytes(B, M, N, D, C, dtype, keops::highd_general(xy, xy, scaled));
      }
      if (B != 1 || D < 1 || C < 1 || C > keops::kMaxLowC) return 0;
      return lowd_scaled_bytes(M, N, D, C, scaled);
    }
    case KEOPS_OP_LSE:
      if (D < 1 || D > keops::kMaxLowD) return 0;
      return lowd_layout(op, M, N, D, 1, 0).total;
    case KEOPS_OP_ARGKMIN_WEIGHTED:
      if (D < 1 || D > keops::kMaxLowD || K < 1 || K > keops::kMaxK || K > N) return 0;
      return lowd_layout(KEOPS_OP_ARGKMIN, M, N, D, 1, K).total;
    case KEOPS_OP_ARGKMIN:
      if (D < 1 || D > keops::kMaxLowD || K < 1 || K > keops::kMaxK || K > N) return 0;
      return lowd_layout(op, M, N, D, 1, K).total;
    case KEOPS_OP_ARGKMIN_LSE:  // the argKmin layout, then a log-sum-exp one for the matrix-core sweep
      if (D < 1 || D > keops::kMaxLowD || K < 1 || K > keops::kMaxK || K > N) return 0;
      return argk_lse_bytes(M, N, D, K);
    case KEOPS_OP_GAUSS_SUM_GRAD_X:
      if (D < 1 || D > keops::kMaxLowD || C < 1 || C > keops::kMaxLowC) return 0;
      return lowd_layout(op, M, N, D, C, 0).total;
    case KEOPS_OP_GAUSS_SUM_GRAD_Y:  // the x-gradient kernel over the transposed pairs
      if (D < 1 || D > keops::kMaxLowD || C < 1 || C > keops::kMaxLowC) return 0;
      return lowd_layout(KEOPS_OP_GAUSS_SUM_GRAD_X, N, M, D, C, 0).total;
    case KEOPS_OP_GAUSS_SUM_GRAD_B:  // the Gauss sum over the transposed pairs
      if (D < 1 || D > keops::kMaxLowD || C < 1 || C > keops::kMaxLowC) return 0;
      return lowd_layout(KEOPS_OP_GAUSS_SUM, N, M, D, C, 0).total;
    case KEOPS_OP_GAUSS_SUM_BACKWARD:
      if (dtype == KEOPS_BF16 || (dtype == KEOPS_F32 && is_highd(dtype, D))) return 0;
      if (dtype == KEOPS_F16) {
        if (!keops::highd_supported(D, C) || B == 0 || M == 0 || N == 0) return 0;
        return backward_bytes(B, M, N, D, C, true, true, true, true);
      }
      if (dtype != KEOPS_F32 || B != 1 || D < 1 || D > keops::kMaxLowD || C < 1 || C > keops::kMaxLowC) return 0;
      if (M == 0 || N == 0) return 0;
      return backward_bytes(B, M, N, D, C, false, true, true, true);
    case KEOPS_OP_DIFFUSION_SCALING:
      if (dtype != KEOPS_F32 && dtype != KEOPS_F16 && dtype != KEOPS_BF16) return 0;
      if (is_highd(dtype, D)) {
        if (!keops::highd_supported(D, 1)) return 0;
      } else if (B != 1 || D < 1) {
        return 0;
      }
      return diffusion_bytes(B, N, D, dtype);
  }
  return 0;
}

int keops_gauss_sum(const void* x, const void* y, const void* b, float* out, int64_t B, int64_t M, int64_t N,
                    int32_t D, int32_t C, float sigma, keops_dtype dtype, void* workspace,
                    size_t workspace_bytes, hipStream_t stream) {
  return gauss_sum_impl(x, y, b, nullptr, nullptr, out, B, M, N, D, C, sigma, dtype, workspace, workspace_bytes,
                        stream, "gauss_sum");
}

int keops_gauss_sum_noalloc(const void* x, const void* y, const void* b, float* out, int64_t B, int64_t M, int64_t N,
                            int32_t D, int32_t C, float sigma, keops_dtype dtype, hipStream_t stream) {
  return gauss_sum_impl(x, y, b, nullptr, nullptr, out, B, M, N, D, C, sigma, dtype, nullptr, 0, stream,
                        "gauss_sum_noalloc", true);
}

int keops_gauss_sum_scaled(const void* x, const void* y, const void* b, const float* row_scale,
                           const float* col_scale, float* out, int64_t B, int64_t M, int64_t N, int32_t D,
                           int32_t C, float sigma, keops_dtype dtype, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  return gauss_sum_impl(x, y, b, row_scale, col_scale, out, B, M, N, D, C, sigma, dtype, workspace,
                        workspace_bytes, stream, "gauss_sum_scaled");
}

int keops_gauss_sum_backward(const void* x, const void* y, const void* b, const float* g, float* grad_x,
                             float* grad_y, float* grad_b, int64_t B, int64_t M, int64_t N, int32_t D, int32_t C,
                             float sigma, keops_dtype dtype, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  KEOPS_TRY(check_extent(B, "B"));
  KEOPS_TRY(check_extent(M, "M"));
  KEOPS_TRY(check_extent(N, "N"));
  KEOPS_TRY(check_sigma(sigma));
  KEOPS_TRY(check_gauss_family(dtype, B, D, C, "gauss_sum_backward"));
  if (dtype == KEOPS_BF16 || (dtype == KEOPS_F32 && is_highd(dtype, D)))
    return fail(KEOPS_ERR_UNSUPPORTED, "gauss_sum_backward: the matrix-core backward takes fp16 inputs "
                "(float32 gradients are built for D <= %d)", keops::kMaxLowD);
  const bool half = (dtype == KEOPS_F16);
  const size_t es = half ? 2 : 4;
  const size_t al = half ? (D % 16 == 0 ? 16 : es) : 4;
  const Range rx{x, (size_t)(B * M * D) * es}, ry{y, (size_t)(B * N * D) * es}, rb{b, (size_t)(B * N * C) * es};
  const Range rg{g, (size_t)(B * M * C) * 4};
  const Range ogx{grad_x, grad_x ? (size_t)(B * M * D) * 4 : 0};
  const Range ogy{grad_y, grad_y ? (size_t)(B * N * D) * 4 : 0};
  const Range ogb{grad_b, grad_b ? (size_t)(B * N * C) * 4 : 0};
  KEOPS_TRY(check_ptr(x, "x", al, rx.bytes));
  KEOPS_TRY(check_ptr(y, "y", al, ry.bytes));
  KEOPS_TRY(check_ptr(b, "b", half ? 16 : 4, rb.bytes));
  KEOPS_TRY(check_ptr(g, "g", 4, rg.bytes));
  const size_t oal = half ? 16 : 4;
  if ((grad_x && !aligned(grad_x, oal)) || (grad_y && !aligned(grad_y, oal)) || (grad_b && !aligned(grad_b, oal)))
    return fail(KEOPS_ERR_INVALID_ARG, "gradients must be %zu-byte aligned", oal);
  const Range ins[] = {rx, ry, rb, rg};
  const Range outs[] = {ogx, ogy, ogb};
  for (const Range& o : outs) {
    for (const Range& in : ins)
      if (overlaps(o, in)) return fail(KEOPS_ERR_INVALID_ARG, "a gradient overlaps an input");
  }
  if (overlaps(ogx, ogy) || overlaps(ogx, ogb) || overlaps(ogy, ogb))
    return fail(KEOPS_ERR_INVALID_ARG, "gradients overlap each other");
  if (B == 0) return ok();
  const bool want_x = grad_x && M > 0, want_y = grad_y && N > 0, want_b = grad_b && N > 0;
  // Empty sums: a gradient over no pairs is zero.
  if (want_x && N == 0) KEOPS_HIP(keops::launch_fill(grad_x, B * M * D, 0.0f, stream), "fill");
  if (want_y && M == 0) KEOPS_HIP(keops::launch_fill(grad_y, B * N * D, 0.0f, stream), "fill");
  if (want_b && M == 0) KEOPS_HIP(keops::launch_fill(grad_b, B * N * C, 0.0f, stream), "fill");
  if (M == 0 || N == 0) return ok();
  const size_t need = backward_bytes(B, M, N, D, C, half, want_x, want_y, want_b);
  KEOPS_TRY(check_workspace(workspace, workspace_bytes, need));
  const Range rw{workspace, need};
  for (const Range& r : {rx, ry, rb, rg, ogx, ogy, ogb})
    if (overlaps(rw, r)) return fail(KEOPS_ERR_INVALID_ARG, "workspace overlaps an input or an output");
  char* ws = static_cast<char*>(workspace);
  if (half) {
    // Widths that are not a multiple of 16 run on zero-padded copies of the points; the x and y
    // gradients then come out Ds wide and are narrowed to D.
    const int D0 = D;
    float* gx = grad_x;
    float* gy = grad_y;
    KEOPS_HIP(highd_pad_points(x, y, B, M, N, D, es, ws, stream), "pad_features");
    if (D != D0) {
      if (want_x) {
        gx = reinterpret_cast<float*>(ws);
        ws += keops::align_up((size_t)(B * M) * D * sizeof(float));
      }
      if (want_y) {
        gy = reinterpret_cast<float*>(ws);
        ws += keops::align_up((size_t)(B * N) * D * sizeof(float));
      }
    }
    // rows x with weights g against columns y with weights b, and the transpose of that.
    if (want_x)
      KEOPS_HIP(keops::launch_gauss_sum_grad_highd(x, y, g, true, b, false, gx, nullptr, ws, B, M, N, D, C, sigma,
                                                   stream),
                "grad_x_highd");
    const bool fuse_b = want_y && want_b && C <= keops::hd_fused_weight_channels();
    if (want_y)
      KEOPS_HIP(keops::launch_gauss_sum_grad_highd(y, x, b, false, g, true, gy, fuse_b ? grad_b : nullptr, ws, B, N,
                                                   M, D, C, sigma, stream),
                "grad_y_highd");
    if (want_b && !fuse_b)
      KEOPS_HIP(keops::launch_gauss_sum_highd(y, x, keops::kElemF16, g, keops::kElemF32, nullptr, nullptr, grad_b, ws,
                                              B, N, M, D, C, sigma, stream),
                "grad_b_highd");
    if (want_x && gx != grad_x) KEOPS_HIP(keops::launch_narrow_rows(gx, grad_x, B * M, D, D0, stream), "narrow");
    if (want_y && gy != grad_y) KEOPS_HIP(keops::launch_narrow_rows(gy, grad_y, B * N, D, D0, stream), "narrow");
    return ok();
  }
  const float* xf = static_cast<const float*>(x);
  const float* yf = static_cast<const float*>(y);
  const float* bf = static_cast<const float*>(b);
  const double s = (double)sigma;
  const float c2f = (float)c2_of(sigma);
  const float inv_sigma2 = (float)(1.0 / (s * s));
  if (want_x) {
    const LowdLayout L = lowd_layout(KEOPS_OP_GAUSS_SUM_GRAD_X, M, N, D, C, 0);
    KEOPS_HIP(keops::launch_grad_x_lowd(xf, yf, bf, g, grad_x, reinterpret_cast<float*>(ws + L.part_off), ws + L.mf_off,
                                        M, N, D, C, c2f, inv_sigma2, L.plan, stream),
              "grad_x_lowd");
  }
  if (want_y) {
    const LowdLayout L = lowd_layout(KEOPS_OP_GAUSS_SUM_GRAD_X, N, M, D, C, 0);
    KEOPS_HIP(keops::launch_grad_x_lowd(yf, xf, g, bf, grad_y, reinterpret_cast<float*>(ws + L.part_off), ws + L.mf_off,
                                        N, M, D, C, c2f, inv_sigma2, L.plan, stream),
              "grad_y_lowd");
  }
  if (want_b) {
    const LowdLayout L = lowd_layout(KEOPS_OP_GAUSS_SUM, N, M, D, C, 0);
    double* cols = reinterpret_cast<double*>(ws + L.cols_off);
    const double c2 = c2_of(sigma);
    KEOPS_HIP(keops::launch_gauss_sum_lowd(yf, xf, cols, g, nullptr, grad_b, reinterpret_cast<float*>(ws + L.part_off),
                                           ws + L.mf_off, N, M, D, C, c2, L.plan, stream),
              "grad_b_lowd");
  }
  return ok();
}

int keops_diffusion_scaling(const void* x, float* s, float* q, float* d, int64_t B, int64_t N, int32_t D,
                            float sigma, float alpha, keops_dtype dtype, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  KEOPS_TRY(check_extent(B, "B"));
  KEOPS_TRY(check_extent(N, "N"));
  KEOPS_TRY(check_sigma(sigma));
  if (!std::isfinite(alpha)) return fail(KEOPS_ERR_INVALID_ARG, "alpha must be finite (got %g)", (double)alpha);
  KEOPS_TRY(check_gauss_family(dtype, B, D, 1, "diffusion_scaling"));
  const bool highd = is_highd(dtype, D);
  const size_t es = elem_size(dtype);
  const size_t n = (size_t)(B * N);
  const Range rx{x, n * D * es}, rs{s, n * 4}, rq{q, q ? n * 4 : 0}, rd{d, d ? n * 4 : 0};
  KEOPS_TRY(check_ptr(x, "x", highd ? (D % 16 == 0 ? 16 : es) : 4, rx.bytes));
  KEOPS_TRY(check_ptr(s, "s", 4, rs.bytes));
  if ((q && !aligned(q, 4)) || (d && !aligned(d, 4))) return fail(KEOPS_ERR_INVALID_ARG, "q and d must be 4-byte aligned");
  if (overlaps(rs, rx) || overlaps(rq, rx) || overlaps(rd, rx) || overlaps(rs, rq) || overlaps(rs, rd) ||
      overlaps(rq, rd))
    return fail(KEOPS_ERR_INVALID_ARG, "s, q and d must not overlap x or each other");
  if (n == 0) return ok();
  const size_t need = diffusion_bytes(B, N, D, dtype);
  KEOPS_TRY(check_workspace(workspace, workspace_bytes, need));
  const Range rw{workspace, need};
  if (overlaps(rw, rx) || overlaps(rw, rs) || overlaps(rw, rq) || overlaps(rw, rd))
    return fail(KEOPS_ERR_INVALID_ARG, "workspace overlaps an input or an output");
  char* ws = static_cast<char*>(workspace);
  const size_t vec = keops::align_up(n * sizeof(float));
  float* ones = reinterpret_cast<float*>(ws);
  float* qb = q ? q : reinterpret_cast<float*>(ws + vec);
  float* pb = reinterpret_cast<float*>(ws + 2 * vec);
  float* db = d ? d : reinterpret_cast<float*>(ws + 3 * vec);
  char* sub = ws + 4 * vec;
  const size_t sub_bytes = need - 4 * vec;
  KEOPS_HIP(keops::launch_fill(ones, (int64_t)n, 1.0f, stream), "fill");
  // q = K 1; p = q^-alpha; d = p (K p); s = p / sqrt(d)
  const Range none[] = {};
  KEOPS_TRY(gauss_sum_run(x, x, dtype, ones, keops::kElemF32, nullptr, nullptr, qb, B, N, N, D, 1, sigma, sub,
                          sub_bytes, none, 0, stream));
  KEOPS_HIP(keops::launch_pow(qb, pb, (int64_t)n, -alpha, stream), "pow");
  KEOPS_TRY(gauss_sum_run(x, x, dtype, pb, keops::kElemF32, pb, nullptr, db, B, N, N, D, 1, sigma, sub, sub_bytes,
                          none, 0, stream));
  KEOPS_HIP(keops::launch_div_sqrt(pb, db, s, (int64_t)n, stream), "div_sqrt");
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
  KEOPS_HIP(keops::launch_lse_lowd(x, y, cols, out, part, ws + L.mf_off, M, N, D, c2, L.plan, stream), "lse_lowd");
  return ok();
}

namespace {

// Shared by keops_argkmin, keops_argkmin_weighted (w != NULL) and keops_argkmin_lse
// (lse != NULL).
int argkmin_impl(const float* x, const float* y, const float* w, int32_t* idx, float* dist, float* lse, int64_t M,
                 int64_t N, int32_t D, int32_t K, float sigma, void* workspace, size_t workspace_bytes,
                 hipStream_t stream) {
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
  const Range rwt{w, w ? (size_t)N * 4 : 0};
  KEOPS_TRY(check_ptr(x, "x", 4, rx.bytes));
  KEOPS_TRY(check_ptr(y, "y", 4, ry.bytes));
  if (w && !aligned(w, 4)) return fail(KEOPS_ERR_INVALID_ARG, "w must be 4-byte aligned");
  KEOPS_TRY(check_ptr(idx, "idx", 4, ri.bytes));
  if (dist && !aligned(dist, 4)) return fail(KEOPS_ERR_INVALID_ARG, "dist must be 4-byte aligned");
  if (with_lse && !aligned(lse, 4)) return fail(KEOPS_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  if (overlaps(ri, rx) || overlaps(ri, ry) || overlaps(rd, rx) || overlaps(rd, ry) || overlaps(ri, rd) ||
      overlaps(rl, rx) || overlaps(rl, ry) || overlaps(rl, ri) || overlaps(rl, rd) || overlaps(ri, rwt) ||
      overlaps(rd, rwt) || overlaps(rl, rwt))
    return fail(KEOPS_ERR_INVALID_ARG, "idx/dist/lse overlap an input or each other");
  if (M == 0) return ok();
  const int op = with_lse ? KEOPS_OP_ARGKMIN_LSE : KEOPS_OP_ARGKMIN;
  const LowdLayout L = lowd_layout(op, M, N, D, 1, K);
  const size_t need = with_lse ? argk_lse_bytes(M, N, D, K) : L.total;
  KEOPS_TRY(check_workspace(workspace, workspace_bytes, need));
  const Range rw{workspace, need};
  if (overlaps(rw, ri) || overlaps(rw, rd) || overlaps(rw, rl) || overlaps(rw, rx) || overlaps(rw, ry) ||
      overlaps(rw, rwt))
    return fail(KEOPS_ERR_INVALID_ARG, "workspace overlaps an input or an output");
  char* ws = static_cast<char*>(workspace);
  double* cols = reinterpret_cast<double*>(ws + L.cols_off);
  double* ymax = reinterpret_cast<double*>(ws + L.aux_off);
  double* lse_part = reinterpret_cast<double*>(ws + L.lse_off);
  const double c2 = with_lse ? c2_of(sigma) : 0.0;
  keops::KnnLse mf_lse{};
  LowdLayout LL;
  if (with_lse && N > 0 && !w) {
    LL = lowd_layout(KEOPS_OP_LSE, M, N, D, 1, 0);
    char* lws = ws + L.total;
    mf_lse.region = lws + LL.mf_off;
    mf_lse.partial = lws + LL.part_off;
    mf_lse.plan = &LL.plan;
  }
  float* scr = reinterpret_cast<float*>(ws + L.scr_off);
  KEOPS_HIP(keops::launch_knn_lowd(x, y, w, cols, scr, ws + L.order_off, ymax, idx, dist, ws + L.part_off, lse, lse_part, M, N, D, K, c2,
                                   with_lse, L.plan, stream, mf_lse.region ? &mf_lse : nullptr),
            "argkmin_lowd");
  return ok();
}

}  // namespace

int keops_argkmin(const float* x, const float* y, int32_t* idx, float* dist, int64_t M, int64_t N, int32_t D,
                  int32_t K, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return argkmin_impl(x, y, nullptr, idx, dist, nullptr, M, N, D, K, 1.0f, workspace, workspace_bytes, stream);
}

int keops_argkmin_weighted(const float* x, const float* y, const float* w, int32_t* idx, float* dist, int64_t M,
                           int64_t N, int32_t D, int32_t K, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  if (!w && N > 0) return fail(KEOPS_ERR_INVALID_ARG, "w must not be NULL");
  return argkmin_impl(x, y, w, idx, dist, nullptr, M, N, D, K, 1.0f, workspace, workspace_bytes, stream);
}

int keops_argkmin_lse(const float* x, const float* y, int32_t* idx, float* dist, float* lse, int64_t M, int64_t N,
                      int32_t D, int32_t K, float sigma, void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  if (!lse && M > 0) return fail(KEOPS_ERR_INVALID_ARG, "lse must not be NULL");
  return argkmin_impl(x, y, nullptr, idx, dist, lse, M, N, D, K, sigma, workspace, workspace_bytes, stream);
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
  char* ws = static_cast<char*>(workspace);
  float* part = reinterpret_cast<float*>(ws + L.part_off);
  KEOPS_HIP(keops::launch_grad_x_lowd(x, y, b, g, grad, part, ws + L.mf_off, M, N, D, C, c2f, inv_sigma2, L.plan,
                                      stream),
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
  char* ws = static_cast<char*>(workspace);
  float* part = reinterpret_cast<float*>(ws + L.part_off);
  KEOPS_HIP(keops::launch_grad_x_lowd(y, x, g, b, grad_y, part, ws + L.mf_off, N, M, D, C, c2f, inv_sigma2, L.plan,
                                      stream),
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
  KEOPS_HIP(keops::launch_gauss_sum_lowd(y, x, cols, g, nullptr, grad_b, part, ws + L.mf_off, N, M, D, C, c2, L.plan,
                                         stream),
            "grad_b_lowd");
  return ok();
}

}  // extern "C"
