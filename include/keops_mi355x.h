/*
 * keops_mi355x.h — C ABI of the MI355X (gfx950) fused pairwise-reduction library.
 *
 * Every entry point evaluates a reduction a_i = Reduction_j F(x_i, y_j, b_j) over all
 * pairs (i, j) without ever storing the M-by-N table ("Kernel matrix reduction" concept
 * page, Overview, and eq. 2 of its Implementation sketch). All work is enqueued on the
 * caller's HIP stream; the call returns as soon as the kernels are queued.
 *
 * Conventions shared by all entry points
 *   - Data pointers are DEVICE pointers to dense, row-major, contiguous arrays, aligned to
 *     their element size (4 bytes for float32 / int32), and to 16 bytes where a call says so
 *     (the matrix-core path's points when D is a multiple of 16, its outputs, and the
 *     workspace). The caller owns every buffer (inputs, outputs, workspace). The library
 *     never allocates or frees device memory. It keeps no state between calls that affects
 *     a result; the only state it holds is a per-device cache of the compute-unit count (used
 *     to plan launches) and, while keops_sweep_timing is enabled, per-thread HIP events.
 *   - `workspace` must hold keops_workspace_bytes(...) bytes for the same arguments, queried
 *     with the same device current; it may be NULL only when that size is 0. Its contents
 *     on entry are ignored. Two calls in flight at once need two workspaces.
 *   - Arguments are validated before anything is enqueued; on any error nothing is written
 *     and the return value says why (keops_last_error() gives the detail, per thread).
 *     Errors: KEOPS_ERR_INVALID_ARG for NULL / misaligned pointers, negative sizes,
 *     non-finite or non-positive sigma, K outside [1, N], an output overlapping an input or a
 *     workspace that is too small; KEOPS_ERR_UNSUPPORTED for dimensions outside the compiled
 *     families (listed per call); KEOPS_ERR_HIP when a HIP call or launch fails.
 *   - Kernel-execution faults surface at the caller's next synchronisation, as for any HIP
 *     launch. No C++ exception crosses this boundary.
 *   - M = 0 is a no-op. Results are deterministic: the same inputs on the same device give
 *     bit-identical outputs (every sum runs in a fixed order; floating-point atomics only
 *     take maxima, whose result does not depend on the order; integer atomics count and place
 *     points when argKmin orders them in space, which decides only which columns are
 *     screened out, never the result).
 *   - sigma is the Gaussian bandwidth: k(x, y) = exp(-||x - y||^2 / (2 sigma^2)). The
 *     flash-attention page's Phi_tau = exp(-tau/2 ||q - k||^2) is sigma = 1/sqrt(tau).
 */
#ifndef KEOPS_MI355X_H
#define KEOPS_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#if defined(__GNUC__) || defined(__clang__)
#define KEOPS_API __attribute__((visibility("default")))
#else
#define KEOPS_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KEOPS_F32 = 0, KEOPS_F16 = 1, KEOPS_BF16 = 2 } keops_dtype;

typedef enum {
  KEOPS_OK = 0,
  KEOPS_ERR_INVALID_ARG = 1,
  KEOPS_ERR_UNSUPPORTED = 2,
  KEOPS_ERR_HIP = 3
} keops_status;

typedef enum {
  KEOPS_OP_GAUSS_SUM = 0,
  KEOPS_OP_LSE = 1,
  KEOPS_OP_ARGKMIN = 2,
  KEOPS_OP_GAUSS_SUM_GRAD_X = 3,
  KEOPS_OP_GAUSS_SUM_GRAD_Y = 4,
  KEOPS_OP_GAUSS_SUM_GRAD_B = 5,
  KEOPS_OP_ARGKMIN_LSE = 6,
  KEOPS_OP_GAUSS_SUM_SCALED = 7,
  KEOPS_OP_GAUSS_SUM_BACKWARD = 8,
  KEOPS_OP_DIFFUSION_SCALING = 9,
  KEOPS_OP_ARGKMIN_WEIGHTED = 10
} keops_op;

/*
 * Gaussian kernel sum ("Kernel matrix reduction", Implementation sketch, eq. 1; batched
 * with signed weights as in "Fast Gauss Sums via Flash Attention", Algorithm 1 Output row):
 *   out[t][i][c] = sum_j exp(-||x[t][i] - y[t][j]||^2 / (2 sigma^2)) * b[t][j][c]
 * Shapes: x (B, M, D), y (B, N, D), b (B, N, C), out (B, M, C) float32.
 * Two kernel families, chosen by dtype and D:
 *   - KEOPS_F32 with 1 <= D <= 8: the low-D float32 path. x, y, b float32; requires B = 1 and
 *     1 <= C <= 8. 4-byte alignment.
 *   - KEOPS_F16, KEOPS_BF16 (any 1 <= D <= 128), and KEOPS_F32 with 9 <= D <= 128: the
 *     matrix-core path, any B >= 1, 1 <= C <= 64. x, y, b are of the dtype; fp32
 *     accumulation. fp16 and bf16 inputs: the kernel values are rounded to fp16 before they
 *     multiply b. With fp16 inputs a block of rows may also take tau log2(e) into its rounded
 *     fp16 query operands, but only where the resulting change of every kernel value is proven
 *     below 9.6e-4 relative (from the rows' and the keys' norms); otherwise the scale is applied
 *     in float32. float32 inputs are split into fp16 high and low parts (three products per
 *     step, float32 accuracy). Features run in steps of 32 and channels in tiles of 16 (both
 *     read as zero past D and C). When D is a multiple of 16, x and y must be 16-byte aligned
 *     and are read in place; any other D is first copied, zero-padded to the next multiple of
 *     16, into the workspace (x and y then need only their element alignment). out must be
 *     16-byte aligned on this path.
 * N = 0 writes zeros.
 */
KEOPS_API int keops_gauss_sum(const void* x, const void* y, const void* b, float* out,
                    int64_t B, int64_t M, int64_t N, int32_t D, int32_t C, float sigma,
                    keops_dtype dtype, void* workspace, size_t workspace_bytes,
                    hipStream_t stream);

/*
 * Allocation-free Gauss sum, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same reduction,
 * arguments, limits and results as keops_gauss_sum (bit-identical outputs: the same kernels
 * and launch plan), without the workspace arguments. A scratch array inside the library,
 * KEOPS_NOALLOC_SCRATCH_BYTES (64 MiB) of static device memory that every device the library
 * is loaded on holds until the process ends, takes the workspace's place. Sizes whose
 * workspace (keops_workspace_bytes for KEOPS_OP_GAUSS_SUM) exceeds it return
 * KEOPS_ERR_UNSUPPORTED; at D = 3, C = 1 that is above about M = N = 250,000. Nothing is
 * allocated or freed (no hipMalloc, hipFree or allocating library call); the first call on a
 * device looks the array's address up once. All calls on one device share that device's
 * array, and its contents from the last call are never read: calls that overlap in time on
 * one device (two streams or two threads) race and must be serialised by the caller.
 */
#define KEOPS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
KEOPS_API int keops_gauss_sum_noalloc(const void* x, const void* y, const void* b, float* out, int64_t B, int64_t M,
                                      int64_t N, int32_t D, int32_t C, float sigma, keops_dtype dtype,
                                      hipStream_t stream);

/*
 * Log-sum-exp reduction ("Kernel matrix reduction", Overview, list of reductions):
 *   out[i] = log sum_j exp(-||x_i - y_j||^2 / (2 sigma^2))
 * Shapes: x (M, D), y (N, D) float32, out (M,) float32. Requires 1 <= D <= 8.
 * Rows far from every column stay finite: their terms are taken relative to the row's
 * largest one (a running maximum, or a float64 recomputation of rows whose plain sum came
 * out below 2^-64).
 * N = 0 writes -inf.
 */
KEOPS_API int keops_lse(const float* x, const float* y, float* out, int64_t M, int64_t N, int32_t D,
              float sigma, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * argKmin ("Kernel matrix reduction", Overview: indices of the K smallest entries per row):
 *   idx[i][0..K-1] = the columns j with the K smallest keys d2_ij, ascending; equal keys
 *   keep the lower j first.
 * The key is the float64 evaluation of the squared distance with the differences taken
 * first and the squares summed in increasing d, each operation rounded (no fused
 * multiply-add): ((dx0*dx0 + dx1*dx1) + dx2*dx2) + ...; for float32 inputs on a dyadic grid
 * fine enough (e.g. multiples of 2^-24 in [0,1)^3) this is the exact squared distance.
 * Shapes: x (M, D), y (N, D) float32; idx (M, K) int32; dist (M, K) float32 or NULL
 * (the keys rounded to float32). Requires 1 <= D <= 8 and 1 <= K <= min(N, 64)
 * (K > 64 is KEOPS_ERR_UNSUPPORTED; K > N is KEOPS_ERR_INVALID_ARG). K = 1 is argmin/min.
 */
KEOPS_API int keops_argkmin(const float* x, const float* y, int32_t* idx, float* dist, int64_t M,
                  int64_t N, int32_t D, int32_t K, void* workspace, size_t workspace_bytes,
                  hipStream_t stream);

/*
 * Weighted argKmin, the min / max reduction of an additively weighted squared distance
 * ("Kernel matrix reduction", Overview: minima and indices of the K smallest entries of a
 * pairwise formula):
 *   idx[i][0..K-1] = the columns j with the K smallest keys d2_ij - w_j, ascending; equal
 *   keys keep the lower j first;  dist[i][k] = that key rounded to float32.
 * d2_ij is the float64 key of keops_argkmin and w_j is widened exactly to float64; the key
 * is their float64 difference (one rounding). K = 1 is the weighted min and argmin, i.e. the
 * max of w_j - d2_ij; with w_j = 2 sigma^2 ln b_j (b_j > 0) it is the max over j of the
 * weighted kernel b_j exp(-d2_ij / (2 sigma^2)) and its argmax.
 * Shapes: x (M, D), y (N, D), w (N,) float32; idx (M, K) int32; dist (M, K) float32 or NULL.
 * Limits as keops_argkmin; the workspace is that of KEOPS_OP_ARGKMIN_WEIGHTED.
 */
KEOPS_API int keops_argkmin_weighted(const float* x, const float* y, const float* w, int32_t* idx, float* dist,
                                     int64_t M, int64_t N, int32_t D, int32_t K, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/*
 * argKmin and the log-sum-exp reduction of the same pairs ("Kernel matrix reduction",
 * Overview: minima, indices of the K smallest entries and log-sum-exp are all reductions of
 * one pairwise formula):
 *   idx, dist as keops_argkmin;  lse[i] = log sum_j exp(-||x_i - y_j||^2 / (2 sigma^2))
 * Shapes: x (M, D), y (N, D) float32; idx (M, K) int32; dist (M, K) float32 or NULL;
 * lse (M,) float32 (must not be NULL). Same limits as keops_argkmin, plus sigma as in
 * keops_lse; the workspace is that of KEOPS_OP_ARGKMIN_LSE. Where the matrix-core
 * log-sum-exp admits the inputs (decided on the device) it runs beside a plain argKmin sweep;
 * otherwise one fused float64 sweep computes both. idx and dist are the same either way.
 */
KEOPS_API int keops_argkmin_lse(const float* x, const float* y, int32_t* idx, float* dist, float* lse,
                                int64_t M, int64_t N, int32_t D, int32_t K, float sigma,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Gradient of the Gauss sum with respect to x ("Kernel matrix reduction", Variants:
 * autodiff through the reduction; the KeOps page's example differentiates sum_i a_i^2),
 * as a vector-Jacobian product with the upstream gradient g = dL/d out:
 *   grad[i][:] = -(1/sigma^2) sum_j k_ij (g_i . b_j) (x_i - y_j)
 * Shapes: x (M, D), y (N, D), b (N, C), g (M, C), grad (M, D), all float32.
 * Requires 1 <= D <= 8, 1 <= C <= 8. N = 0 writes zeros.
 */
KEOPS_API int keops_gauss_sum_grad_x(const float* x, const float* y, const float* b, const float* g,
                           float* grad, int64_t M, int64_t N, int32_t D, int32_t C,
                           float sigma, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Gradient of the Gauss sum with respect to the columns y ("Kernel matrix reduction",
 * Variants: each partial derivative is its own reduction), for the upstream gradient g:
 *   grad_y[j][:] = (1/sigma^2) sum_i k_ij (g_i . b_j) (x_i - y_j)
 * Shapes: x (M, D), y (N, D), b (N, C), g (M, C), grad_y (N, D), all float32.
 * Requires 1 <= D <= 8, 1 <= C <= 8. M = 0 writes zeros; N = 0 is a no-op.
 */
KEOPS_API int keops_gauss_sum_grad_y(const float* x, const float* y, const float* b, const float* g,
                                     float* grad_y, int64_t M, int64_t N, int32_t D, int32_t C,
                                     float sigma, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/*
 * Gradient of the Gauss sum with respect to the weights b (the sum is linear in b):
 *   grad_b[j][c] = sum_i k_ij g[i][c]
 * Shapes: x (M, D), y (N, D), g (M, C), grad_b (N, C), all float32.
 * Requires 1 <= D <= 8, 1 <= C <= 8. M = 0 writes zeros; N = 0 is a no-op.
 */
KEOPS_API int keops_gauss_sum_grad_b(const float* x, const float* y, const float* g, float* grad_b,
                                     int64_t M, int64_t N, int32_t D, int32_t C, float sigma,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Two-sided scaled Gauss sum ("FlashDiffusion: Fused Tiled Kernel Spectral Decomposition",
 * section 2.2: the operator diag(s) K diag(s) applied to a block V, with the right scaling
 * folded into the block and the left scaling into the accumulation):
 *   out[t][i][c] = row_scale[t][i] * sum_j k_ij col_scale[t][j] b[t][j][c]
 * Shapes and dtypes as keops_gauss_sum; row_scale (B, M) and col_scale (B, N) are float32 and
 * either may be NULL (= all ones). The diffusion operator is row_scale = col_scale = s with
 * x = y (see keops_diffusion_scaling). On the fp16 path a col_scale (of any sign) is applied
 * in float32 before the weights are normalised and rounded to fp16.
 */
KEOPS_API int keops_gauss_sum_scaled(const void* x, const void* y, const void* b, const float* row_scale,
                                     const float* col_scale, float* out, int64_t B, int64_t M, int64_t N,
                                     int32_t D, int32_t C, float sigma, keops_dtype dtype, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/*
 * Backward pass of the Gauss sum out = keops_gauss_sum(x, y, b) for an upstream gradient
 * g = dL/d out (the reverse-mode rule of "Kernel Operations on the GPU, with Autodiff,
 * without Memory Overflows": every partial derivative of a reduction is a reduction of the
 * same pairs; the flash-attention page times this forward + backward in its Figure 2):
 *   grad_x[t][i] = -(1/sigma^2) sum_j k_ij (g_i . b_j)(x_i - y_j)
 *   grad_y[t][j] =  (1/sigma^2) sum_i k_ij (g_i . b_j)(x_i - y_j)
 *   grad_b[t][j] =  sum_i k_ij g_i
 * Any of grad_x (B, M, D), grad_y (B, N, D), grad_b (B, N, C) may be NULL (not computed).
 * g (B, M, C) and every gradient are float32. dtype KEOPS_F32: x, y, b float32 with the
 * limits of keops_gauss_sum_grad_x (B = 1, 1 <= D <= 8, 1 <= C <= 8). dtype KEOPS_F16: x, y, b
 * fp16 with the limits and alignment of the fp16 keops_gauss_sum (any B, 1 <= D <= 128,
 * 1 <= C <= 64), b and every gradient 16-byte aligned; the pair weights k_ij (g_i . b_j) are
 * rounded to fp16 (after the weight vectors are normalised, so nothing overflows) and
 * accumulate in fp32. KEOPS_BF16, and KEOPS_F32 with D > 8, return KEOPS_ERR_UNSUPPORTED.
 */
KEOPS_API int keops_gauss_sum_backward(const void* x, const void* y, const void* b, const float* g, float* grad_x,
                                       float* grad_y, float* grad_b, int64_t B, int64_t M, int64_t N, int32_t D,
                                       int32_t C, float sigma, keops_dtype dtype, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/*
 * Normalisation passes of the diffusion operator ("FlashDiffusion: Fused Tiled Kernel
 * Spectral Decomposition", section 2.2: the q and d passes are kernel applications with the
 * block replaced by ones and by q^-alpha), for the self-kernel K_ij = k(x_i, x_j):
 *   q = K 1,   p = q^-alpha,   d = p * (K p),   s = p / sqrt(d)
 * so that diag(s) K diag(s) = D^-1/2 K_alpha D^-1/2 with K_alpha = diag(p) K diag(p) and
 * D = diag(K_alpha 1), the symmetric form of the alpha-normalised diffusion matrix.
 * Shapes: x (B, N, D) of the dtype, with the limits of keops_gauss_sum for C = 1 (float32
 * with D <= 8 needs B = 1; fp16, bf16, and float32 with 9 <= D <= 128 take any B);
 * s (B, N) float32; q and d (B, N) float32 or NULL. alpha must be finite.
 */
KEOPS_API int keops_diffusion_scaling(const void* x, float* s, float* q, float* d, int64_t B, int64_t N, int32_t D,
                                      float sigma, float alpha, keops_dtype dtype, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes `op` (a keops_op) needs for these arguments on the current device
 * (unused arguments are ignored; KEOPS_OP_DIFFUSION_SCALING reads N, D and B). For
 * KEOPS_OP_GAUSS_SUM_SCALED and KEOPS_OP_GAUSS_SUM_BACKWARD the size covers every choice of
 * the optional arguments. Returns 0 for unsupported or invalid arguments. */
KEOPS_API size_t keops_workspace_bytes(int op, int64_t B, int64_t M, int64_t N, int32_t D, int32_t C,
                             int32_t K, keops_dtype dtype);

/* Static text for a status code. */
KEOPS_API const char* keops_status_string(int status);

/* Detail of the last failure on the calling thread ("" after a success). */
KEOPS_API const char* keops_last_error(void);

/* Library version string. */
KEOPS_API const char* keops_version(void);

/* Measurement aid (not needed to compute anything): timing of the main sweep of a Gauss sum,
 * i.e. the launch of the kernel that carries the pair work (the low-D float32 family's
 * matrix-core sweep, or the matrix-core family's forward sweep); the preparation and
 * split-combine kernels around it are excluded. keops_gauss_sum, keops_gauss_sum_noalloc and
 * keops_gauss_sum_scaled record it.
 *   keops_sweep_timing(1) makes every following such call on the calling thread record a
 *   pair of HIP events on its stream around that launch; keops_sweep_timing(0)
 *   stops and discards what was recorded.
 *   keops_sweep_timing_read(&ms, &count) waits for the recorded pairs, returns their summed
 *   elapsed milliseconds and their number, and clears them (timing stays enabled).
 * The events are created with hipEventCreate and destroyed by the read; no device memory is
 * allocated. Returns KEOPS_OK, or KEOPS_ERR_HIP if an event call failed (detail in
 * keops_last_error). */
KEOPS_API int keops_sweep_timing(int enable);
KEOPS_API int keops_sweep_timing_read(float* ms, int* count);

#ifdef __cplusplus
}
#endif

#endif /* KEOPS_MI355X_H */
