// Internal declarations shared by the C-ABI layer and the kernel files. Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace keops {

constexpr int kBlock = 256;          // threads per workgroup (4 wave64s) for the low-D family
constexpr int kMaxLowD = 8;          // largest D of the low-D family
constexpr int kMaxLowC = 8;          // largest C of the low-D family
constexpr int kMaxK = 64;            // largest K of argKmin (the per-row list lives in VGPRs)
constexpr size_t kAlign = 256;       // alignment of workspace sections

// Column record stride (doubles) of the prepared low-D column table: D centred coordinates
// followed by one per-column exponent term, padded to an even count (16-byte records).
__host__ __device__ inline int col_stride(int D) { return (D + 2) & ~1; }

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Launch plan of one low-D reduction: rows per workgroup and the number of column splits.
struct Plan {
  int rows_per_block;   // kBlock * R
  int R;                // rows per lane
  int64_t row_blocks;   // ceil(M / rows_per_block)
  int64_t splits;       // S: column ranges reduced independently, then combined in order
  int64_t cols_per_split;
  // Gauss sum only: the matrix-core sweep's row tiles of 16 per wave and its workgroup count
  // along the rows (it shares the column splits with the float64 sweep).
  int mf_rt = 0;
  int64_t mf_row_blocks = 0;
};

Plan plan_lowd(int op, int64_t M, int64_t N, int D, int C, int K, int num_cus);
int device_cus();

// Per-op partial-result bytes per (split, row). Ops follow keops_op; 6 is argKmin + LSE.
size_t partial_bytes_per_row(int op, int D, int C, int K);

// ---- launchers (return hipError_t of the launch) ----------------------------------------
// cols[j] = (y_j - o, -c2 |y_j - o|^2) in float64, o = y_0 when `centre`, else o = 0.
hipError_t launch_prep_cols(const float* y, double* cols, int64_t N, int D, double c2,
                            bool centre, hipStream_t s);
// out[i][c] = rscale[i] * sum_j 2^{-c2 |x_i - y_j|^2} b[j][c] (rscale may be null). Prepares the
// matrix-core operands in `mf` (mf_region_bytes) and the float64 column table in `cols`, then
// launches both sweeps; the device-side decision lets exactly one of them do the work.
hipError_t launch_gauss_sum_lowd(const float* x, const float* y, double* cols, const float* b,
                                 const float* rscale, float* out, float* partial, void* mf,
                                 int64_t M, int64_t N, int D, int C, double c2, const Plan& p,
                                 hipStream_t s);
// Matrix-core Gauss sum pieces (lowd_mfma.hip): operand region size (C = 0: no weights); the
// decision, two ints (gate, bad): the matrix-core sweep runs when gate != 0 and bad == 0; row
// tiles per wave for C channels; preparation (also writes the float64 column table; b may be
// null) and sweeps.
// Measurement aid: records a HIP event pair on the stream around the main sweep's launch while
// keops_sweep_timing is enabled on the calling thread (begin before the launch, end after).
void sweep_event(hipStream_t s, bool begin);
size_t mf_region_bytes(int64_t M, int64_t N, int D, int W, bool grad = false);  // W: floats per column record
const int* mf_decision(const void* region);
int mf_rows_per_lane(int op, int D, int C);   // op: 0 sum, 1 log-sum-exp, 3 gradient
int mf_occupancy(int op, int D, int C, int rt);  // resident workgroups per CU of that sweep
// The single-channel sum at D <= 3 runs on 32 x 32 tiles when the plan gives 2 or 4 row tiles
// of 16 per wave (the preparation must then write that layout: square = true).
bool mf_sum_square(int D, int C, int rt);
// The log-sum-exp likewise (D <= 3); its rows far from every column are then recomputed by
// launch_mf_lse_fix after the split combine.
bool mf_lse_square(int D, int rt);
int knn_occupancy(int D, int K);                 // resident workgroups per CU of the argKmin sweep
// set_aside (the Gauss sum only): a box too wide for the matrix cores may be replaced by one
// around the sample median that sets a few outlying points aside (launch_mf_finish then sums
// their terms).
hipError_t launch_mf_prepare(const float* x, const float* y, const float* b, bool with_y, double* cols,
                             void* region, int64_t M, int64_t N, int D, int C, double c2, hipStream_t s,
                             bool set_aside = false, bool square = false);
// The Gauss sum's last step after either sweep: combines the S column splits of partial into out
// (S > 1) with rscale, and when the preparation set points aside adds the set-aside columns'
// terms to every other row and sums every set-aside row over all columns.
hipError_t launch_mf_finish(const float* partial, float* out, const float* x, const float* y, const float* b,
                            const float* rscale, void* region, int64_t M, int64_t N, int D, int C, int64_t S,
                            double c2, hipStream_t s);
// gradient with respect to x, one channel: dst[i][d] = -(g_i / sigma^2) sum_j k_ij b_j (x_i - y_j)
hipError_t launch_mf_grad(const float* x, const float* g, float* dst, float inv_sigma2, void* region,
                          int64_t M, int64_t N, int D, const Plan& p, hipStream_t s);
hipError_t launch_mf_sum(const float* rscale, float* dst, void* region, int64_t M, int64_t N, int D,
                         int C, const Plan& p, hipStream_t s);
// log-sum-exp on the matrix cores: out (one split) or per-split (m, l) pairs in `partial`
hipError_t launch_mf_lse(float* out, void* partial, void* region, int64_t M, int64_t N, int D,
                         const Plan& p, hipStream_t s);
// Recomputes, from a float64 exponent, the rows of a finished matrix-core log-sum-exp whose value
// is below 64 ln 2 or not finite (only after the 32 x 32 form; the decision in region gates it).
hipError_t launch_mf_lse_fix(const float* x, const float* y, float* out, void* region, int64_t M, int64_t N, int D,
                             double c2, const Plan& p, hipStream_t s);
// log-sum-exp: prepares as launch_gauss_sum_lowd (no weights) and runs the matrix-core or the
// float64 sweep, chosen on the device.
hipError_t launch_lse_lowd(const float* x, const float* y, double* cols, float* out,
                           double* partial, void* mf, int64_t M, int64_t N, int D, double c2,
                           const Plan& p, hipStream_t s);
// The matrix-core log-sum-exp that the argKmin + LSE call may run beside a plain argKmin
// sweep: its operand region, its per-split partials and its plan (a log-sum-exp plan).
struct KnnLse {
  void* region;
  void* partial;
  const Plan* plan;
};
// argKmin of d^2_ij - w_j (w may be null), optionally with the log-sum-exp reduction
// (with_lse, only without weights): builds the uncentred column table in `cols` and the
// screening bound in *ymax, then screens every pair. With mf_lse the log-sum-exp runs on the
// matrix cores beside the plain argKmin sweep whenever the device-side decision admits the
// inputs, and in the fused float64 sweep otherwise.
// Bytes of the float32 screening table of the plain argKmin sweep (N records).
size_t knn_screen_bytes(int64_t N, int D);
// argKmin sweeps take their rows in spatial order, and start each row's screen from the K-th
// smallest key over a few nearby columns, from this many rows on; the workspace (a bounding
// box, cell counts, the row and column orders, the M starting thresholds and, for the
// matrix-core screen, its pieces) is knn_order_bytes(M, N, D, K).
constexpr int64_t kKnnOrderMinRows = 16384;
bool knn_orders_rows(int64_t M);
size_t knn_order_bytes(int64_t M, int64_t N, int D, int K);
// Whether the argKmin workspace holds the pieces of the matrix-core screen (rows in spatial
// order, D <= 3, K <= 16); the plain sweep (no weights, fewer than 65000 columns per split)
// then runs on it.
bool knn_screens_on_matrix_cores(int64_t M, int64_t N, int D, int K);
hipError_t launch_knn_lowd(const float* x, const float* y, const float* w, double* cols, float* scr, void* order_ws,
                           double* ymax,
                           int32_t* idx, float* dist, void* partial, float* lse_out,
                           double* lse_partial, int64_t M, int64_t N, int D, int K, double c2,
                           bool with_lse, const Plan& p, hipStream_t s, const KnnLse* mf_lse = nullptr);
// Gradient with respect to x (float32 sweep; with C = 1 the matrix-core sweep, prepared in `mf`,
// takes it when the device-side decision admits the inputs).
hipError_t launch_grad_x_lowd(const float* x, const float* y, const float* b, const float* g,
                              float* grad, float* partial, void* mf, int64_t M, int64_t N, int D, int C,
                              float c2f, float inv_sigma2, const Plan& p, hipStream_t s);
hipError_t launch_fill(float* out, int64_t n, float value, hipStream_t s);
// Element-wise steps: out[j][c] = scale[j] b[j][c]; out = in^e; out = p / sqrt(d).
hipError_t launch_scale_rows(const float* b, const float* scale, float* out, int64_t N, int C,
                             hipStream_t s);
hipError_t launch_pow(const float* in, float* out, int64_t n, float e, hipStream_t s);
hipError_t launch_div_sqrt(const float* p, const float* d, float* out, int64_t n, hipStream_t s);

// Matrix-core batched Gauss sums. x, y: [B][M|N][D] of `xy` type (fp16, bf16, or float32
// split into fp16 hi + lo parts on the matrix cores).
enum ElemType { kElemF16 = 0, kElemBF16 = 1, kElemF32 = 2 };
// Any 1 <= D <= 128 and 1 <= C <= 64. The kernels read rows of a multiple of 16 features
// (16-byte vectors); other widths are first copied into the workspace with zero features
// appended (zeros change no squared distance), see highd_stored_features.
bool highd_supported(int D, int C);
// Feature count the matrix-core kernels are launched with: D rounded up to a multiple of 16.
int highd_stored_features(int D);
// rows x Dp copies of rows x D arrays (elements of elem_bytes = 2 or 4), zero past D; and the
// float32 narrowing back from Dp to D columns.
hipError_t launch_pad_rows(const void* in, void* out, int64_t rows, int D, int Dp, int elem_bytes, hipStream_t s);
hipError_t launch_narrow_rows(const float* in, float* out, int64_t rows, int Dp, int D, hipStream_t s);
// out[t][i][c] = rscale[t][i] * sum_j Phi_ij cscale[t][j] b[t][j][c]; b is of type bt;
// rscale and cscale may be null. Anything but fp16 points with fp16 weights and no column
// scale takes the weight-normalising column preparation (`general`), which needs a slightly
// larger workspace.
bool highd_general(ElemType xy, ElemType bt, bool col_scaled);
size_t highd_workspace_bytes(int64_t B, int64_t M, int64_t N, int D, int C, ElemType xy, bool general);
hipError_t launch_gauss_sum_highd(const void* x, const void* y, ElemType xy, const void* b, ElemType bt,
                                  const float* rscale, const float* cscale, float* out,
                                  void* workspace, int64_t B, int64_t M, int64_t N, int D, int C,
                                  float sigma, hipStream_t s);
// out[t][i] = -tau sum_j Phi_ij (a_i . bv_j)(x_i - y_j): rows x with weights a [B][M][C],
// columns y with weights bv [B][N][C] (each fp16, or fp32 when flagged); out [B][M][D].
// Channels of b up to which the y-gradient sweep also produces the b-gradient.
int hd_fused_weight_channels();
// With out2 (C <= hd_fused_weight_channels() only), the same sweep also writes out2[t][i] = sum_j Phi_ij bv_j, [B][M][C].
size_t highd_grad_workspace_bytes(int64_t B, int64_t M, int64_t N, int D, int C, bool fused);
hipError_t launch_gauss_sum_grad_highd(const void* x, const void* y, const void* a, bool a_f32,
                                       const void* bv, bool bv_f32, float* out, float* out2,
                                       void* workspace, int64_t B, int64_t M, int64_t N, int D,
                                       int C, float sigma, hipStream_t s);

}  // namespace keops
