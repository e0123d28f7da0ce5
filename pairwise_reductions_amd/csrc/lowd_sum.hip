// Low-D float32 Gauss sum ("Kernel matrix reduction", Implementation sketch: the Gaussian
// kernel matrix-vector product a_i = sum_j exp(-|x_i - y_j|^2 / (2 sigma^2)) b_j). The sweep
// here evaluates the exponent in float64; it runs when the device-side decision declines the
// matrix-core sweep of lowd_mfma.hip (both are launched, one returns at once).
//
// Gaussian exponent. For the sum and log-sum-exp reductions the exponent in base 2,
//   e_ij = -c2 ||x_i - y_j||^2,  c2 = log2(e) / (2 sigma^2),
// is evaluated in float64 from centred coordinates u_i = x_i - o, v_j = y_j - o (o = y_0):
//   e_ij = A_i + B_j + sum_d (2 c2 u_id) v_jd,  A_i = -c2 |u_i|^2,  B_j = -c2 |v_j|^2,
// i.e. one add and D fused multiply-adds per pair at full float64 VALU rate (the same
// issue rate as unpacked float32 on this chip). float64 keeps the cancellation between the
// large terms below 1e-11 in e for inputs within 1e4 sigma of one another, far more exact
// than a float32 difference would be; e is then rounded to float32 for v_exp_f32.
#include "lowd_common.h"

namespace keops {
namespace lowd {
namespace {

// out[i][c] = sum_j 2^{e_ij} b[j][c] over the columns [j0, j1) of this split. With one split
// `out` is the final output (times rscale[i] when given), otherwise partial[split][i][c].
template <int D, int C, int R>
__global__ void __launch_bounds__(kBlock)
gauss_sum_kernel(const float* __restrict__ x, const float* __restrict__ y,
                 const double* __restrict__ cols, const float* __restrict__ b,
                 float* __restrict__ out, const float* __restrict__ rscale, int64_t M, int64_t N, int64_t cps,
                 double c2, const int* __restrict__ skip) {
  if (skip && skip[0] && !skip[1]) return;  // the matrix-core sweep takes these inputs
  constexpr int P = (D + 2) & ~1;
  const int64_t split = blockIdx.y;
  const int64_t j0 = split * cps;
  const int64_t j1 = (j0 + cps < N) ? j0 + cps : N;
  const int64_t row0 = (int64_t)blockIdx.x * (kBlock * R) + threadIdx.x;

  double xp[R][D], A[R];
  float acc[R][C];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int64_t i = row0 + (int64_t)r * kBlock;
    i = i < M ? i : M - 1;
    double s = 0.0;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const double u = (double)x[i * D + d] - (double)y[d];
      xp[r][d] = 2.0 * c2 * u;
      s = fma(u, u, s);
    }
    A[r] = -c2 * s;
#pragma unroll
    for (int c = 0; c < C; ++c) acc[r][c] = 0.0f;
  }

  for (int64_t jc = j0; jc < j1; jc += kChunk) {
    const int64_t je = (jc + kChunk < j1) ? jc + kChunk : j1;
    float part[R][C];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < C; ++c) part[r][c] = 0.0f;
#pragma unroll 4
    for (int64_t j = jc; j < je; ++j) {
      const double* cj = cols + j * P;
      double v[D];
#pragma unroll
      for (int d = 0; d < D; ++d) v[d] = cj[d];
      const double Bj = cj[D];
      float bj[C];
#pragma unroll
      for (int c = 0; c < C; ++c) bj[c] = b[j * C + c];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        double e = A[r] + Bj;
#pragma unroll
        for (int d = 0; d < D; ++d) e = fma(xp[r][d], v[d], e);
        const float k = exp2_hw((float)e);
#pragma unroll
        for (int c = 0; c < C; ++c) part[r][c] = fmaf(k, bj[c], part[r][c]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int c = 0; c < C; ++c) acc[r][c] += part[r][c];
  }

  float* dst = out + split * M * C;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t i = row0 + (int64_t)r * kBlock;
    if (i < M) {
      const float sc = (rscale && gridDim.y == 1) ? rscale[i] : 1.0f;
#pragma unroll
      for (int c = 0; c < C; ++c) dst[i * C + c] = sc * acc[r][c];
    }
  }
}

template <int D, int C>
hipError_t gauss_sum_dc(const float* x, const float* y, const double* cols, const float* b, float* dst,
                        const float* rscale, int64_t M, int64_t N, double c2, const int* skip, const Plan& p,
                        hipStream_t s) {
  dim3 grid((unsigned)p.row_blocks, (unsigned)p.splits);
  if (p.R == kRowsSumSmall)
    gauss_sum_kernel<D, C, kRowsSumSmall><<<grid, kBlock, 0, s>>>(x, y, cols, b, dst, rscale, M, N, p.cols_per_split,
                                                                   c2, skip);
  else
    gauss_sum_kernel<D, C, kRowsSum><<<grid, kBlock, 0, s>>>(x, y, cols, b, dst, rscale, M, N, p.cols_per_split, c2,
                                                             skip);
  return hipGetLastError();
}

template <int D>
hipError_t gauss_sum_d(int C, const float* x, const float* y, const double* cols, const float* b, float* dst,
                       const float* rscale, int64_t M, int64_t N, double c2, const int* skip, const Plan& p,
                       hipStream_t s) {
#define KEOPS_GS_C(Cv) gauss_sum_dc<D, Cv>(x, y, cols, b, dst, rscale, M, N, c2, skip, p, s)
  KEOPS_SWITCH_C(C, KEOPS_GS_C)
#undef KEOPS_GS_C
}

}  // namespace
}  // namespace lowd

hipError_t launch_gauss_sum_lowd(const float* x, const float* y, double* cols, const float* b, const float* rscale,
                                 float* out, float* partial, void* mf, int64_t M, int64_t N, int D, int C, double c2,
                                 const Plan& p, hipStream_t s) {
  float* dst = p.splits > 1 ? partial : out;
  // Operands of both sweeps and the device-side choice between them.
  hipError_t e = launch_mf_prepare(x, y, b, false, cols, mf, M, N, D, C, c2, s, true, mf_sum_square(D, C, p.mf_rt));
  if (e != hipSuccess) return e;
  const int* gate = mf_decision(mf);
  auto run = [&]() -> hipError_t {
#define KEOPS_GS(Dv) lowd::gauss_sum_d<Dv>(C, x, y, cols, b, dst, rscale, M, N, c2, gate, p, s)
    KEOPS_SWITCH_D(D, KEOPS_GS)
#undef KEOPS_GS
  };
  e = run();
  if (e != hipSuccess) return e;
  sweep_event(s, true);
  e = launch_mf_sum(rscale, dst, mf, M, N, D, C, p, s);
  sweep_event(s, false);
  if (e != hipSuccess) return e;
  return launch_mf_finish(partial, out, x, y, b, rscale, mf, M, N, D, C, p.splits, c2, s);
}

}  // namespace keops
