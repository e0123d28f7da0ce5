// Low-D gradient of the Gauss sum with respect to x ("Kernel Operations on the GPU, with
// Autodiff, without Memory Overflows": each partial derivative of a reduction is itself a
// reduction over the same pairs):
//   grad_i = -(1/sigma^2) sum_j k_ij (g_i . b_j) (x_i - y_j).
// With one channel the matrix-core sweep of lowd_mfma.hip runs instead whenever the
// device-side decision admits the inputs; this float32 sweep covers the rest.
#include "lowd_common.h"

namespace keops {
namespace lowd {
namespace {

// grad_i = -(1/sigma^2) sum_j k_ij (g_i . b_j) (x_i - y_j), with the differences taken
// first in float32 (they are reused for d^2 and for the accumulation).
template <int D, int C, int R>
__global__ void __launch_bounds__(kBlock)
grad_x_kernel(const float* __restrict__ x, const float* __restrict__ y, const float* __restrict__ b,
              const float* __restrict__ g, float* __restrict__ out, int64_t M, int64_t N,
              int64_t cps, float c2f, float inv_sigma2, const int* __restrict__ skip) {
  if (skip && skip[0] && !skip[1]) return;  // the matrix-core sweep takes these inputs
  const int64_t split = blockIdx.y;
  const int64_t j0 = split * cps;
  const int64_t j1 = (j0 + cps < N) ? j0 + cps : N;
  const int64_t row0 = (int64_t)blockIdx.x * (kBlock * R) + threadIdx.x;

  float xr[R][D], gr[R][C], acc[R][D];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int64_t i = row0 + (int64_t)r * kBlock;
    i = i < M ? i : M - 1;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      xr[r][d] = x[i * D + d];
      acc[r][d] = 0.0f;
    }
#pragma unroll
    for (int c = 0; c < C; ++c) gr[r][c] = g[i * C + c];
  }

  for (int64_t jc = j0; jc < j1; jc += kChunk) {
    const int64_t je = (jc + kChunk < j1) ? jc + kChunk : j1;
    float part[R][D];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int d = 0; d < D; ++d) part[r][d] = 0.0f;
#pragma unroll 4
    for (int64_t j = jc; j < je; ++j) {
      float yj[D], bj[C];
#pragma unroll
      for (int d = 0; d < D; ++d) yj[d] = y[j * D + d];
#pragma unroll
      for (int c = 0; c < C; ++c) bj[c] = b[j * C + c];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float dx[D];
        float d2 = 0.0f;
#pragma unroll
        for (int d = 0; d < D; ++d) {
          dx[d] = xr[r][d] - yj[d];
          d2 = fmaf(dx[d], dx[d], d2);
        }
        const float k = exp2_hw(-(c2f * d2));
        float w;
        if constexpr (C == 1) {
          w = k * bj[0];  // g_i is applied once per row at the end
        } else {
          float gb = 0.0f;
#pragma unroll
          for (int c = 0; c < C; ++c) gb = fmaf(gr[r][c], bj[c], gb);
          w = k * gb;
        }
#pragma unroll
        for (int d = 0; d < D; ++d) part[r][d] = fmaf(w, dx[d], part[r][d]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int d = 0; d < D; ++d) acc[r][d] += part[r][d];
  }

  float* dst = out + split * M * D;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t i = row0 + (int64_t)r * kBlock;
    if (i >= M) continue;
    const float scale = (C == 1) ? -inv_sigma2 * gr[r][0] : -inv_sigma2;
#pragma unroll
    for (int d = 0; d < D; ++d) dst[i * D + d] = scale * acc[r][d];
  }
}

template <int D, int C>
hipError_t grad_dc(const float* x, const float* y, const float* b, const float* g, float* dst,
                   int64_t M, int64_t N, float c2f, float inv_sigma2, const int* skip, const Plan& p,
                   hipStream_t s) {
  dim3 grid((unsigned)p.row_blocks, (unsigned)p.splits);
  grad_x_kernel<D, C, kRowsGrad><<<grid, kBlock, 0, s>>>(x, y, b, g, dst, M, N, p.cols_per_split, c2f, inv_sigma2,
                                                         skip);
  return hipGetLastError();
}

template <int D>
hipError_t grad_d(int C, const float* x, const float* y, const float* b, const float* g, float* dst,
                  int64_t M, int64_t N, float c2f, float inv_sigma2, const int* skip, const Plan& p,
                  hipStream_t s) {
#define KEOPS_GR_C(Cv) grad_dc<D, Cv>(x, y, b, g, dst, M, N, c2f, inv_sigma2, skip, p, s)
  KEOPS_SWITCH_C(C, KEOPS_GR_C)
#undef KEOPS_GR_C
}

}  // namespace
}  // namespace lowd

hipError_t launch_grad_x_lowd(const float* x, const float* y, const float* b, const float* g, float* grad,
                              float* partial, void* mf, int64_t M, int64_t N, int D, int C, float c2f,
                              float inv_sigma2, const Plan& p, hipStream_t s) {
  float* dst = p.splits > 1 ? partial : grad;
  hipError_t e = hipSuccess;
  const int* skip = nullptr;
  if (C == 1) {
    // the matrix-core sweep's operands: row and column pieces (log2 |b_j| in the exponent),
    // (sign b_j, -sign b_j y_j) per column
    e = launch_mf_prepare(x, y, b, true, nullptr, mf, M, N, D, 1, (double)c2f, s);
    if (e != hipSuccess) return e;
    skip = mf_decision(mf);
  }
  {
#define KEOPS_GR(Dv) lowd::grad_d<Dv>(C, x, y, b, g, dst, M, N, c2f, inv_sigma2, skip, p, s)
    auto run = [&]() -> hipError_t { KEOPS_SWITCH_D(D, KEOPS_GR) };
#undef KEOPS_GR
    e = run();
  }
  if (e != hipSuccess) return e;
  if (C == 1) {
    e = launch_mf_grad(x, g, dst, inv_sigma2, mf, M, N, D, p, s);
    if (e != hipSuccess) return e;
  }
  if (p.splits == 1) return e;
  const int64_t n = M * D;
  return lowd::launch_combine_sum(partial, grad, n, p.splits, nullptr, 1, s);
}

}  // namespace keops
