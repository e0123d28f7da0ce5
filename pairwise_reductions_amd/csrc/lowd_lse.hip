// Low-D log-sum-exp reduction ("Kernel matrix reduction", Overview: the reductions include
// a log-sum-exp over j): out_i = log sum_j exp(-|x_i - y_j|^2 / (2 sigma^2)), with the
// exponent evaluated as in lowd_sum.hip. The float64 form of lowd_mfma.hip's matrix-core sweep:
// it runs when the device-side decision declines the matrix cores.
#include "lowd_common.h"

namespace keops {
namespace lowd {
namespace {

// Per row a running shift m (float64, log2 units) and l = sum_j 2^{e_ij - m}. The shift is
// raised only when a tile holds a term above 2^kLseSlack, so rescales are rare.
template <int D, int R, int U>
__global__ void __launch_bounds__(kBlock)
lse_kernel(const float* __restrict__ x, const float* __restrict__ y,
           const double* __restrict__ cols, float* __restrict__ out,
           LsePartial* __restrict__ partial, int64_t M, int64_t N, int64_t cps, double c2,
           const int* __restrict__ skip) {
  if (skip[0] && !skip[1]) return;  // the matrix-core sweep takes these inputs
  constexpr int P = (D + 2) & ~1;
  const int64_t split = blockIdx.y;
  const int64_t j0 = split * cps;
  const int64_t j1 = (j0 + cps < N) ? j0 + cps : N;
  const int64_t row0 = (int64_t)blockIdx.x * (kBlock * R) + threadIdx.x;

  double xp[R][D], Ap[R], mref[R];
  float l[R];
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
    const double A = -c2 * s;
    // The first column of the split sets the initial shift exactly.
    double e0 = A + cols[j0 * P + D];
#pragma unroll
    for (int d = 0; d < D; ++d) e0 = fma(xp[r][d], cols[j0 * P + d], e0);
    mref[r] = e0;
    Ap[r] = A - e0;
    l[r] = 0.0f;
  }

  int64_t j = j0;
  for (; j + U <= j1; j += U) {
    float e32[R][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const double* cj = cols + (j + u) * P;
      double v[D];
#pragma unroll
      for (int d = 0; d < D; ++d) v[d] = cj[d];
      const double Bj = cj[D];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        double e = Ap[r] + Bj;
#pragma unroll
        for (int d = 0; d < D; ++d) e = fma(xp[r][d], v[d], e);
        e32[r][u] = (float)e;
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float tmax = e32[r][0];
#pragma unroll
      for (int u = 1; u < U; ++u) tmax = fmaxf(tmax, e32[r][u]);
      if (tmax > kLseSlack) {
        l[r] *= exp2_hw(-tmax);
        mref[r] += (double)tmax;
        Ap[r] -= (double)tmax;
        // The float values were rounded relative to the old shift (up to 2^-9 at |e| ~ 2^14):
        // evaluate the tile again, in float64, relative to the new one.
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const double* cj = cols + (j + u) * P;
          double e = Ap[r] + cj[D];
#pragma unroll
          for (int d = 0; d < D; ++d) e = fma(xp[r][d], cj[d], e);
          e32[r][u] = (float)e;
        }
      }
      float t = 0.0f;
#pragma unroll
      for (int u = 0; u < U; ++u) t += exp2_hw(e32[r][u]);
      l[r] += t;
    }
  }
  for (; j < j1; ++j) {
    const double* cj = cols + j * P;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      double e = Ap[r] + cj[D];
#pragma unroll
      for (int d = 0; d < D; ++d) e = fma(xp[r][d], cj[d], e);
      float e32 = (float)e;
      if (e32 > kLseSlack) {
        l[r] *= exp2_hw(-e32);
        mref[r] += (double)e32;
        Ap[r] -= (double)e32;
        e32 = (float)(e - (double)e32);  // the remainder the float rounding dropped
      }
      l[r] += exp2_hw(e32);
    }
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t i = row0 + (int64_t)r * kBlock;
    if (i >= M) continue;
    if (gridDim.y == 1) {
      out[i] = (float)((mref[r] + (double)log2f(l[r])) * M_LN2);
    } else {
      LsePartial p;
      p.m = mref[r];
      p.l = l[r];
      p.pad = 0.0f;
      partial[split * M + i] = p;
    }
  }
}

template <int D>
hipError_t lse_d(const float* x, const float* y, const double* cols, float* out, double* partial,
                 int64_t M, int64_t N, double c2, const int* skip, const Plan& p, hipStream_t s) {
  dim3 grid((unsigned)p.row_blocks, (unsigned)p.splits);
  lse_kernel<D, kRowsLse, kLseTile><<<grid, kBlock, 0, s>>>(
      x, y, cols, out, reinterpret_cast<LsePartial*>(partial), M, N, p.cols_per_split, c2, skip);
  return hipGetLastError();
}

}  // namespace
}  // namespace lowd

hipError_t launch_lse_lowd(const float* x, const float* y, double* cols, float* out, double* partial, void* mf,
                           int64_t M, int64_t N, int D, double c2, const Plan& p, hipStream_t s) {
  hipError_t e = launch_mf_prepare(x, y, nullptr, false, cols, mf, M, N, D, 0, c2, s, false, mf_lse_square(D, p.mf_rt));
  if (e != hipSuccess) return e;
  const int* skip = mf_decision(mf);
  {
#define KEOPS_LSE(Dv) lowd::lse_d<Dv>(x, y, cols, out, partial, M, N, c2, skip, p, s)
    auto run = [&]() -> hipError_t { KEOPS_SWITCH_D(D, KEOPS_LSE) };
#undef KEOPS_LSE
    e = run();
  }
  if (e != hipSuccess) return e;
  e = launch_mf_lse(out, partial, mf, M, N, D, p, s);
  if (e != hipSuccess) return e;
  if (p.splits > 1) {
    e = lowd::launch_combine_lse(reinterpret_cast<const lowd::LsePartial*>(partial), out, M, p.splits, s);
    if (e != hipSuccess) return e;
  }
  return launch_mf_lse_fix(x, y, out, mf, M, N, D, c2, p, s);
}

}  // namespace keops
