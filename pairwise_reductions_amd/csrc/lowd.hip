// Shared low-D pieces: the column table, fills, the fixed-order combines of per-split
// partials, a few element-wise steps and the launch planner. The sweeps live in
// lowd_mfma.hip (matrix-core exponent), lowd_sum.hip, lowd_lse.hip, lowd_knn.hip and
// lowd_grad.hip.
#include "lowd_common.h"

namespace keops {
namespace lowd {
namespace {

// ------------------------------------------------------------------------ column prep
// cols[j] = (y_j - o, B_j) in float64, o = y_0 when `centre`, else o = 0 (then B_j unused).
__global__ void __launch_bounds__(kBlock)
prep_cols_kernel(const float* __restrict__ y, double* __restrict__ cols, int64_t N, int D, int P,
                 double c2, int centre) {
  const int64_t j = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (j >= N) return;
  double s = 0.0;
  for (int d = 0; d < D; ++d) {
    const double o = centre ? (double)y[d] : 0.0;
    const double v = (double)y[j * D + d] - o;
    cols[j * P + d] = v;
    s = fma(v, v, s);
  }
  cols[j * P + D] = -c2 * s;
  for (int d = D + 1; d < P; ++d) cols[j * P + d] = 0.0;
}

__global__ void __launch_bounds__(kBlock) fill_kernel(float* out, int64_t n, float value) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i < n) out[i] = value;
}

// out[i] = rscale[i / C] * sum over s of partial[s][i], in increasing s.
__global__ void __launch_bounds__(kBlock)
combine_sum_kernel(const float* __restrict__ partial, float* __restrict__ out, int64_t n, int64_t S,
                   const float* __restrict__ rscale, int C) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  for (int64_t k = 0; k < S; ++k) s += partial[k * n + i];
  if (rscale) s *= rscale[i / C];
  out[i] = s;
}

__global__ void __launch_bounds__(kBlock)
combine_lse_kernel(const LsePartial* __restrict__ partial, float* __restrict__ out, int64_t M,
                   int64_t S, const int* __restrict__ mf, int run_if_mf) {
  if (mf && mf_admits(mf) != run_if_mf) return;  // the other form's partials
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i >= M) return;
  double m = partial[i].m;
  for (int64_t k = 1; k < S; ++k) m = fmax(m, partial[k * M + i].m);
  double l = 0.0;
  for (int64_t k = 0; k < S; ++k) {
    const LsePartial p = partial[k * M + i];
    l += (double)p.l * exp2(p.m - m);
  }
  out[i] = (float)((m + log2(l)) * M_LN2);
}

// out[j][c] = cs[j] * b[j][c]
__global__ void __launch_bounds__(kBlock)
scale_rows_kernel(const float* __restrict__ b, const float* __restrict__ cs, float* __restrict__ out, int64_t n,
                  int C) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i < n) out[i] = cs[i / C] * b[i];
}

// out[i] = in[i]^e (in > 0)
__global__ void __launch_bounds__(kBlock)
pow_kernel(const float* __restrict__ in, float* __restrict__ out, int64_t n, float e) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i < n) out[i] = powf(in[i], e);
}

// s[i] = p[i] / sqrt(d[i])
__global__ void __launch_bounds__(kBlock)
div_sqrt_kernel(const float* __restrict__ p, const float* __restrict__ d, float* __restrict__ s, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i < n) s[i] = p[i] / sqrtf(d[i]);
}

}  // namespace

hipError_t launch_combine_sum(const float* partial, float* out, int64_t n, int64_t S, const float* rscale, int C,
                              hipStream_t s) {
  if (n <= 0) return hipSuccess;
  combine_sum_kernel<<<(unsigned)ceil_div(n, kBlock), kBlock, 0, s>>>(partial, out, n, S, rscale, C);
  return hipGetLastError();
}

hipError_t launch_combine_lse(const LsePartial* partial, float* out, int64_t M, int64_t S, hipStream_t s,
                              const int* mf, int run_if_mf) {
  if (M <= 0) return hipSuccess;
  combine_lse_kernel<<<(unsigned)ceil_div(M, kBlock), kBlock, 0, s>>>(partial, out, M, S, mf, run_if_mf);
  return hipGetLastError();
}

}  // namespace lowd

using lowd::ceil_div;

// ------------------------------------------------------------------------- planning
size_t partial_bytes_per_row(int op, int D, int C, int K) {
  switch (op) {
    case 0: return sizeof(float) * (size_t)C;
    case 1: return sizeof(lowd::LsePartial);
    case 2: return sizeof(lowd::KeyIdx) * (size_t)lowd::argk_bucket(K);
    case 6: return sizeof(lowd::KeyIdx) * (size_t)lowd::argk_bucket(K) + sizeof(lowd::LsePartial);
    case 3: return sizeof(float) * (size_t)D;
  }
  return 0;
}

Plan plan_lowd(int op, int64_t M, int64_t N, int D, int C, int K, int num_cus) {
  Plan p;
  switch (op) {
    case 0: p.R = lowd::kRowsSum; break;
    case 1: p.R = lowd::kRowsLse; break;
    case 2:
    case 6: p.R = lowd::argk_rows(lowd::argk_bucket(K)); break;
    default: p.R = lowd::kRowsGrad; break;
  }
  if (op == 0) {
    // Few rows: four rows per lane would leave most CUs idle even with every column split,
    // so take one row per lane.
    const int64_t max_cols_splits = N / 256 > 1 ? N / 256 : 1;
    if (ceil_div(M, (int64_t)kBlock * p.R) * max_cols_splits < (int64_t)num_cus * 4) p.R = lowd::kRowsSumSmall;
  }
  p.rows_per_block = kBlock * p.R;
  p.row_blocks = M > 0 ? ceil_div(M, p.rows_per_block) : 0;
  // The matrix-core sweeps (Gauss sum, log-sum-exp, one-channel gradient) take 16 RT rows per
  // wave; the column splits are planned for them (the float64 / float32 sweeps, which run only
  // when the matrix-core ones decline, share them).
  int64_t lead_blocks = p.row_blocks;
  int64_t granule = 8;
  const bool mf = op == 0 || op == 1 || (op == 3 && C == 1);
  if (mf) {
    const int64_t max_cols_splits = N / 256 > 1 ? N / 256 : 1;
    int rt = mf_rows_per_lane(op, D, C);
    while (rt > 1 && ceil_div(M, (int64_t)64 * rt) * max_cols_splits < (int64_t)num_cus * 4) rt /= 2;
    p.mf_rt = rt;
    p.mf_row_blocks = M > 0 ? ceil_div(M, (int64_t)64 * rt) : 0;
    lead_blocks = p.mf_row_blocks;
    granule = 32;
  }
  // argKmin's matrix-core screen halves each split into runs of 16-column tiles
  if ((op == 2 || op == 6) && knn_screens_on_matrix_cores(M, N, D, K)) granule = 32;
  // Split the columns so that (a) there are at least lowd::wg_per_cu(op, C, D) workgroups per
  // compute unit over the launch, and (b) one split's column table stays within
  // lowd::kSplitCols columns, a working set that fits one XCD's L2 while the resident
  // workgroups (consecutive row blocks of the same split) stream it together. Every split
  // keeps >= 256 columns.
  const int64_t target = (int64_t)num_cus * lowd::wg_per_cu(op, C, D);
  int64_t S = 1;
  if (lead_blocks > 0 && lead_blocks < target) S = ceil_div(target, lead_blocks);
  if (S < ceil_div(N, lowd::kSplitCols)) S = ceil_div(N, lowd::kSplitCols);
  int64_t max_split = N / 256 > 1 ? N / 256 : 1;
  if ((op == 2 || op == 6) && max_split > 16) max_split = 16;  // argKmin partial lists are K entries per row
  if (S > max_split) S = max_split;
  if (S < 1) S = 1;
  // Columns per split: a multiple of 8 (32, two tiles, for the matrix-core sweep); the split
  // count is what that leaves.
  auto split_of = [&](int64_t s, int64_t& cps_out) {
    int64_t c = s > 1 ? ceil_div(N, s) : (N > 0 ? N : 1);
    c = ceil_div(c, granule) * granule;
    cps_out = c;
    return s > 1 ? ceil_div(N, c) : (int64_t)1;
  };
  int64_t cps = 0;
  S = split_of(S, cps);
  // The sweeps are long and uniform, so the launch runs in rounds of one workgroup per
  // resident slot; a last round that is only partly filled idles the rest of the chip for a
  // whole workgroup's duration. Among split counts between half and twice the one above
  // (keeping the L2 bound), take the one whose workgroups fill their rounds best.
  // resident workgroups per CU (register budgets)
  const int occupancy = mf ? mf_occupancy(op, D, C, p.mf_rt) : 8;
  if ((op == 0 || op == 1 || op == 3) && lead_blocks > 0) {
    const int64_t slots = (int64_t)num_cus * occupancy;
    const int64_t s_min = ceil_div(N, lowd::kSplitCols);
    const int64_t lo = S / 2 > s_min ? S / 2 : s_min;
    const int64_t hi = 2 * S < max_split ? 2 * S : max_split;
    double best = -1.0;
    int64_t best_s = S, best_cps = cps;
    for (int64_t s = lo > 1 ? lo : 1; s <= hi; ++s) {
      int64_t c = 0;
      const int64_t real = split_of(s, c);
      const int64_t total = lead_blocks * real;
      const double fill = (double)total / (double)(ceil_div(total, slots) * slots);
      if (fill > best + 1e-9) {
        best = fill;
        best_s = real;
        best_cps = c;
      }
    }
    S = best_s;
    cps = best_cps;
  }
  // argKmin: every split finds its rows' K smallest keys afresh, so fewer splits queue fewer
  // candidates. Among 1..8 splits (keeping the L2 bound), take the fewest whose workgroups fill
  // their rounds of resident slots to at least 98 % of the best fill (100k x 100k, K = 10: 5
  // splits in one round instead of 11 in three, 3.21 -> 3.01 ms; with few row blocks the fill
  // grows with the split count, so the most splits win).
  if ((op == 2 || op == 6) && p.row_blocks > 0) {
    const int64_t slots = (int64_t)num_cus * knn_occupancy(D, K);
    const int64_t s_min = ceil_div(N, lowd::kSplitCols);
    const int64_t s_max = max_split < 8 ? max_split : 8;
    double fill[9] = {};
    int64_t real[9] = {}, cpss[9] = {};
    double best = -1.0;
    for (int64_t s = 1; s <= s_max; ++s) {
      if (s < s_min) continue;
      real[s] = split_of(s, cpss[s]);
      const int64_t total = p.row_blocks * real[s];
      fill[s] = (double)total / (double)(ceil_div(total, slots) * slots);
      if (fill[s] > best) best = fill[s];
    }
    for (int64_t s = 1; s <= s_max; ++s) {
      if (s < s_min || fill[s] < 0.98 * best) continue;
      S = real[s];
      cps = cpss[s];
      break;
    }
  }
  p.splits = S;
  p.cols_per_split = cps;
  return p;
}

// ------------------------------------------------------------------------- launchers
hipError_t launch_prep_cols(const float* y, double* cols, int64_t N, int D, double c2, bool centre,
                            hipStream_t s) {
  if (N <= 0) return hipSuccess;
  lowd::prep_cols_kernel<<<(unsigned)ceil_div(N, kBlock), kBlock, 0, s>>>(y, cols, N, D, col_stride(D), c2,
                                                                           centre ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_fill(float* out, int64_t n, float value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  lowd::fill_kernel<<<(unsigned)ceil_div(n, kBlock), kBlock, 0, s>>>(out, n, value);
  return hipGetLastError();
}

hipError_t launch_scale_rows(const float* b, const float* scale, float* out, int64_t N, int C, hipStream_t s) {
  const int64_t n = N * C;
  if (n <= 0) return hipSuccess;
  lowd::scale_rows_kernel<<<(unsigned)ceil_div(n, kBlock), kBlock, 0, s>>>(b, scale, out, n, C);
  return hipGetLastError();
}

hipError_t launch_pow(const float* in, float* out, int64_t n, float e, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  lowd::pow_kernel<<<(unsigned)ceil_div(n, kBlock), kBlock, 0, s>>>(in, out, n, e);
  return hipGetLastError();
}

hipError_t launch_div_sqrt(const float* p, const float* d, float* out, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  lowd::div_sqrt_kernel<<<(unsigned)ceil_div(n, kBlock), kBlock, 0, s>>>(p, d, out, n);
  return hipGetLastError();
}

}  // namespace keops
