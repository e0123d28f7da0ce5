// Low-dimensional (D <= 8) float32 reductions for gfx950.
//
// Every kernel streams the column set j through wave-uniform loads (the column record of j
// is the same for all 64 lanes, so it lands in scalar registers) while each lane keeps R
// rows i in vector registers for the whole sweep; the M-by-N table never exists.
//
// Gaussian exponent. For the sum and log-sum-exp reductions the exponent in base 2,
//   e_ij = -c2 ||x_i - y_j||^2,  c2 = log2(e) / (2 sigma^2),
// is evaluated in float64 from centred coordinates u_i = x_i - o, v_j = y_j - o (o = y_0):
//   e_ij = A_i + B_j + sum_d (2 c2 u_id) v_jd,  A_i = -c2 |u_i|^2,  B_j = -c2 |v_j|^2,
// i.e. one add and D fused multiply-adds per pair at full float64 VALU rate (the same
// issue rate as unpacked float32 on this chip). float64 keeps the cancellation between the
// large terms below 1e-11 in e for inputs within 1e4 sigma of one another, far more exact
// than a float32 difference would be; e is then rounded to float32 for v_exp_f32.
#include "internal.h"

#include <math.h>

namespace keops {
namespace {

__device__ __forceinline__ float exp2_hw(float v) { return __builtin_amdgcn_exp2f(v); }

constexpr int kChunk = 512;            // columns per first-level partial sum
constexpr float kLseSlack = 16.0f;     // lazy rescale: terms may grow to 2^16 before a rescale

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

// ------------------------------------------------------------------------- Gauss sum
// out[i][c] = sum_j 2^{e_ij} b[j][c] over the columns [j0, j1) of this split. With one split
// `out` is the final output, otherwise partial[split][i][c].
template <int D, int C, int R>
__global__ void __launch_bounds__(kBlock)
gauss_sum_kernel(const float* __restrict__ x, const float* __restrict__ y,
                 const double* __restrict__ cols, const float* __restrict__ b,
                 float* __restrict__ out, int64_t M, int64_t N, int64_t cps, double c2) {
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
#pragma unroll
      for (int c = 0; c < C; ++c) dst[i * C + c] = acc[r][c];
    }
  }
}

// out[i] = sum over s of partial[s][i], in increasing s.
__global__ void __launch_bounds__(kBlock)
combine_sum_kernel(const float* __restrict__ partial, float* __restrict__ out, int64_t n, int64_t S) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  for (int64_t k = 0; k < S; ++k) s += partial[k * n + i];
  out[i] = s;
}

// ------------------------------------------------------------------------ log-sum-exp
// Per row a running shift m (float64, log2 units) and l = sum_j 2^{e_ij - m}. The shift is
// raised only when a tile holds a term above 2^kLseSlack, so rescales are rare.
struct LsePartial {
  double m;
  float l;
  float pad;
};

template <int D, int R, int U>
__global__ void __launch_bounds__(kBlock)
lse_kernel(const float* __restrict__ x, const float* __restrict__ y,
           const double* __restrict__ cols, float* __restrict__ out,
           LsePartial* __restrict__ partial, int64_t M, int64_t N, int64_t cps, double c2) {
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
#pragma unroll
        for (int u = 0; u < U; ++u) e32[r][u] -= tmax;
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
        e32 = 0.0f;
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

__global__ void __launch_bounds__(kBlock)
combine_lse_kernel(const LsePartial* __restrict__ partial, float* __restrict__ out, int64_t M,
                   int64_t S) {
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

// ---------------------------------------------------------------------------- argKmin
// Keys are the float64 squared distances ((dx0*dx0 + dx1*dx1) + dx2*dx2) + ... with every
// operation rounded separately (no contraction), dx = (double)x - (double)y. Each lane keeps
// its rows' K best (key, j) sorted ascending; columns arrive in increasing j and a new key
// enters only when strictly smaller, so equal keys keep the lower j first.
struct KeyIdx {
  double key;
  int32_t idx;
  int32_t pad;
};

template <int K>
__device__ __forceinline__ void topk_insert(double (&keys)[K], int32_t (&ids)[K], double key, int32_t j) {
#pragma unroll
  for (int k = K - 1; k > 0; --k) {
    const bool before_prev = key < keys[k - 1];
    const bool before_this = key < keys[k];
    const double nk = before_prev ? keys[k - 1] : (before_this ? key : keys[k]);
    const int32_t ni = before_prev ? ids[k - 1] : (before_this ? j : ids[k]);
    keys[k] = nk;
    ids[k] = ni;
  }
  if (key < keys[0]) {
    keys[0] = key;
    ids[0] = j;
  }
}

template <int D>
__device__ __forceinline__ double sq_dist_key(const double (&xu)[D], const double* v) {
#pragma clang fp contract(off)
  double key = 0.0;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const double dd = xu[d] - v[d];
    const double sq = dd * dd;
    key = (d == 0) ? sq : key + sq;
  }
  return key;
}

// Largest squared norm in the column table (cols[j][D] holds |y_j|^2), one workgroup, fixed
// reduction order.
__global__ void __launch_bounds__(1024)
max_norm_kernel(const double* __restrict__ cols, int64_t N, int P, int D, double* __restrict__ out) {
  __shared__ double red[1024];
  double m = 0.0;
  for (int64_t j = threadIdx.x; j < N; j += 1024) m = fmax(m, cols[j * P + D]);
  red[threadIdx.x] = m;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + w]);
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = red[0];
}

// Screening bound: the float64 expansion a = |x|^2 + |y|^2 - 2 x.y (D+1 FMAs after the two
// norms, each rounded once) differs from the exact squared distance by at most
// (4D + 8) 2^-53 (|x|^2 + |y|^2) <= 2^-46 (|x|^2 + max_j |y_j|^2) for D <= 8.
constexpr double kScreenMargin = 1.4210854715202004e-14;  // 2^-46

// argKmin (and, with LSE, the log-sum-exp of -c2 d^2 in base 2) over the columns of one split.
// Each pair first gets the cheap expansion a_ij; only when a_ij is below the row's K-th key
// plus the margin is the exact key computed and the sorted list updated, which after the
// first columns is rare. For the log-sum-exp the row's running shift is -c2 times its
// smallest key so far, raised lazily (only when it grows by more than kLseSlack), so every
// term 2^(-c2 a_ij - m) stays below 2^kLseSlack; it is updated before a tile's terms are added.
template <int D, int K, int R, bool LSE>
__global__ void __launch_bounds__(kBlock)
knn_kernel(const float* __restrict__ x, const double* __restrict__ cols, const double* __restrict__ ymax,
           int32_t* __restrict__ idx, float* __restrict__ dist, KeyIdx* __restrict__ partial,
           float* __restrict__ lse_out, LsePartial* __restrict__ lse_partial, int64_t M, int64_t N,
           int64_t cps, int Kout, double c2) {
  constexpr int P = (D + 2) & ~1;
  constexpr int U = D <= 4 ? 4 : 2;  // columns per screened tile
  const int64_t split = blockIdx.y;
  const int64_t j0 = split * cps;
  const int64_t j1 = (j0 + cps < N) ? j0 + cps : N;
  const int64_t row0 = (int64_t)blockIdx.x * (kBlock * R) + threadIdx.x;
  const double bmax = *ymax;

  double xd[R][D], xp[R][D], A[R], marg[R], thr[R];
  double keys[R][K];
  int32_t ids[R][K];
  double mref[R];
  float l[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int64_t i = row0 + (int64_t)r * kBlock;
    i = i < M ? i : M - 1;
    double s = 0.0;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      xd[r][d] = (double)x[i * D + d];
      xp[r][d] = -2.0 * xd[r][d];
      s = fma(xd[r][d], xd[r][d], s);
    }
    A[r] = s;
    marg[r] = kScreenMargin * (s + bmax);
    thr[r] = INFINITY;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      keys[r][k] = INFINITY;
      ids[r][k] = -1;
    }
    mref[r] = -INFINITY;
    l[r] = 0.0f;
  }

  // Columns [j, j + n) of a tile, n <= U, for row r: screen, update the list, add LSE terms.
  auto tile = [&](int r, int64_t j, int n, const double (&yv)[U][D], const double (&bv)[U]) {
    double a[U];
    double mn = INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u < n) {
        double t = A[r] + bv[u];
#pragma unroll
        for (int d = 0; d < D; ++d) t = fma(xp[r][d], yv[u][d], t);
        a[u] = t;
        mn = fmin(mn, t);
      }
    }
    if (mn < thr[r]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (u < n && a[u] < thr[r]) {
          const double key = sq_dist_key<D>(xd[r], yv[u]);
          if (key < keys[r][K - 1]) {
            topk_insert<K>(keys[r], ids[r], key, (int32_t)(j + u));
            thr[r] = keys[r][K - 1] + marg[r];
            if constexpr (LSE) {
              const double nm = -c2 * keys[r][0];
              if (nm > mref[r] + (double)kLseSlack) {
                l[r] *= exp2_hw((float)(mref[r] - nm));
                mref[r] = nm;
              }
            }
          }
        }
      }
    }
    if constexpr (LSE) {
      float t = 0.0f;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (u < n) t += exp2_hw((float)fma(a[u], -c2, -mref[r]));
      l[r] += t;
    }
  };

  int64_t j = j0;
  for (; j + U <= j1; j += U) {
    double yv[U][D], bv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int d = 0; d < D; ++d) yv[u][d] = cols[(j + u) * P + d];
      bv[u] = cols[(j + u) * P + D];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) tile(r, j, U, yv, bv);
  }
  if (j < j1) {
    const int n = (int)(j1 - j);
    double yv[U][D], bv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t jj = (u < n) ? j + u : j;
#pragma unroll
      for (int d = 0; d < D; ++d) yv[u][d] = cols[jj * P + d];
      bv[u] = cols[jj * P + D];
    }
#pragma unroll
    for (int r = 0; r < R; ++r) tile(r, j, n, yv, bv);
  }

#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t i = row0 + (int64_t)r * kBlock;
    if (i >= M) continue;
    if (gridDim.y == 1) {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        if (k < Kout) {
          idx[i * Kout + k] = ids[r][k];
          if (dist) dist[i * Kout + k] = (float)keys[r][k];
        }
      }
      if constexpr (LSE) lse_out[i] = (float)((mref[r] + (double)log2f(l[r])) * M_LN2);
    } else {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        KeyIdx p;
        p.key = keys[r][k];
        p.idx = ids[r][k];
        p.pad = 0;
        partial[(split * M + i) * K + k] = p;
      }
      if constexpr (LSE) {
        LsePartial p;
        p.m = mref[r];
        p.l = l[r];
        p.pad = 0.0f;
        lse_partial[split * M + i] = p;
      }
    }
  }
}

// Merge the S per-split lists of row i in increasing split order (lower columns first), so
// equal keys keep the lower column index first.
template <int K>
__global__ void __launch_bounds__(kBlock)
merge_topk_kernel(const KeyIdx* __restrict__ partial, int32_t* __restrict__ idx,
                  float* __restrict__ dist, int64_t M, int64_t S, int Kout) {
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i >= M) return;
  double keys[K];
  int32_t ids[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    keys[k] = INFINITY;
    ids[k] = -1;
  }
  for (int64_t s = 0; s < S; ++s) {
    const KeyIdx* p = partial + (s * M + i) * K;
    for (int k = 0; k < K; ++k) {
      const KeyIdx q = p[k];
      if (q.idx < 0) break;
      if (q.key < keys[K - 1]) topk_insert<K>(keys, ids, q.key, q.idx);
      else break;  // the split's list is sorted: nothing later can enter
    }
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    if (k < Kout) {
      idx[i * Kout + k] = ids[k];
      if (dist) dist[i * Kout + k] = (float)keys[k];
    }
  }
}

// ---------------------------------------------------------------------- gradient wrt x
// grad_i = -(1/sigma^2) sum_j k_ij (g_i . b_j) (x_i - y_j), with the differences taken
// first in float32 (they are reused for d^2 and for the accumulation).
template <int D, int C, int R>
__global__ void __launch_bounds__(kBlock)
grad_x_kernel(const float* __restrict__ x, const float* __restrict__ y, const float* __restrict__ b,
              const float* __restrict__ g, float* __restrict__ out, int64_t M, int64_t N,
              int64_t cps, float c2f, float inv_sigma2) {
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

// ----------------------------------------------------------------- template dispatch
constexpr int kRowsSum = 4;
constexpr int kRowsLse = 4;
constexpr int kRowsGrad = 2;
constexpr int kLseTile = 8;
constexpr int64_t kSplitCols = 65536;

inline int argk_bucket(int K) {
  if (K <= 1) return 1;
  if (K <= 2) return 2;
  if (K <= 4) return 4;
  if (K <= 8) return 8;
  if (K <= 10) return 10;
  if (K <= 16) return 16;
  if (K <= 32) return 32;
  return 64;
}
inline int argk_rows(int Kb) { return Kb <= 16 ? 2 : 1; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

template <int D, int C>
hipError_t gauss_sum_dc(const float* x, const float* y, const double* cols, const float* b,
                        float* dst, int64_t M, int64_t N, double c2, const Plan& p, hipStream_t s) {
  dim3 grid((unsigned)p.row_blocks, (unsigned)p.splits);
  gauss_sum_kernel<D, C, kRowsSum><<<grid, kBlock, 0, s>>>(x, y, cols, b, dst, M, N, p.cols_per_split, c2);
  return hipGetLastError();
}

template <int D>
hipError_t gauss_sum_d(int C, const float* x, const float* y, const double* cols, const float* b,
                       float* dst, int64_t M, int64_t N, double c2, const Plan& p, hipStream_t s) {
  switch (C) {
    case 1: return gauss_sum_dc<D, 1>(x, y, cols, b, dst, M, N, c2, p, s);
    case 2: return gauss_sum_dc<D, 2>(x, y, cols, b, dst, M, N, c2, p, s);
    case 3: return gauss_sum_dc<D, 3>(x, y, cols, b, dst, M, N, c2, p, s);
    case 4: return gauss_sum_dc<D, 4>(x, y, cols, b, dst, M, N, c2, p, s);
    case 5: return gauss_sum_dc<D, 5>(x, y, cols, b, dst, M, N, c2, p, s);
    case 6: return gauss_sum_dc<D, 6>(x, y, cols, b, dst, M, N, c2, p, s);
    case 7: return gauss_sum_dc<D, 7>(x, y, cols, b, dst, M, N, c2, p, s);
    case 8: return gauss_sum_dc<D, 8>(x, y, cols, b, dst, M, N, c2, p, s);
  }
  return hipErrorInvalidValue;
}

template <int D, int C>
hipError_t grad_dc(const float* x, const float* y, const float* b, const float* g, float* dst,
                   int64_t M, int64_t N, float c2f, float inv_sigma2, const Plan& p, hipStream_t s) {
  dim3 grid((unsigned)p.row_blocks, (unsigned)p.splits);
  grad_x_kernel<D, C, kRowsGrad><<<grid, kBlock, 0, s>>>(x, y, b, g, dst, M, N, p.cols_per_split, c2f, inv_sigma2);
  return hipGetLastError();
}

template <int D>
hipError_t grad_d(int C, const float* x, const float* y, const float* b, const float* g, float* dst,
                  int64_t M, int64_t N, float c2f, float inv_sigma2, const Plan& p, hipStream_t s) {
  switch (C) {
    case 1: return grad_dc<D, 1>(x, y, b, g, dst, M, N, c2f, inv_sigma2, p, s);
    case 2: return grad_dc<D, 2>(x, y, b, g, dst, M, N, c2f, inv_sigma2, p, s);
    case 3: return grad_dc<D, 3>(x, y, b, g, dst, M, N, c2f, inv_sigma2, p, s);
    case 4: return grad_dc<D, 4>(x, y, b, g, dst, M, N, c2f, inv_sigma2, p, s);
    case 5: return grad_dc<D, 5>(x, y, b, g, dst, M, N, c2f, inv_sigma2, p, s);
    case 6: return grad_dc<D, 6>(x, y, b, g, dst, M, N, c2f, inv_sigma2, p, s);
    case 7: return grad_dc<D, 7>(x, y, b, g, dst, M, N, c2f, inv_sigma2, p, s);
    case 8: return grad_dc<D, 8>(x, y, b, g, dst, M, N, c2f, inv_sigma2, p, s);
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t lse_d(const float* x, const float* y, const double* cols, float* out, double* partial,
                 int64_t M, int64_t N, double c2, const Plan& p, hipStream_t s) {
  dim3 grid((unsigned)p.row_blocks, (unsigned)p.splits);
  lse_kernel<D, kRowsLse, kLseTile><<<grid, kBlock, 0, s>>>(
      x, y, cols, out, reinterpret_cast<LsePartial*>(partial), M, N, p.cols_per_split, c2);
  return hipGetLastError();
}

template <int D, int K, bool LSE>
hipError_t knn_dk(const float* x, const double* cols, const double* ymax, int32_t* idx, float* dist,
                  void* partial, float* lse_out, double* lse_partial, int64_t M, int64_t N, int Kout, double c2,
                  const Plan& p, hipStream_t s) {
  dim3 grid((unsigned)p.row_blocks, (unsigned)p.splits);
  knn_kernel<D, K, (K <= 16 ? 2 : 1), LSE><<<grid, kBlock, 0, s>>>(
      x, cols, ymax, idx, dist, reinterpret_cast<KeyIdx*>(partial), lse_out,
      reinterpret_cast<LsePartial*>(lse_partial), M, N, p.cols_per_split, Kout, c2);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  merge_topk_kernel<K><<<(unsigned)ceil_div(M, kBlock), kBlock, 0, s>>>(
      reinterpret_cast<const KeyIdx*>(partial), idx, dist, M, p.splits, Kout);
  e = hipGetLastError();
  if (e != hipSuccess || !LSE) return e;
  combine_lse_kernel<<<(unsigned)ceil_div(M, kBlock), kBlock, 0, s>>>(
      reinterpret_cast<const LsePartial*>(lse_partial), lse_out, M, p.splits);
  return hipGetLastError();
}

template <int D, bool LSE>
hipError_t knn_d(int Kb, const float* x, const double* cols, const double* ymax, int32_t* idx, float* dist,
                 void* partial, float* lse_out, double* lse_partial, int64_t M, int64_t N, int Kout, double c2,
                 const Plan& p, hipStream_t s) {
#define KEOPS_KNN_K(Kv) return knn_dk<D, Kv, LSE>(x, cols, ymax, idx, dist, partial, lse_out, lse_partial, M, N, Kout, c2, p, s)
  switch (Kb) {
    case 1: KEOPS_KNN_K(1);
    case 2: KEOPS_KNN_K(2);
    case 4: KEOPS_KNN_K(4);
    case 8: KEOPS_KNN_K(8);
    case 10: KEOPS_KNN_K(10);
    case 16: KEOPS_KNN_K(16);
    case 32: KEOPS_KNN_K(32);
    case 64: KEOPS_KNN_K(64);
  }
#undef KEOPS_KNN_K
  return hipErrorInvalidValue;
}

#define KEOPS_SWITCH_D(D_, CALL)                   \
  switch (D_) {                                    \
    case 1: return CALL(1);                        \
    case 2: return CALL(2);                        \
    case 3: return CALL(3);                        \
    case 4: return CALL(4);                        \
    case 5: return CALL(5);                        \
    case 6: return CALL(6);                        \
    case 7: return CALL(7);                        \
    case 8: return CALL(8);                        \
  }                                                \
  return hipErrorInvalidValue;

}  // namespace

// ------------------------------------------------------------------------- planning
size_t partial_bytes_per_row(int op, int D, int C, int K) {
  switch (op) {
    case 0: return sizeof(float) * (size_t)C;
    case 1: return sizeof(LsePartial);
    case 2: return sizeof(KeyIdx) * (size_t)argk_bucket(K);
    case 6: return sizeof(KeyIdx) * (size_t)argk_bucket(K) + sizeof(LsePartial);
    case 3: return sizeof(float) * (size_t)D;
  }
  return 0;
}

Plan plan_lowd(int op, int64_t M, int64_t N, int D, int C, int K, int num_cus) {
  (void)D;
  (void)C;
  Plan p;
  switch (op) {
    case 0: p.R = kRowsSum; break;
    case 1: p.R = kRowsLse; break;
    case 2:
    case 6: p.R = argk_rows(argk_bucket(K)); break;
    default: p.R = kRowsGrad; break;
  }
  p.rows_per_block = kBlock * p.R;
  p.row_blocks = M > 0 ? ceil_div(M, p.rows_per_block) : 0;
  // Split the columns so that (a) there are at least eight workgroups (32 wave64s) per compute
  // unit over the launch, and (b) one split's column table stays within kSplitCols columns,
  // a working set that fits one XCD's L2 while the resident workgroups (consecutive row
  // blocks of the same split) stream it together. Every split keeps >= 256 columns.
  const int64_t target = (int64_t)num_cus * 8;
  int64_t S = 1;
  if (p.row_blocks > 0 && p.row_blocks < target) S = ceil_div(target, p.row_blocks);
  if (S < ceil_div(N, kSplitCols)) S = ceil_div(N, kSplitCols);
  int64_t max_split = N / 256 > 1 ? N / 256 : 1;
  if ((op == 2 || op == 6) && max_split > 16) max_split = 16;  // argKmin partial lists are K entries per row
  if (S > max_split) S = max_split;
  if (S < 1) S = 1;
  int64_t cps = S > 1 ? ceil_div(N, S) : (N > 0 ? N : 1);
  cps = ceil_div(cps, 8) * 8;
  if (S > 1) S = ceil_div(N, cps);
  p.splits = S;
  p.cols_per_split = cps;
  return p;
}

// ------------------------------------------------------------------------- launchers
hipError_t launch_prep_cols(const float* y, double* cols, int64_t N, int D, double c2, bool centre,
                            hipStream_t s) {
  if (N <= 0) return hipSuccess;
  prep_cols_kernel<<<(unsigned)ceil_div(N, kBlock), kBlock, 0, s>>>(y, cols, N, D, col_stride(D), c2,
                                                                     centre ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_fill(float* out, int64_t n, float value, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  fill_kernel<<<(unsigned)ceil_div(n, kBlock), kBlock, 0, s>>>(out, n, value);
  return hipGetLastError();
}

hipError_t launch_gauss_sum_lowd(const float* x, const float* y, const double* cols, const float* b,
                                 float* out, float* partial, int64_t M, int64_t N, int D, int C,
                                 double c2, const Plan& p, hipStream_t s) {
  float* dst = p.splits > 1 ? partial : out;
  hipError_t e;
  {
#define KEOPS_GS(Dv) gauss_sum_d<Dv>(C, x, y, cols, b, dst, M, N, c2, p, s)
    auto run = [&]() -> hipError_t { KEOPS_SWITCH_D(D, KEOPS_GS) };
#undef KEOPS_GS
    e = run();
  }
  if (e != hipSuccess || p.splits == 1) return e;
  const int64_t n = M * C;
  combine_sum_kernel<<<(unsigned)ceil_div(n, kBlock), kBlock, 0, s>>>(partial, out, n, p.splits);
  return hipGetLastError();
}

hipError_t launch_lse_lowd(const float* x, const float* y, const double* cols, float* out, double* partial,
                           int64_t M, int64_t N, int D, double c2, const Plan& p, hipStream_t s) {
  hipError_t e;
  {
#define KEOPS_LSE(Dv) lse_d<Dv>(x, y, cols, out, partial, M, N, c2, p, s)
    auto run = [&]() -> hipError_t { KEOPS_SWITCH_D(D, KEOPS_LSE) };
#undef KEOPS_LSE
    e = run();
  }
  if (e != hipSuccess || p.splits == 1) return e;
  combine_lse_kernel<<<(unsigned)ceil_div(M, kBlock), kBlock, 0, s>>>(
      reinterpret_cast<const LsePartial*>(partial), out, M, p.splits);
  return hipGetLastError();
}

hipError_t launch_knn_lowd(const float* x, const float* y, double* cols, double* ymax, int32_t* idx,
                           float* dist, void* partial, float* lse_out, double* lse_partial, int64_t M, int64_t N,
                           int D, int K, double c2, bool with_lse, const Plan& p, hipStream_t s) {
  // column table (y_j, |y_j|^2) uncentred, then its largest norm for the screening margin
  hipError_t e = launch_prep_cols(y, cols, N, D, -1.0, false, s);
  if (e != hipSuccess) return e;
  max_norm_kernel<<<1, 1024, 0, s>>>(cols, N, col_stride(D), D, ymax);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int Kb = argk_bucket(K);
  if (with_lse) {
#define KEOPS_KNN(Dv) knn_d<Dv, true>(Kb, x, cols, ymax, idx, dist, partial, lse_out, lse_partial, M, N, K, c2, p, s)
    auto run = [&]() -> hipError_t { KEOPS_SWITCH_D(D, KEOPS_KNN) };
#undef KEOPS_KNN
    return run();
  }
#define KEOPS_KNN(Dv) knn_d<Dv, false>(Kb, x, cols, ymax, idx, dist, partial, lse_out, lse_partial, M, N, K, c2, p, s)
  auto run = [&]() -> hipError_t { KEOPS_SWITCH_D(D, KEOPS_KNN) };
#undef KEOPS_KNN
  return run();
}

hipError_t launch_grad_x_lowd(const float* x, const float* y, const float* b, const float* g, float* grad,
                              float* partial, int64_t M, int64_t N, int D, int C, float c2f,
                              float inv_sigma2, const Plan& p, hipStream_t s) {
  float* dst = p.splits > 1 ? partial : grad;
  hipError_t e;
  {
#define KEOPS_GR(Dv) grad_d<Dv>(C, x, y, b, g, dst, M, N, c2f, inv_sigma2, p, s)
    auto run = [&]() -> hipError_t { KEOPS_SWITCH_D(D, KEOPS_GR) };
#undef KEOPS_GR
    e = run();
  }
  if (e != hipSuccess || p.splits == 1) return e;
  const int64_t n = M * D;
  combine_sum_kernel<<<(unsigned)ceil_div(n, kBlock), kBlock, 0, s>>>(partial, grad, n, p.splits);
  return hipGetLastError();
}

}  // namespace keops
