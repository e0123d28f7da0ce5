// Low-D argKmin ("Kernel matrix reduction", Overview: the indices of the K smallest values
// of a row), alone or fused with the log-sum-exp reduction in the same sweep.
#include "lowd_common.h"

#include <atomic>

namespace keops {
namespace lowd {
namespace {

// Keys are the float64 squared distances ((dx0*dx0 + dx1*dx1) + dx2*dx2) + ... with every
// operation rounded separately (no contraction), dx = (double)x - (double)y. Each lane keeps
// its rows' K best (key, j) sorted ascending; columns arrive in increasing j and a new key
// enters only when strictly smaller, so equal keys keep the lower j first.

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

// Largest |y_j|^2 + |w_j| over the column table (cols[j][D] holds |y_j|^2 on entry; w may be
// null). Each workgroup reduces a grid-strided share and folds it into *out with an atomic
// maximum on the bit patterns (non-negative doubles order like their bits), so the result is
// the exact maximum in any order; *out is cleared by zero_kernel first. With weights the
// table's screening term becomes |y_j|^2 - w_j (each entry is rewritten by the one thread that
// reads it).
__global__ void zero_kernel(double* __restrict__ out) { *out = 0.0; }

__global__ void __launch_bounds__(256)
max_norm_kernel(double* __restrict__ cols, const float* __restrict__ w, int64_t N, int P, int D,
                double* __restrict__ out) {
  __shared__ double red[256];
  double m = 0.0;
  const int64_t step = (int64_t)gridDim.x * 256;
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < N; j += step) {
    const double yy = cols[j * P + D];
    if (w) {
      const double wj = (double)w[j];
      m = fmax(m, yy + fabs(wj));
      cols[j * P + D] = yy - wj;
    } else {
      m = fmax(m, yy);
    }
  }
  red[threadIdx.x] = m;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) red[threadIdx.x] = fmax(red[threadIdx.x], red[threadIdx.x + h]);
    __syncthreads();
  }
  if (threadIdx.x == 0)
    atomicMax(reinterpret_cast<unsigned long long*>(out), (unsigned long long)__double_as_longlong(red[0]));
}

// Screening bound: the float64 expansion a' = (|y|^2 - w) - 2 x.y (D FMAs from the column's
// table entry, each rounded once) is compared with the row's threshold (key_K - |x|^2) + margin,
// key_K the row's current K-th key. With u = 2^-53 and B = |x|^2 + max_j (|y_j|^2 + |w_j|):
// a' differs from d^2 - w - |x|^2 by at most 2D u B (2|x_d y_d| <= x_d^2 + y_d^2), the row
// norm |x|^2 (D FMAs) by D u B, the subtraction key_K - |x|^2 (key_K <= 2B) by 3 u B and the
// added margin by 3 u B: (3D + 6) u B in all, below 2^-46 B for D <= 8 (w = 0 without
// weights).
constexpr double kScreenMargin = 1.4210854715202004e-14;  // 2^-46

// argKmin of d^2_ij - w_j (w_j = 0 when w is null; with LSE, also the log-sum-exp of -c2 d^2 in
// base 2, never combined with weights) over the columns of one split.
// Each pair first gets the cheap expansion a'_ij. A column whose a'_ij is below the row's
// threshold is only queued (its index goes into the lane's queue in LDS); for K <= 16 the
// queueing runs only in tiles where some lane of the wave has such a column (a wave-uniform
// branch), so the common tile costs the D FMAs and one compare per pair. When some lane's queue could overflow,
// every lane of the wave computes the exact keys of its queued columns, in column order, and
// updates its sorted list and threshold. The wave thus runs the list updates once per kQueue
// candidates of its busiest lane instead of once per tile in which any of its 64 lanes has a
// candidate. The threshold a column is screened against may lag behind the list (it is
// refreshed at each flush), which only queues extra columns. For the log-sum-exp the row's
// running shift m (log2 units) is raised lazily, whenever a tile holds a term above
// 2^kLseSlack, so every term 2^(-c2 (|x|^2 + a'_ij) - m) stays below 2^kLseSlack.
constexpr int kQueue = 16;  // queued candidate columns per lane and row

// A pointer into the constant address space: loads through it at a wave-uniform address are
// scalar loads (the data is read-only for the whole launch).
template <typename T>
using ConstPtr = const __attribute__((address_space(4))) T*;

// The value of a wave-uniform 64-bit integer, held in scalar registers.
__device__ __forceinline__ int64_t uniform(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

template <int D, int K, int R, bool LSE>
__global__ void __launch_bounds__(kBlock)
knn_kernel(const float* __restrict__ x, const double* __restrict__ cols, const float* __restrict__ w,
           const double* __restrict__ ymax, int32_t* __restrict__ idx, float* __restrict__ dist, KeyIdx* __restrict__ partial,
           float* __restrict__ lse_out, LsePartial* __restrict__ lse_partial, int64_t M, int64_t N,
           int64_t cps, int Kout, double c2, const int* __restrict__ mf, int run_if_mf) {
  if (mf && mf_admits(mf) != run_if_mf) return;  // the other form takes these inputs
  constexpr int P = (D + 2) & ~1;
  constexpr int U = D <= 4 ? 4 : 2;  // columns per screened tile
  static_assert(kQueue >= 2 * U, "queue holds at least two tiles");
  __shared__ int32_t queue[R][kQueue][kBlock];
  const int64_t split = blockIdx.y;
  const int64_t j0 = split * cps;
  const int64_t j1 = (j0 + cps < N) ? j0 + cps : N;
  const int64_t row0 = (int64_t)blockIdx.x * (kBlock * R) + threadIdx.x;
  const double bmax = *ymax;

  double xd[R][D], xp[R][D], A[R], marg[R], thr[R], off[R];
  double keys[R][K];
  int32_t ids[R][K];
  int cnt[R];
  bool full[R];  // wave-uniform: some lane's queue could overflow on the next tile
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
    cnt[r] = 0;
    full[r] = false;
    mref[r] = -INFINITY;
    off[r] = 0.0;
    l[r] = 0.0f;
  }

  // Exact keys of this lane's queued columns for row r, in queue (= column) order.
  auto flush = [&](int r) {
    for (int e = 0; e < cnt[r]; ++e) {
      const int32_t jj = queue[r][e][threadIdx.x];
      double key = sq_dist_key<D>(xd[r], cols + (int64_t)jj * P);
      if (w) key -= (double)w[jj];
      if (key < keys[r][K - 1]) topk_insert<K>(keys[r], ids[r], key, jj);
    }
    thr[r] = (keys[r][K - 1] - A[r]) + marg[r];
    cnt[r] = 0;
  };

  // Columns [j, j + n) of a tile, n <= U, for row r: screen, queue, add LSE terms.
  auto tile = [&](int r, int64_t j, int n, const double (&yv)[U][D], const double (&bv)[U]) {
    if (full[r]) {
      flush(r);
      full[r] = false;
    }
    double a[U];
    bool hit[U];
    uint64_t hits = 0;  // lanes with a candidate in this tile
#pragma unroll
    for (int u = 0; u < U; ++u) {
      double t = bv[u];
#pragma unroll
      for (int d = 0; d < D; ++d) t = fma(xp[r][d], yv[u][d], t);
      a[u] = t;
      hit[u] = u < n && t < thr[r];
      hits |= __ballot(hit[u]);
    }
    // At K > 16 most tiles hold candidates somewhere in the wave: queue without the test.
    if (K > 16 || __builtin_expect(hits != 0, 0)) {
      // at most kQueue - U entries on entry, so the U writes stay inside the queue
#pragma unroll
      for (int u = 0; u < U; ++u) {
        // written every time, kept only when the count advances
        queue[r][cnt[r]][threadIdx.x] = (int32_t)(j + u);
        cnt[r] += hit[u] ? 1 : 0;
      }
      full[r] = __any(cnt[r] > kQueue - U);
    }
    if constexpr (LSE) {
      double mn = INFINITY;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (u < n) mn = fmin(mn, a[u]);
      const double nm = fma(mn, -c2, -c2 * A[r]);
      if (nm > mref[r] + (double)kLseSlack) {
        l[r] *= exp2_hw((float)(mref[r] - nm));
        mref[r] = nm;
        off[r] = -c2 * A[r] - nm;
      }
      float t = 0.0f;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (u < n) t += exp2_hw((float)fma(a[u], -c2, off[r]));
      l[r] += t;
    }
  };

  // The column records are the same for every lane: with two rows per lane they are read
  // through the scalar unit (at K > 16 the scalar registers they would take are short).
  ConstPtr<double> ccols = (ConstPtr<double>)cols;
  auto col = [&](int64_t e) { return R == 2 ? ccols[e] : cols[e]; };
  const int64_t nfull = (j1 - j0) / U;  // whole tiles of the split
  for (int64_t t = 0; t < nfull; ++t) {
    const int64_t ja = uniform(j0 + t * U);
    double yv[U][D], bv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int d = 0; d < D; ++d) yv[u][d] = col((ja + u) * P + d);
      bv[u] = col((ja + u) * P + D);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) tile(r, ja, U, yv, bv);
  }
  const int64_t j = j0 + nfull * U;
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
  for (int r = 0; r < R; ++r) flush(r);

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

// The sweep(s) and the merges. With mf (the device-side decision of a prepared matrix-core
// log-sum-exp) the fused sweep runs only when that decision declines and the plain one only
// when it admits; the caller runs the matrix-core log-sum-exp itself.
template <int D, int K>
hipError_t knn_dk(const float* x, const double* cols, const float* w, const double* ymax, int32_t* idx, float* dist,
                  void* partial, float* lse_out, double* lse_partial, int64_t M, int64_t N, int Kout, double c2,
                  bool with_lse, const int* mf, const Plan& p, hipStream_t s) {
  constexpr int R = K <= 16 ? 2 : 1;
  dim3 grid((unsigned)p.row_blocks, (unsigned)p.splits);
  KeyIdx* part = reinterpret_cast<KeyIdx*>(partial);
  LsePartial* lpart = reinterpret_cast<LsePartial*>(lse_partial);
  if (with_lse)
    knn_kernel<D, K, R, true><<<grid, kBlock, 0, s>>>(x, cols, w, ymax, idx, dist, part, lse_out, lpart, M, N,
                                                       p.cols_per_split, Kout, c2, mf, 0);
  if (!with_lse || mf)
    knn_kernel<D, K, R, false><<<grid, kBlock, 0, s>>>(x, cols, w, ymax, idx, dist, part, lse_out, lpart, M, N,
                                                        p.cols_per_split, Kout, c2, mf, 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  merge_topk_kernel<K><<<(unsigned)ceil_div(M, kBlock), kBlock, 0, s>>>(part, idx, dist, M, p.splits, Kout);
  e = hipGetLastError();
  if (e != hipSuccess || !with_lse) return e;
  return launch_combine_lse(lpart, lse_out, M, p.splits, s, mf, 0);
}

template <int D>
hipError_t knn_d(int Kb, const float* x, const double* cols, const float* w, const double* ymax, int32_t* idx, float* dist,
                 void* partial, float* lse_out, double* lse_partial, int64_t M, int64_t N, int Kout, double c2,
                 bool with_lse, const int* mf, const Plan& p, hipStream_t s) {
#define KEOPS_KNN_K(Kv) return knn_dk<D, Kv>(x, cols, w, ymax, idx, dist, partial, lse_out, lse_partial, M, N, Kout, c2, with_lse, mf, p, s)
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

// Resident workgroups per CU of the plain sweep: the runtime's figure, but with the LDS queues
// strictly inside the CU's LDS (workgroups whose queues would fill it exactly, 5 x 32 KB of
// 160 KB, measured as 4 resident).
template <int D, int K>
int occupancy_dk(int dev) {
  constexpr int R = K <= 16 ? 2 : 1;
  auto kernel = knn_kernel<D, K, R, false>;
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kBlock, 0) != hipSuccess || n < 1) return 1;
  hipFuncAttributes attr;
  int lds_cu = 0;
  if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(kernel)) == hipSuccess && attr.sharedSizeBytes > 0 &&
      hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) == hipSuccess &&
      lds_cu > 0) {
    const int fit = (int)((lds_cu - 1) / (int)attr.sharedSizeBytes);
    if (fit < n) n = fit > 0 ? fit : 1;
  }
  return n;
}

template <int D>
int occupancy_d(int Kb, int dev) {
  switch (Kb) {
    case 1: return occupancy_dk<D, 1>(dev);
    case 2: return occupancy_dk<D, 2>(dev);
    case 4: return occupancy_dk<D, 4>(dev);
    case 8: return occupancy_dk<D, 8>(dev);
    case 10: return occupancy_dk<D, 10>(dev);
    case 16: return occupancy_dk<D, 16>(dev);
    case 32: return occupancy_dk<D, 32>(dev);
    case 64: return occupancy_dk<D, 64>(dev);
  }
  return 1;
}

}  // namespace
}  // namespace lowd

int knn_occupancy(int D, int K) {
  // resident workgroups per CU of the plain argKmin sweep (cached per instance; 1 when the
  // runtime cannot say)
  static std::atomic<int> cache[kMaxLowD + 1][8];
  int dev = 0;
  if (D < 1 || D > kMaxLowD || K < 1 || hipGetDevice(&dev) != hipSuccess) return 1;
  static const int kBuckets[8] = {1, 2, 4, 8, 10, 16, 32, 64};
  const int Kb = lowd::argk_bucket(K);
  int kslot = 0;
  while (kBuckets[kslot] != Kb) ++kslot;
  std::atomic<int>& slot = cache[D][kslot];
  int n = slot.load(std::memory_order_relaxed);
  if (n > 0) return n;
  switch (D) {
    case 1: n = lowd::occupancy_d<1>(Kb, dev); break;
    case 2: n = lowd::occupancy_d<2>(Kb, dev); break;
    case 3: n = lowd::occupancy_d<3>(Kb, dev); break;
    case 4: n = lowd::occupancy_d<4>(Kb, dev); break;
    case 5: n = lowd::occupancy_d<5>(Kb, dev); break;
    case 6: n = lowd::occupancy_d<6>(Kb, dev); break;
    case 7: n = lowd::occupancy_d<7>(Kb, dev); break;
    case 8: n = lowd::occupancy_d<8>(Kb, dev); break;
  }
  slot.store(n, std::memory_order_relaxed);
  return n;
}

hipError_t launch_knn_lowd(const float* x, const float* y, const float* w, double* cols, double* ymax,
                           int32_t* idx, float* dist, void* partial, float* lse_out, double* lse_partial, int64_t M,
                           int64_t N, int D, int K, double c2, bool with_lse, const Plan& p, hipStream_t s,
                           const KnnLse* mf_lse) {
  // column table (y_j, |y_j|^2 - w_j) uncentred, then the largest |y_j|^2 + |w_j| for the
  // screening margin
  hipError_t e = launch_prep_cols(y, cols, N, D, -1.0, false, s);
  if (e != hipSuccess) return e;
  lowd::zero_kernel<<<1, 1, 0, s>>>(ymax);
  const int64_t nb = lowd::ceil_div(N, 256);
  lowd::max_norm_kernel<<<(unsigned)(nb < 512 ? nb : 512), 256, 0, s>>>(cols, w, N, col_stride(D), D, ymax);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int Kb = lowd::argk_bucket(K);
  // With the log-sum-exp and a matrix-core region: the matrix-core log-sum-exp sweep and the
  // plain argKmin sweep when the device-side decision admits the inputs (the two sweeps cost
  // less than the fused one on this chip), the fused float64 sweep otherwise.
  const int* mf = nullptr;
  if (with_lse && mf_lse && !w) {
    e = launch_mf_prepare(x, y, nullptr, false, nullptr, mf_lse->region, M, N, D, 0, c2, s);
    if (e != hipSuccess) return e;
    mf = mf_decision(mf_lse->region);
  }
#define KEOPS_KNN(Dv) lowd::knn_d<Dv>(Kb, x, cols, w, ymax, idx, dist, partial, lse_out, lse_partial, M, N, K, c2, with_lse, mf, p, s)
  auto run = [&]() -> hipError_t { KEOPS_SWITCH_D(D, KEOPS_KNN) };
#undef KEOPS_KNN
  e = run();
  if (e != hipSuccess || !mf) return e;
  const Plan& lp = *mf_lse->plan;
  e = launch_mf_lse(lse_out, lp.splits > 1 ? mf_lse->partial : nullptr, mf_lse->region, M, N, D, lp, s);
  if (e != hipSuccess || lp.splits == 1) return e;
  return lowd::launch_combine_lse(static_cast<const lowd::LsePartial*>(mf_lse->partial), lse_out, M, lp.splits, s,
                                  mf, 1);
}

}  // namespace keops
