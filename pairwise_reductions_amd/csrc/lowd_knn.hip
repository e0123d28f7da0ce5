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
// reads it). The same pass writes the float32 screening table scr[j] = (y_j, |y_j|^2 - w_j
// rounded to float32, zeros) with records of S32 floats, followed by kScreenPad records (0, +inf)
// that no row can take (tiles running past the last column read them).
__global__ void zero_kernel(double* __restrict__ out) { *out = 0.0; }

constexpr int kScreenPad = 16;  // records after the last column (a sweep reads up to 3 tiles past it)

__global__ void __launch_bounds__(256)
max_norm_kernel(double* __restrict__ cols, const float* __restrict__ w, int64_t N, int P, int D,
                float* __restrict__ scr, int S32, double* __restrict__ out) {
  __shared__ double red[256];
  double m = 0.0;
  const int64_t step = (int64_t)gridDim.x * 256;
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < N; j += step) {
    double yy = cols[j * P + D];
    if (w) {
      const double wj = (double)w[j];
      m = fmax(m, yy + fabs(wj));
      yy -= wj;
      cols[j * P + D] = yy;
    } else {
      m = fmax(m, yy);
    }
    for (int d = 0; d < D; ++d) scr[j * S32 + d] = (float)cols[j * P + d];
    scr[j * S32 + D] = (float)yy;
    for (int d = D + 1; d < S32; ++d) scr[j * S32 + d] = 0.0f;
  }
  if (blockIdx.x == 0 && (int)threadIdx.x < kScreenPad * S32) {
    const int d = (int)threadIdx.x % S32;
    scr[N * S32 + threadIdx.x] = (d == D) ? INFINITY : 0.0f;
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

// The plain sweep (no log-sum-exp) screens in float32 instead: a32 = fl(t_j + sum_d (-2 x_d) y_d)
// with t_j = |y_j|^2 - w_j rounded to float32 (|t_j| <= max_j(|y_j|^2 + |w_j|)) and one rounding
// per FMA (-2 x_d and y_d are exact float32 values). Every partial sum is at most
// |t_j| + 2 sum_d |x_d y_d| <= 2B with B = |x|^2 + max_j(|y_j|^2 + |w_j|), so a32 differs from
// the exact d^2 - w - |x|^2 by at most (2D + 1) 2^-24 B; the float64 threshold (key_K - |x|^2)
// is rounded up to float32, and 2^-19 B covers both for D <= 8. The float32 FMA issues about
// 1.6 times as fast as the float64 one on this chip.
constexpr double kScreenMargin32 = 0x1p-19;
// Floats per record of the float32 screening table: D coordinates and the column term, rounded
// up to a multiple of 4 (whole 16-byte chunks for the vector loads and LDS reads).
__host__ __device__ constexpr int screen_stride(int D) { return (D + 1 + 3) & ~3; }

// The smallest float32 value >= v (v finite or +inf): the rounded value, moved one step up
// (one unit in its bit pattern) when rounding went down.
__device__ __forceinline__ float round_up_f32(double v) {
  const float f = (float)v;
  if (!((double)f < v)) return f;
  if (f == 0.0f) return __int_as_float(1);
  const int b = __float_as_int(f);
  return __int_as_float(f > 0.0f ? b + 1 : b - 1);
}

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

// Rows in spatial order. A wave takes 128 rows; when they lie close together their candidate
// columns are mostly the same, so far fewer tiles hold a candidate for some lane of the wave
// than with rows in input order (each row's result does not depend on which lane computes it).
// The order is a counting sort of the rows by the Morton code of their cell on a 2^15-cell grid
// over the bounding box of rows and columns together (5 bits per dimension over the first
// three dimensions; 15 bits for D = 1, 7 per dimension for D = 2); rows within one cell keep an
// arbitrary order. The columns are sorted the same way, for the starting thresholds below.
constexpr int kOrderBits = 15;
constexpr int kOrderCells = 1 << kOrderBits;

__device__ __forceinline__ unsigned int ord_of_f(float f) {
  const unsigned int u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f_of_ord(unsigned int u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// box[0..2] = per-dimension minima, box[3..5] maxima (order-preserving encodings; cleared to
// 0xffffffff / 0 first), both cell-count tables (rows, columns) = 0.
__global__ void __launch_bounds__(256)
order_clear_kernel(unsigned int* __restrict__ box, unsigned int* __restrict__ counts, unsigned int* __restrict__ ccounts) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t < kOrderCells) {
    counts[t] = 0u;
    ccounts[t] = 0u;
  }
  if (t < 3) box[t] = 0xffffffffu;
  else if (t < 6) box[t] = 0u;
}

// One pass over the rows and the columns; each workgroup reduces its share in LDS and folds it
// in with one atomic minimum / maximum per dimension.
__global__ void __launch_bounds__(256)
order_box_kernel(const float* __restrict__ x, int64_t M, const float* __restrict__ y, int64_t N, int D,
                 unsigned int* __restrict__ box) {
  __shared__ unsigned int red[2][3][4];
  const int nd = D < 3 ? D : 3;
  unsigned int lo[3] = {0xffffffffu, 0xffffffffu, 0xffffffffu}, hi[3] = {0u, 0u, 0u};
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < M + N; i += stride) {
    const float* p = i < M ? x + i * D : y + (i - M) * D;
    for (int d = 0; d < nd; ++d) {
      const unsigned int v = ord_of_f(p[d]);
      lo[d] = v < lo[d] ? v : lo[d];
      hi[d] = v > hi[d] ? v : hi[d];
    }
  }
  const int wave = threadIdx.x >> 6;
  for (int d = 0; d < nd; ++d) {
    for (int m = 32; m >= 1; m >>= 1) {
      const unsigned int a = __shfl_xor(lo[d], m), b = __shfl_xor(hi[d], m);
      lo[d] = a < lo[d] ? a : lo[d];
      hi[d] = b > hi[d] ? b : hi[d];
    }
    if ((threadIdx.x & 63) == 0) {
      red[0][d][wave] = lo[d];
      red[1][d][wave] = hi[d];
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < nd) {
    const int d = threadIdx.x;
    unsigned int l = red[0][d][0], h = red[1][d][0];
    for (int w = 1; w < 4; ++w) {
      l = red[0][d][w] < l ? red[0][d][w] : l;
      h = red[1][d][w] > h ? red[1][d][w] : h;
    }
    atomicMin(box + d, l);
    atomicMax(box + 3 + d, h);
  }
}

__device__ __forceinline__ unsigned int order_cell(const float* __restrict__ xi, int D, const unsigned int* __restrict__ box) {
  const int nd = D < 3 ? D : 3;
  const int bits = kOrderBits / nd;
  unsigned int c[3] = {0u, 0u, 0u};
  for (int d = 0; d < nd; ++d) {
    const float lo = f_of_ord(box[d]), hi = f_of_ord(box[3 + d]);
    const float span = hi - lo;
    float t = span > 0.0f ? (xi[d] - lo) / span : 0.0f;
    int q = (int)(t * (float)(1 << bits));
    q = q < 0 ? 0 : (q >= (1 << bits) ? (1 << bits) - 1 : q);
    c[d] = (unsigned int)q;
  }
  unsigned int code = 0u;
  for (int b = bits - 1; b >= 0; --b)
    for (int d = 0; d < nd; ++d) code = (code << 1) | ((c[d] >> b) & 1u);
  return code;
}

// Cell counts of the rows (threads [0, M)) and of the columns (threads [M, M + N)).
__global__ void __launch_bounds__(256)
order_count_kernel(const float* __restrict__ x, int64_t M, const float* __restrict__ y, int64_t N, int D,
                   const unsigned int* __restrict__ box, unsigned int* __restrict__ counts,
                   unsigned int* __restrict__ ccounts) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < M) atomicAdd(counts + order_cell(x + i * D, D, box), 1u);
  else if (i < M + N) atomicAdd(ccounts + order_cell(y + (i - M) * D, D, box), 1u);
}

// Exclusive prefix sums of the two count tables in place, one workgroup of 1024 threads each
// (workgroup 0: rows, 1: columns).
__global__ void __launch_bounds__(1024) order_scan_kernel(unsigned int* __restrict__ counts, unsigned int* __restrict__ ccounts) {
  constexpr int kPer = kOrderCells / 1024;
  __shared__ unsigned int part[1024];
  unsigned int* c = blockIdx.x == 0 ? counts : ccounts;
  const int t = threadIdx.x;
  unsigned int v[kPer];
  unsigned int sum = 0u;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    v[k] = c[t * kPer + k];
    sum += v[k];
  }
  part[t] = sum;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan (Hillis-Steele)
    const unsigned int a = t >= off ? part[t - off] : 0u;
    __syncthreads();
    part[t] += a;
    __syncthreads();
  }
  unsigned int run = part[t] - sum;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    c[t * kPer + k] = run;
    run += v[k];
  }
}

// Rows to their places in the row order (threads [0, M)), columns in the column order.
__global__ void __launch_bounds__(256)
order_scatter_kernel(const float* __restrict__ x, int64_t M, const float* __restrict__ y, int64_t N, int D,
                     const unsigned int* __restrict__ box, unsigned int* __restrict__ offsets,
                     unsigned int* __restrict__ coffsets, int32_t* __restrict__ order, int32_t* __restrict__ corder) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < M) order[atomicAdd(offsets + order_cell(x + i * D, D, box), 1u)] = (int32_t)i;
  else if (i < M + N) corder[atomicAdd(coffsets + order_cell(y + (i - M) * D, D, box), 1u)] = (int32_t)(i - M);
}

// Starting thresholds. Any K columns bound a row's K-th smallest key from above, so the row's
// screen may start from the K-th smallest exact key over a few columns instead of from
// infinity: it then drops only columns that cannot enter the result (and every column split
// starts with a threshold near the final one). The columns taken are the nseed ones around the
// end of the row's cell in the columns' spatial order (cend[c] = end of cell c there), mostly
// close to the row; which ones are taken does not change the result. Keys are computed as in
// the sweep (sq_dist_key, then minus w_j). One thread per row, rows in spatial order.
template <int D, int K>
__global__ void __launch_bounds__(256)
seed_kernel(const float* __restrict__ x, const int32_t* __restrict__ order, const double* __restrict__ cols,
            const float* __restrict__ w, const int32_t* __restrict__ corder, const unsigned int* __restrict__ cend,
            const unsigned int* __restrict__ box, int64_t M, int64_t N, int nseed, double* __restrict__ seed) {
  constexpr int P = (D + 2) & ~1;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= M) return;
  const int64_t i = order[t];
  double xd[D];
#pragma unroll
  for (int d = 0; d < D; ++d) xd[d] = (double)x[i * D + d];
  int64_t lo = (int64_t)cend[order_cell(x + i * D, D, box)] - nseed / 2;
  lo = lo > N - nseed ? N - nseed : lo;
  lo = lo < 0 ? 0 : lo;
  const int64_t hi = lo + nseed < N ? lo + nseed : N;
  double keys[K];
  int32_t ids[K];
#pragma unroll
  for (int k = 0; k < K; ++k) {
    keys[k] = INFINITY;
    ids[k] = -1;
  }
  // eight columns at a time: their indices, then their coordinates, are loaded together
  constexpr int kB = 8;
  for (int64_t e0 = lo; e0 < hi; e0 += kB) {
    int32_t jj[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) jj[u] = corder[e0 + u < hi ? e0 + u : e0];
    double yv[kB][P];
    float wv[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
#pragma unroll
      for (int d = 0; d < D; ++d) yv[u][d] = cols[(int64_t)jj[u] * P + d];
      wv[u] = w ? w[jj[u]] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      if (e0 + u >= hi) break;
      double key = sq_dist_key<D>(xd, yv[u]);
      if (w) key -= (double)wv[u];
      if (key < keys[K - 1]) topk_insert<K>(keys, ids, key, jj[u]);
    }
  }
  seed[i] = keys[K - 1];
}

template <int D, int K, int R, bool LSE>
__global__ void __launch_bounds__(kBlock)
knn_kernel(const float* __restrict__ x, const int32_t* __restrict__ order, const double* __restrict__ seed,
           const double* __restrict__ cols,
           const float* __restrict__ scr,
           const float* __restrict__ w, const double* __restrict__ ymax, int32_t* __restrict__ idx,
           float* __restrict__ dist, KeyIdx* __restrict__ partial, float* __restrict__ lse_out,
           LsePartial* __restrict__ lse_partial, int64_t M, int64_t N, int64_t cps, int Kout, double c2,
           const int* __restrict__ mf, int run_if_mf) {
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

  constexpr int S32 = screen_stride(D);
  double xd[R][D], xp[R][D], A[R], marg[R], thr[R], off[R];
  float xs[R][D], thr32[R];  // the float32 screen (plain sweep): -2 x and the rounded-up threshold
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
    if (order) i = order[i];
    double s = 0.0;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      xd[r][d] = (double)x[i * D + d];
      xp[r][d] = -2.0 * xd[r][d];
      xs[r][d] = -2.0f * x[i * D + d];
      s = fma(xd[r][d], xd[r][d], s);
    }
    A[r] = s;
    marg[r] = (LSE ? kScreenMargin : kScreenMargin32) * (s + bmax);
    // (a starting key of -inf, from infinite weights, would screen out the -inf keys themselves)
    const double sk = seed ? seed[i] : INFINITY;
    thr[r] = sk > -INFINITY ? (sk - s) + marg[r] : INFINITY;
    thr32[r] = round_up_f32(thr[r]);
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
    // until the list holds K keys the starting threshold stands
    if (keys[r][K - 1] < INFINITY) {
      thr[r] = (keys[r][K - 1] - A[r]) + marg[r];
      thr32[r] = round_up_f32(thr[r]);
    }
    cnt[r] = 0;
  };

  // The float32 screen (plain sweep). screen32 computes a32 for the U columns of a tile and every
  // row (D FMAs per pair) and tells whether any lane has a candidate in any row, from the
  // smallest value of each row (one compare per row and tile, one wave-uniform branch per tile).
  // Only then does queue32 queue the candidates; the rows are flushed once per two tiles, when
  // some lane's queue could not take two more, so the common tile runs no other branch. Columns
  // past the split's end are never candidates: the last split ends in the table's (0, +inf)
  // records and the others hold whole tiles.
  auto screen32 = [&](const float (&yv)[U][D], const float (&tv)[U], float (&a)[R][U]) -> bool {
    bool hit = false;  // this lane, any row
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float mn = INFINITY;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float t = tv[u];
#pragma unroll
        for (int d = 0; d < D; ++d) t = fmaf(xs[r][d], yv[u][d], t);
        a[r][u] = t;
        mn = fminf(mn, t);
      }
      hit |= mn < thr32[r];
    }
    return hit;
  };
  bool need = false;  // wave-uniform: some row's queue could not take two more tiles
  auto queue32 = [&](int64_t j, const float (&a)[R][U]) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // at most kQueue - 2 U entries at the last flush check, so the U writes stay inside
#pragma unroll
      for (int u = 0; u < U; ++u) {
        queue[r][cnt[r]][threadIdx.x] = (int32_t)(j + u);  // kept only when the count advances
        cnt[r] += a[r][u] < thr32[r] ? 1 : 0;
      }
      need = need || __any(cnt[r] > kQueue - 2 * U);
    }
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

  const int64_t nfull = (j1 - j0) / U;  // whole tiles of the split
  if constexpr (!LSE) {
    // float32 records staged through a wave-private LDS slab: a block of kRecs records is read
    // with one 16-byte vector load per lane a whole block ahead (vector loads complete in
    // order, so the wait for one block never waits for a later one), written to the slab once
    // the block before it is screened, and read back with broadcast LDS reads (every lane the
    // same address). Every split but the last holds whole tile pairs; the last one's columns
    // past its end read the table's (0, +inf) padding.
    constexpr int C4 = S32 / 4;                                  // 16-byte chunks per record
    constexpr int kRecs = (64 / C4) / (2 * U) * (2 * U);         // records per block
    static_assert(kRecs >= 2 * U, "a block holds a tile pair");
    __shared__ float4 slab[kBlock / 64][2][64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t ntab = N + kScreenPad;
    const float4* tab = reinterpret_cast<const float4*>(scr);
    auto stage_load = [&](int64_t jb) -> float4 {
      float4 v = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (lane < kRecs * C4) {
        int64_t rec = jb + lane / C4;
        rec = rec < ntab ? rec : ntab - 1;
        v = tab[rec * C4 + lane % C4];
      }
      return v;
    };
    struct Recs {
      float y[U][D], t[U];
    };
    auto read = [&](int buf, int k0, Recs& o) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float f[S32];
#pragma unroll
        for (int c = 0; c < C4; ++c) {
          const float4 q = slab[wave][buf][(k0 + u) * C4 + c];
          f[4 * c] = q.x;
          f[4 * c + 1] = q.y;
          f[4 * c + 2] = q.z;
          f[4 * c + 3] = q.w;
        }
#pragma unroll
        for (int d = 0; d < D; ++d) o.y[u][d] = f[d];
        o.t[u] = f[D];
      }
    };
    const int ntiles = j1 > j0 ? (int)((j1 - j0 + U - 1) / U) : 0;  // fewer than 2^31 columns
    int buf = 0, k0 = 0;
    float4 stg = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (ntiles > 0) {
      slab[wave][0][lane] = stage_load(j0);
      stg = stage_load(j0 + kRecs);
    }
    int64_t j = j0;
    for (int t = 0; t < ntiles; t += 2) {
      Recs ra, rb;
      read(buf, k0, ra);
      read(buf, k0 + U, rb);
      float aa[R][U], ab[R][U];
      const bool ha = screen32(ra.y, ra.t, aa);
      const bool hb = screen32(rb.y, rb.t, ab);
      if (__builtin_expect(__any(ha || hb), 0)) {
        queue32(j, aa);
        queue32(j + U, ab);
        if (need) {
#pragma unroll
          for (int r = 0; r < R; ++r)
            if (__any(cnt[r] > kQueue - 2 * U)) flush(r);
          need = false;
        }
      }
      j += 2 * U;
      k0 += 2 * U;
      if (k0 == kRecs) {
        k0 = 0;
        buf ^= 1;
        slab[wave][buf][lane] = stg;
        stg = stage_load(j + kRecs);
      }
    }
  }
  // The column records are the same for every lane: with two rows per lane they are read
  // through the scalar unit (at K > 16 the scalar registers they would take are short).
  ConstPtr<double> ccols = (ConstPtr<double>)cols;
  auto col = [&](int64_t e) { return R == 2 ? ccols[e] : cols[e]; };
  for (int64_t t = 0; LSE && t < nfull; ++t) {
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
  if (LSE && j < j1) {
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
    int64_t i = row0 + (int64_t)r * kBlock;
    if (i >= M) continue;
    if (order) i = order[i];
    if constexpr (LSE) {
      if (gridDim.y == 1) {
        lse_out[i] = (float)((mref[r] + (double)log2f(l[r])) * M_LN2);
      } else {
        LsePartial p;
        p.m = mref[r];
        p.l = l[r];
        p.pad = 0.0f;
        lse_partial[split * M + i] = p;
      }
    }
    if (gridDim.y == 1) {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        if (k < Kout) {
          idx[i * Kout + k] = ids[r][k];
          if (dist) dist[i * Kout + k] = (float)keys[r][k];
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        KeyIdx p;
        p.key = keys[r][k];
        p.idx = ids[r][k];
        p.pad = 0;
        partial[(split * M + i) * K + k] = p;
      }
    }
  }
}

// ---- The screen on the matrix cores (plain argKmin, D <= 3, K <= 16, no weights, rows in
// spatial order). In the frame u = s (x - o), v = s (y - o) (o the centre of the bounding box
// of rows and columns, s a power of two with |u_d|, |v_d| < 1) the key of a pair is
// d^2_ij = (|u_i|^2 + a_ij) / s^2 with a_ij = |v_j|^2 - 2 u_i.v_j, so a column can enter row
// i's K smallest keys only if a_ij < s^2 key_K - |u_i|^2, key_K any upper bound on the row's
// K-th key. a_ij is a rank-(D + 1) product: one v_mfma_f32_32x32x16_f16 gives it for 1024
// pairs from fp16 pieces (u = uh + ul + ru, v = vh + vl + rv, t = |v|^2 = th + tl + rt, each
// hi piece the fp16 rounding of the value and each lo piece that of the rest):
//   a'_ij = sum_d (-2 uh_d vh_d - 2 uh_d vl_d - 2 ul_d vh_d) + th_j + tl_j   (3D + 2 products).
// Error bound: |ru|, |rv| <= 2^-22 + 2^-25 (fp16 keeps 11 bits, subnormals to 2^-24, which the
// matrix cores take exactly) and |ul|, |vl| <= 2^-11, so the dropped products
// 2 (uh rv + ul vl + ul rv + ru v) are below 2^-18.5 per dimension, the dropped rt below
// 2^-22 D; the products themselves are exact in float32 and their sum, at most 3.04 D in
// magnitude, rounds by at most (3D + 2) 2^-24 3.04 D < 2^-19 D for D <= 3. So
// |a'_ij - a_ij| < 2^-17.5 D, and the screen compares a'_ij with the threshold
// s^2 key_K - |u_i|^2 + 2^-16 D (float64, rounded up to float32). What the screen admits is
// only queued: the kept columns get their exact float64 keys as in knn_kernel, so the result
// is that of the exact keys. A non-finite frame (a point at infinity or NaN) admits every
// column.
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int kScreenQueue = 32;     // queued column offsets (16-bit) per lane and row
constexpr int kScreenPieces = 64;    // piece records past the last column
// Row tiles of 32 per wave: one (more resident waves, 92 VGPRs) measured 5 % faster than two
// (168 VGPRs), which share each column operand between two MFMAs.
constexpr int kScreenRT = 1;
constexpr int kScreenRows = kBlock / 64 * 32 * kScreenRT;  // rows per workgroup of the screen

struct ScreenFrame {
  double o[3], s;
  bool finite;
};
__device__ __forceinline__ ScreenFrame screen_frame(const unsigned int* __restrict__ box, int D) {
  ScreenFrame F;
  double h = 0.0;
  F.o[0] = F.o[1] = F.o[2] = 0.0;
  for (int d = 0; d < D; ++d) {
    const double lo = (double)f_of_ord(box[d]), hi = (double)f_of_ord(box[3 + d]);
    F.o[d] = 0.5 * (lo + hi);
    h = fmax(h, fmax(hi - F.o[d], F.o[d] - lo));
  }
  F.finite = isfinite(h);
  int ex = 0;
  if (F.finite && h > 0.0) frexp(h, &ex);  // h = m 2^ex, m in [0.5, 1): s h < 1
  F.s = F.finite && h > 0.0 ? ldexp(1.0, -ex) : 1.0;
  return F;
}

// The pieces, 16 fp16 slots per record, the row and column sides of each product:
//   slot d: -2 uh_d | vh_d    slot D + d: -2 uh_d | vl_d    slot 2D + d: -2 ul_d | vh_d
//   slot 3D: 1 | th           slot 3D + 1: 1 | tl           other slots 0.
// A record past the last column has th = 65504 and nothing else, a screen value above every
// threshold. Threads [0, M): row records rpc[i]; [M, M + N + kScreenPieces): column records,
// from the float64 column table (y_j at cols[j P], the float32 inputs widened exactly).
template <int D>
__global__ void __launch_bounds__(256)
screen_prep_kernel(const float* __restrict__ x, int64_t M, const double* __restrict__ cols, int64_t N,
                   const unsigned int* __restrict__ box, half8* __restrict__ rpc, half8* __restrict__ cpc) {
  constexpr int P = (D + 2) & ~1;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= M + N + kScreenPieces) return;
  const ScreenFrame F = screen_frame(box, D);
  half8 lo = {0, 0, 0, 0, 0, 0, 0, 0}, hi = lo;
  _Float16 sl[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) sl[k] = (_Float16)0.0f;
  if (t < M) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const double u = ((double)x[t * D + d] - F.o[d]) * F.s;
      const _Float16 uh = (_Float16)u;
      const _Float16 ul = (_Float16)(u - (double)uh);
      sl[d] = (_Float16)(-2.0f * (float)uh);
      sl[D + d] = sl[d];
      sl[2 * D + d] = (_Float16)(-2.0f * (float)ul);
    }
    sl[3 * D] = (_Float16)1.0f;
    sl[3 * D + 1] = (_Float16)1.0f;
  } else {
    const int64_t j = t - M;
    if (j < N) {
      double tt = 0.0;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const double v = (cols[j * P + d] - F.o[d]) * F.s;
        const _Float16 vh = (_Float16)v;
        sl[d] = vh;
        sl[D + d] = (_Float16)(v - (double)vh);
        sl[2 * D + d] = vh;
        tt = fma(v, v, tt);
      }
      const _Float16 th = (_Float16)tt;
      sl[3 * D] = th;
      sl[3 * D + 1] = (_Float16)(tt - (double)th);
    } else {
      sl[3 * D] = (_Float16)65504.0f;
    }
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    lo[k] = sl[k];
    hi[k] = sl[8 + k];
  }
  half8* dst = t < M ? rpc + 2 * t : cpc + 2 * (t - M);
  dst[0] = lo;
  dst[1] = hi;
}

// The sweep. A wave takes kScreenRT tiles of 32 rows (in spatial order); lane (g, l) (g = lane / 32,
// l = lane % 32) keeps row l of each tile and screens half g of the split's columns: the split
// [j0, j1) is cut into halves of H columns (H a multiple of 16) and the 32-column MFMA tile t
// takes columns j0 + g H + 16 t + q, q < 16, for lane group g. With the column of A-operand row
// m chosen so, lane (g, l) gets back exactly its 16 columns, in increasing order (MFMA output
// item q of lane (g, l) is row 8 (q / 4) + 4 g + q % 4 of the tile). Each lane keeps its own
// list of its half's K smallest keys; the row's threshold takes the smaller of the two lanes'
// K-th keys (each bounds the row's K-th key from above). At the end the two lists are merged
// into the row's list of the split.
template <int D, int K>
__global__ void __launch_bounds__(kBlock)
knn_screen_kernel(const float* __restrict__ x, const int32_t* __restrict__ order, const double* __restrict__ seed,
                  const double* __restrict__ cols, const half8* __restrict__ rpc, const half8* __restrict__ cpc,
                  const unsigned int* __restrict__ box, int32_t* __restrict__ idx, float* __restrict__ dist,
                  KeyIdx* __restrict__ partial, int64_t M, int64_t N, int64_t cps, int64_t row_blocks, int64_t splits,
                  int Kout, const int* __restrict__ mf, int run_if_mf) {
  if (mf && mf_admits(mf) != run_if_mf) return;  // the fused sweep takes these inputs
  constexpr int RT = kScreenRT;
  constexpr int P = (D + 2) & ~1;
  constexpr uint32_t kXcds = 8;  // accelerator complexes (each with its own L2) on the chip
  __shared__ uint16_t queue[RT][kScreenQueue][kBlock];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  // Workgroups go to the XCDs round-robin by id; renumbered, each XCD takes a contiguous run of
  // (split, row block) pairs, split-major, so its resident workgroups read the same split's
  // pieces, which stay in that XCD's L2.
  const uint32_t wg = blockIdx.x, total = gridDim.x;
  const uint32_t per = total / kXcds, extra = total % kXcds, xcd = wg % kXcds;
  const int64_t pair = (int64_t)xcd * per + (xcd < extra ? xcd : extra) + wg / kXcds;
  const int64_t split = pair / row_blocks, rblock = pair % row_blocks;
  const int64_t j0 = split * cps;
  const int64_t j1 = (j0 + cps < N) ? j0 + cps : N;
  const int64_t ncols = j1 > j0 ? j1 - j0 : 0;
  const int64_t H = ((ncols + 1) / 2 + 15) / 16 * 16;
  const ScreenFrame F = screen_frame(box, D);
  const double s2 = F.s * F.s;
  const double marg = 0x1p-16 * (double)D;

  half8 brow[RT];
  double xd[RT][D], au[RT], kb[RT];
  float thr32[RT];
  double keys[RT][K];
  int32_t ids[RT][K];
  int cnt[RT];
  int64_t irow[RT];
  bool valid[RT];
  auto thr_of = [&](double k, double a) __attribute__((always_inline)) -> float {
    if (!F.finite) return INFINITY;
    const float t = round_up_f32(fma(s2, k, -a) + marg);
    return t < 60000.0f ? t : 60000.0f;  // below the padding records' 65504
  };
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    const int64_t pos = (rblock * (kBlock / 64) + wave) * (32 * RT) + r * 32 + l32;
    valid[r] = pos < M;
    const int64_t i = order[pos < M ? pos : M - 1];
    irow[r] = i;
    brow[r] = rpc[2 * i + g];
    double a = 0.0;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      xd[r][d] = (double)x[i * D + d];
      const double u = (xd[r][d] - F.o[d]) * F.s;
      a = fma(u, u, a);
    }
    au[r] = a;
    kb[r] = seed[i];
    thr32[r] = thr_of(kb[r], a);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      keys[r][k] = INFINITY;
      ids[r][k] = -1;
    }
    cnt[r] = 0;
  }

  // Exact keys of this lane's queued columns (in column order), then the row's bound.
  auto flush = [&](int r) __attribute__((always_inline)) {
    for (int e = 0; e < cnt[r]; ++e) {
      const int64_t jj = j0 + (int64_t)queue[r][e][threadIdx.x];
      const double key = sq_dist_key<D>(xd[r], cols + jj * P);
      if (key < keys[r][K - 1]) topk_insert<K>(keys[r], ids[r], key, (int32_t)jj);
    }
    cnt[r] = 0;
    double kth = keys[r][K - 1];
    const double other = __shfl_xor(kth, 32);
    kth = other < kth ? other : kth;
    if (kth < kb[r]) kb[r] = kth;
    thr32[r] = thr_of(kb[r], au[r]);
  };

  // A-operand row m = l32 of tile t holds column j0 + ((m >> 2) & 1) H + 16 t + 4 (m >> 3) + (m & 3)
  // (column offsets from j0 fit 16 bits: the split holds fewer than 65000 columns)
  const int aoff = ((l32 >> 2) & 1) * (int)H + 4 * (l32 >> 3) + (l32 & 3);
  const half8* abase = cpc + 2 * (j0 + aoff) + g;
  const int ntile = (int)(H / 16), ncol = (int)ncols, goff = g * (int)H;
  const f32x16 zero16 = {};
  auto step = [&](int t, const half8& a) __attribute__((always_inline)) {
    f32x16 e[RT];
    bool hit = false;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      e[r] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, brow[r], zero16, 0, 0, 0);
      float mn = e[r][0];
#pragma unroll
      for (int q = 1; q < 16; ++q) mn = fminf(mn, e[r][q]);
      hit = hit | (mn < thr32[r]);
    }
    if (__builtin_expect(__any(hit), 0)) {
      const int off0 = goff + 16 * t;  // this lane's first column, from j0
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        // at most kScreenQueue - 16 entries on entry, so the 16 writes stay inside the queue
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          queue[r][cnt[r]][threadIdx.x] = (uint16_t)(off0 + q);  // kept only when the count advances
          cnt[r] += (off0 + q < ncol && e[r][q] < thr32[r]) ? 1 : 0;
        }
      }
#pragma unroll
      for (int r = 0; r < RT; ++r)
        if (__any(cnt[r] > kScreenQueue - 16)) flush(r);
    }
  };
  auto load = [&](int t) __attribute__((always_inline)) -> half8 { return t < ntile ? abase[32 * t] : half8{}; };
  if (!F.finite) {
    // no usable frame: every column of the lane's half is queued and gets its exact key
    for (int t = 0; t < ntile; ++t)
#pragma unroll
      for (int r = 0; r < RT; ++r) {
        for (int q = 0; q < 16; ++q) {
          const int off = goff + 16 * t + q;
          queue[r][cnt[r]][threadIdx.x] = (uint16_t)off;
          cnt[r] += off < ncol ? 1 : 0;
        }
        flush(r);
      }
  } else {
    // three operand sets in a ring, each loaded two tiles before its use (vector loads complete
    // in order, so each wait is for the oldest load only)
    half8 a0 = load(0), a1 = load(1), a2;
    for (int t = 0; t < ntile; t += 3) {
      a2 = load(t + 2);
      step(t, a0);
      if (t + 1 >= ntile) break;
      a0 = load(t + 3);
      step(t + 1, a1);
      if (t + 2 >= ntile) break;
      a1 = load(t + 4);
      step(t + 2, a2);
    }
  }
#pragma unroll
  for (int r = 0; r < RT; ++r) flush(r);

  // The two lanes of a row hold the lists of the split's two halves; lane g = 0 takes in the
  // second half's entries (higher columns: on equal keys they go after its own) and writes the
  // row's list of the split.
#pragma unroll
  for (int r = 0; r < RT; ++r) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const double ok = __shfl_xor(keys[r][k], 32);
      const int32_t oi = __shfl_xor(ids[r][k], 32);
      if (g == 0 && oi >= 0 && ok < keys[r][K - 1]) topk_insert<K>(keys[r], ids[r], ok, oi);
    }
    if (g != 0 || !valid[r]) continue;
    const int64_t i = irow[r];
    if (splits == 1) {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        if (k < Kout) {
          idx[i * Kout + k] = ids[r][k];
          if (dist) dist[i * Kout + k] = (float)keys[r][k];
        }
      }
    } else {
#pragma unroll
      for (int k = 0; k < K; ++k) {
        KeyIdx p;
        p.key = keys[r][k];
        p.idx = ids[r][k];
        p.pad = 0;
        partial[(split * M + i) * K + k] = p;
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
// The spatial orders and the starting thresholds (all null for few rows).
struct Order {
  const int32_t* rows = nullptr;
  const int32_t* cols = nullptr;
  const unsigned int* cend = nullptr;
  const unsigned int* box = nullptr;
  double* seed = nullptr;
  half8* rpc = nullptr;  // the matrix-core screen's row and column pieces (null: no such screen)
  half8* cpc = nullptr;
};

template <int D, int K>
hipError_t knn_dk(const float* x, const Order& o, const double* cols, const float* scr, const float* w, const double* ymax, int32_t* idx,
                  float* dist,
                  void* partial, float* lse_out, double* lse_partial, int64_t M, int64_t N, int Kout, double c2,
                  bool with_lse, const int* mf, const Plan& p, hipStream_t s) {
  constexpr int R = K <= 16 ? 2 : 1;
  if (o.seed) {
    const int nseed = 4 * K > 64 ? 4 * K : 64;
    seed_kernel<D, K><<<(unsigned)ceil_div(M, 256), 256, 0, s>>>(x, o.rows, cols, w, o.cols, o.cend, o.box, M, N, nseed,
                                                                  o.seed);
  }
  dim3 grid((unsigned)p.row_blocks, (unsigned)p.splits);
  KeyIdx* part = reinterpret_cast<KeyIdx*>(partial);
  LsePartial* lpart = reinterpret_cast<LsePartial*>(lse_partial);
  // the matrix-core screen takes the plain sweep's place
  bool screen = false;
  // (column offsets within a split are queued as 16-bit values)
  if constexpr (D <= 3 && K <= 16) screen = !w && o.rpc && o.cpc && o.box && o.seed && p.cols_per_split <= 65000;
  if (screen) {
    screen_prep_kernel<D><<<(unsigned)ceil_div(M + N + kScreenPieces, 256), 256, 0, s>>>(x, M, cols, N, o.box, o.rpc,
                                                                                         o.cpc);
  }
  if (with_lse)
    knn_kernel<D, K, R, true><<<grid, kBlock, 0, s>>>(x, o.rows, o.seed, cols, scr, w, ymax, idx, dist, part, lse_out, lpart,
                                                       M, N, p.cols_per_split, Kout, c2, mf, 0);
  if ((!with_lse || mf) && !screen)
    knn_kernel<D, K, R, false><<<grid, kBlock, 0, s>>>(x, o.rows, o.seed, cols, scr, w, ymax, idx, dist, part, lse_out, lpart,
                                                        M, N, p.cols_per_split, Kout, c2, mf, 1);
  if constexpr (D <= 3 && K <= 16) {
    if ((!with_lse || mf) && screen) {
      const int64_t rblocks = ceil_div(M, (int64_t)kScreenRows);
      knn_screen_kernel<D, K><<<(unsigned)(rblocks * p.splits), kBlock, 0, s>>>(
          x, o.rows, o.seed, cols, o.rpc, o.cpc, o.box, idx, dist, part, M, N, p.cols_per_split, rblocks, p.splits,
          Kout, mf, 1);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  merge_topk_kernel<K><<<(unsigned)ceil_div(M, kBlock), kBlock, 0, s>>>(part, idx, dist, M, p.splits, Kout);
  e = hipGetLastError();
  if (e != hipSuccess || !with_lse) return e;
  return launch_combine_lse(lpart, lse_out, M, p.splits, s, mf, 0);
}

template <int D>
hipError_t knn_d(int Kb, const float* x, const Order& order, const double* cols, const float* scr, const float* w, const double* ymax,
                 int32_t* idx, float* dist,
                 void* partial, float* lse_out, double* lse_partial, int64_t M, int64_t N, int Kout, double c2,
                 bool with_lse, const int* mf, const Plan& p, hipStream_t s) {
#define KEOPS_KNN_K(Kv) return knn_dk<D, Kv>(x, order, cols, scr, w, ymax, idx, dist, partial, lse_out, lse_partial, M, N, Kout, c2, with_lse, mf, p, s)
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

size_t knn_screen_bytes(int64_t N, int D) {
  return (size_t)(N + lowd::kScreenPad) * lowd::screen_stride(D) * sizeof(float);
}

bool knn_orders_rows(int64_t M) { return M >= kKnnOrderMinRows; }

namespace {
// The order workspace: box | row cell counts | column cell counts | row order (M) | column
// order (N) | starting thresholds (M doubles) | with the matrix-core screen, its row (M) and
// column (N + kScreenPieces) pieces of 32 bytes.
struct OrderLayout {
  size_t box, counts, ccounts, rows, cols, seed, rpc, cpc, total;
};
OrderLayout order_layout(int64_t M, int64_t N, int D, int K) {
  OrderLayout L;
  const size_t cells = align_up((size_t)lowd::kOrderCells * sizeof(unsigned int));
  L.box = 0;
  L.counts = align_up(8 * sizeof(unsigned int));
  L.ccounts = L.counts + cells;
  L.rows = L.ccounts + cells;
  L.cols = L.rows + align_up((size_t)M * sizeof(int32_t));
  L.seed = L.cols + align_up((size_t)N * sizeof(int32_t));
  L.rpc = L.seed + align_up((size_t)M * sizeof(double));
  const bool screen = knn_screens_on_matrix_cores(M, N, D, K);
  L.cpc = L.rpc + (screen ? align_up((size_t)M * 32) : 0);
  L.total = L.cpc + (screen ? align_up((size_t)(N + lowd::kScreenPieces) * 32) : 0);
  return L;
}
}  // namespace

bool knn_screens_on_matrix_cores(int64_t M, int64_t N, int D, int K) {
  (void)N;
  return knn_orders_rows(M) && D >= 1 && D <= 3 && K >= 1 && lowd::argk_bucket(K) <= 16;
}

size_t knn_order_bytes(int64_t M, int64_t N, int D, int K) {
  if (!knn_orders_rows(M)) return 0;
  return order_layout(M, N, D, K).total;
}

hipError_t launch_knn_lowd(const float* x, const float* y, const float* w, double* cols, float* scr, void* order_ws,
                           double* ymax,
                           int32_t* idx, float* dist, void* partial, float* lse_out, double* lse_partial, int64_t M,
                           int64_t N, int D, int K, double c2, bool with_lse, const Plan& p, hipStream_t s,
                           const KnnLse* mf_lse) {
  // column table (y_j, |y_j|^2 - w_j) uncentred, then the largest |y_j|^2 + |w_j| for the
  // screening margin
  hipError_t e = launch_prep_cols(y, cols, N, D, -1.0, false, s);
  if (e != hipSuccess) return e;
  lowd::zero_kernel<<<1, 1, 0, s>>>(ymax);
  const int64_t nb = lowd::ceil_div(N, 256);
  lowd::max_norm_kernel<<<(unsigned)(nb < 512 ? nb : 512), 256, 0, s>>>(cols, w, N, col_stride(D), D, scr,
                                                                         lowd::screen_stride(D), ymax);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // rows and columns in spatial order and the rows' starting thresholds (large M only)
  lowd::Order order;
  if (knn_orders_rows(M)) {
    char* ow = static_cast<char*>(order_ws);
    const OrderLayout L = order_layout(M, N, D, K);
    unsigned int* box = reinterpret_cast<unsigned int*>(ow + L.box);
    unsigned int* counts = reinterpret_cast<unsigned int*>(ow + L.counts);
    unsigned int* ccounts = reinterpret_cast<unsigned int*>(ow + L.ccounts);
    int32_t* rord = reinterpret_cast<int32_t*>(ow + L.rows);
    int32_t* cord = reinterpret_cast<int32_t*>(ow + L.cols);
    const int64_t tb = lowd::ceil_div(M + N, 256);
    lowd::order_clear_kernel<<<(unsigned)(lowd::kOrderCells / 256), 256, 0, s>>>(box, counts, ccounts);
    lowd::order_box_kernel<<<(unsigned)(tb < 64 ? tb : 64), 256, 0, s>>>(x, M, y, N, D, box);
    lowd::order_count_kernel<<<(unsigned)tb, 256, 0, s>>>(x, M, y, N, D, box, counts, ccounts);
    lowd::order_scan_kernel<<<2, 1024, 0, s>>>(counts, ccounts);
    lowd::order_scatter_kernel<<<(unsigned)tb, 256, 0, s>>>(x, M, y, N, D, box, counts, ccounts, rord, cord);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    order.rows = rord;
    order.cols = cord;
    order.cend = ccounts;  // after the scatter: the end of each cell in the column order
    order.box = box;
    order.seed = reinterpret_cast<double*>(ow + L.seed);
    if (knn_screens_on_matrix_cores(M, N, D, K)) {
      order.rpc = reinterpret_cast<lowd::half8*>(ow + L.rpc);
      order.cpc = reinterpret_cast<lowd::half8*>(ow + L.cpc);
    }
  }
  const int Kb = lowd::argk_bucket(K);
  // With the log-sum-exp and a matrix-core region: the matrix-core log-sum-exp sweep and the
  // plain argKmin sweep when the device-side decision admits the inputs (the two sweeps cost
  // less than the fused one on this chip), the fused float64 sweep otherwise.
  const int* mf = nullptr;
  if (with_lse && mf_lse && !w) {
    e = launch_mf_prepare(x, y, nullptr, false, nullptr, mf_lse->region, M, N, D, 0, c2, s, false,
                          mf_lse_square(D, mf_lse->plan->mf_rt));
    if (e != hipSuccess) return e;
    mf = mf_decision(mf_lse->region);
  }
#define KEOPS_KNN(Dv) lowd::knn_d<Dv>(Kb, x, order, cols, scr, w, ymax, idx, dist, partial, lse_out, lse_partial, M, N, K, c2, with_lse, mf, p, s)
  auto run = [&]() -> hipError_t { KEOPS_SWITCH_D(D, KEOPS_KNN) };
#undef KEOPS_KNN
  e = run();
  if (e != hipSuccess || !mf) return e;
  const Plan& lp = *mf_lse->plan;
  e = launch_mf_lse(lse_out, lp.splits > 1 ? mf_lse->partial : nullptr, mf_lse->region, M, N, D, lp, s);
  if (e != hipSuccess) return e;
  if (lp.splits > 1) {
    e = lowd::launch_combine_lse(static_cast<const lowd::LsePartial*>(mf_lse->partial), lse_out, M, lp.splits, s,
                                 mf, 1);
    if (e != hipSuccess) return e;
  }
  return launch_mf_lse_fix(x, y, lse_out, mf_lse->region, M, N, D, c2, lp, s);
}

}  // namespace keops
