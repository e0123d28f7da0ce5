// Low-D float32 Gauss sum with the exponent on the fp16 matrix cores ("Kernel matrix
// reduction", Implementation sketch: a_i = sum_j exp(-|x_i - y_j|^2 / (2 sigma^2)) b_j; the same
// reduction as lowd_sum.hip, which remains the float64 path for inputs this one declines).
//
// Exponent, base 2: e_ij = -c |u_i - v_j|^2 with u = (x - o)/h and v = (y - o)/h, o the centre
// and h the half-width of the bounding box of all points (so |u_d|, |v_d| <= 1), c = c2 h^2.
// Expanded, e_ij = A_i + B_j + sum_d a_id v_jd with a = 2c u, A = -c|u|^2, B = -c|v|^2, and the
// three terms cancel to a small e for the pairs that matter. A float32 accumulator adds
// multiples of 2^g without error while every partial sum stays below 2^(g+24), in any order.
// So each operand is cut, in fixed point, into fp16 pieces:
//   high part   Ah_i + Bh1_j + Bh2_j + sum_d ah_id vh_jd
//               ah, vh: a and v rounded to grids whose product grid is 2^g (11 significant bits
//               each at most); Ah, Bh = Bh1 + Bh2: A and B rounded to 2^g. Every term is a
//               multiple of 2^g and the partial sums are below 2^(g+23): the sum is exact.
//   low part    sum_d (ah vl1 + ah vl2 + al1 vh + al2 vh + al1 vl1) + Al1 + Bl1
//               vl1, vl2 and al1, al2: the next two 11-bit pieces of v - vh and a - ah;
//               Al1, Bl1: the remainders of A and B. Terms dropped are below 2^-20 of e.
// One 16x16x32 MFMA starts from Ah in the accumulator and adds the high part exactly; a second
// adds the low part onto it. Its float32 rounding is relative to |e| plus the size of the low
// part (a few units here), not to the cancelling terms (up to 2^(g+23)), which is what makes
// float32 accumulation exact enough. Each fp16 piece is scaled by a power of two (row side
// 2^-s, column side 2^s, one s per product kind) to sit inside fp16's range. The preparations
// check that every piece converts exactly; when one does not, or when the low part could grow
// past 32 (a narrow kernel on widely spread data), the float64 path runs instead: both sweeps
// are launched and each reads the decision from device memory, so nothing waits on the host.
//
// Set-aside points (Gauss sum only). When the bounding box of all points is too wide for the
// low part, but a box of the largest admissible half-width centred on the per-dimension median
// of an evenly spaced sample of the points holds all but a few of them (at most kMaxAside rows
// and kMaxAside columns), those few are set aside: a set-aside column gets the padding record (its 2^e is exactly 0 in the sweep) and
// a set-aside row zero pieces; afterwards every row gets the set-aside columns' terms added in
// a fixed order, and every set-aside row is summed over all columns from a float64 exponent.
// One far outlier thus no longer sends the whole sum to the float64 sweep.
//
// Per pair the VALU then does one v_exp_f32 and C FMAs; the two MFMAs of a 16 x 16 tile run on
// the matrix core beside them.
//
// 32 x 32 tiles (the single-channel sum for D <= 3). A 16x16x32 MFMA leaves most of its K unused
// here (D + 2 high and 5D + 2 low terms of 32), and on this chip each MFMA also delays the
// exponentials issued beside it. v_mfma_f32_32x32x16_f16 covers 1024 pairs with K = 16: the
// high MFMA takes A_i as two more products (Ah1, Ah2 against column-side ones, so the
// accumulator starts at zero; the high part stays a sum of multiples of 2^g whose partial sums
// are below 2^(g+23), exact in any order), and the low MFMA takes the low part without A's
// remainder Al1_i (5D + 1 <= 16 terms), which factors out of the row's sum:
// sum_j 2^{e_ij} b_j = 2^{Al1_i} sum_j 2^{e_ij - Al1_i} b_j, applied once per row at the end.
// Per 1024 pairs a wave then issues 2 MFMAs instead of 8.
#include "lowd_common.h"

#include <math.h>

#include <atomic>
#include <type_traits>

namespace keops {
namespace lowd {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMinK = 4;           // exponent scales below 2^4 are treated as 2^4
constexpr double kMaxLow = 32.0;   // largest admissible bound on the low part
constexpr int kBoundBlocks = 256;  // most workgroups of the bounds pass
constexpr uint32_t kXcds = 8;      // accelerator complexes (each with its own L2) on the chip
constexpr int64_t kMaxLaunch = int64_t(1) << 30;  // most workgroups per sweep launch
constexpr int kMaxAside = 256;     // most set-aside rows, and most set-aside columns (and samples)
static_assert(kBoundBlocks <= kMaxAside, "every bounds workgroup records at least one sample");
constexpr int kChunkTiles = kChunk / 16;

// Product kinds (row piece x column piece); the shift table is indexed by these.
enum Slot { kAhVh = 0, kOneBh1, kOneBh2, kAhVl1, kAhVl2, kAl1Vh, kAl2Vh, kAl1Vl1, kAl1One, kOneBl1, kSlots };

// Decisions and constants shared by the preparation and the sweeps, written on the device.
// The matrix-core sweep runs when gate != 0 and bad == 0, the float64 sweep otherwise.
struct MfParams {
  int gate;           // the scales admit the matrix-core path
  int bad;            // some piece did not convert exactly, or too many points were set aside
  int robust;         // the box is centred on the sampled median and points outside it are set aside
  int nbr, nbc;       // set-aside rows and columns so far (lists in the operand region)
  int alpha, beta, gamma;
  int sh[kSlots];
  double o[kMaxLowD];
  double inv_h;
  double cp;          // c2 h^2
};

__device__ __forceinline__ unsigned int ord_of(float f) {
  const unsigned int u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float float_of(unsigned int u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}
// v rounded to the nearest multiple of 2^g
__device__ __forceinline__ double rnd(double v, int g) { return ldexp(rint(ldexp(v, -g)), g); }

// Per-dimension min and max over the rows of x and of y: one (min, max) record per workgroup in
// parts[blockIdx] (order-preserving unsigned encodings, dimension d at d and kMaxLowD + d).
// Workgroup k also records samples k*spw .. k*spw + spw - 1 of an evenly spaced sample of the
// points (x then y), dimension d of sample s at samples[d * kMaxAside + s]. Workgroup 0 also
// clears the bad flag and the set-aside counts.
__global__ void __launch_bounds__(kBlock)
mf_bounds_kernel(const float* __restrict__ x, const float* __restrict__ y, int64_t M, int64_t N, int D,
                 unsigned int* __restrict__ parts, float* __restrict__ samples, int spw, MfParams* __restrict__ P) {
  __shared__ unsigned int red[kBlock / 64][2 * kMaxLowD];
  unsigned int lo[kMaxLowD], hi[kMaxLowD];
#pragma unroll
  for (int d = 0; d < kMaxLowD; ++d) {
    lo[d] = 0xffffffffu;
    hi[d] = 0u;
  }
  if ((int)threadIdx.x < spw) {
    const int64_t ns = (int64_t)gridDim.x * spw, k = (int64_t)blockIdx.x * spw + threadIdx.x;
    const int64_t pt = k * (M + N) / ns;
    for (int d = 0; d < D; ++d) samples[d * kMaxAside + k] = pt < M ? x[pt * D + d] : y[(pt - M) * D + d];
  }
  const int64_t n = M > N ? M : N;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n; i += (int64_t)gridDim.x * kBlock) {
#pragma unroll
    for (int d = 0; d < kMaxLowD; ++d) {
      if (d >= D) break;
      if (i < M) {
        const unsigned int v = ord_of(x[i * D + d]);
        lo[d] = v < lo[d] ? v : lo[d];
        hi[d] = v > hi[d] ? v : hi[d];
      }
      if (i < N) {
        const unsigned int v = ord_of(y[i * D + d]);
        lo[d] = v < lo[d] ? v : lo[d];
        hi[d] = v > hi[d] ? v : hi[d];
      }
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int d = 0; d < kMaxLowD; ++d) {
    unsigned int a = lo[d], b = hi[d];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const unsigned int a2 = __shfl_xor(a, m), b2 = __shfl_xor(b, m);
      a = a2 < a ? a2 : a;
      b = b2 > b ? b2 : b;
    }
    if (lane == 0) {
      red[wave][d] = a;
      red[wave][kMaxLowD + d] = b;
    }
  }
  __syncthreads();
  if (threadIdx.x < 2 * kMaxLowD) {
    const int t = threadIdx.x;
    unsigned int v = red[0][t];
    for (int w = 1; w < kBlock / 64; ++w) {
      const unsigned int u = red[w][t];
      v = (t < kMaxLowD) ? (u < v ? u : v) : (u > v ? u : v);
    }
    parts[blockIdx.x * 2 * kMaxLowD + t] = v;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    P->bad = 0;
    P->nbr = 0;
    P->nbc = 0;
  }
}

// Exponent of the largest scale bound 2^k (2 c2 h^2 <= 2^k) whose low part stays within kMaxLow.
__device__ int max_scale_exp(int D) {
  int lg = 0;
  while ((1 << lg) < D) ++lg;
  int k = kMinK;
  while (D * (ldexp(1.0, k + 1 + lg - 12) + ldexp(1.0, k + 1 - 12)) <= kMaxLow) ++k;
  return k;
}

// Half-width (times 1 + 2^-40, which keeps |u|, |v| <= 1 after rounding) and centre (o, D
// values) of the bounding box in mm; clears finite when a bound is not finite.
__device__ double box_of(const unsigned int* mm, int D, double* o, bool& finite) {
  double h = 0.0;
  finite = true;
  for (int d = 0; d < D; ++d) {
    const double lo = (double)float_of(mm[d]), hi = (double)float_of(mm[kMaxLowD + d]);
    finite = finite && isfinite(lo) && isfinite(hi);
    o[d] = (double)(float)(0.5 * (lo + hi));
    h = fmax(h, fmax(hi - o[d], o[d] - lo));
  }
  if (!(h > 0.0)) h = 1.0;  // all points equal: any scale will do
  return h * (1.0 + 0x1p-40);
}

// Whether the box of half-width h is too wide for the low part at this c2.
__device__ bool too_wide(double h, int D, double c2) { return !(2.0 * c2 * h * h <= ldexp(1.0, max_scale_exp(D))); }

// Centre, scale, grids and shifts from the bounds; gate = 0 when the low part could exceed
// kMaxLow or a shift has no admissible value. With a centre `med` (set-aside mode, given only
// when the bounding box is too wide), the box is instead the one of the largest admissible
// half-width around med, and robust = 1: the points outside it are set aside by the
// preparation. One thread.
__device__ void mf_params(const unsigned int* mm, const double* med, int D, double c2, MfParams& P) {
  bool finite = true;
  double h = box_of(mm, D, P.o, finite);
  P.robust = 0;
  if (med && finite) {
    bool ok = true;
    for (int d = 0; d < D; ++d) {
      ok = ok && isfinite(med[d]);
      P.o[d] = med[d];
    }
    // the largest half-width whose scale stays within the bound (kept a little inside it)
    h = sqrt(ldexp(1.0, max_scale_exp(D) - 1) / c2) * (1.0 - 0x1p-20);
    if (ok && h > 0.0 && isfinite(h)) P.robust = 1;
    else finite = false;
  }
  const double cp = c2 * h * h;
  P.inv_h = 1.0 / h;
  P.cp = cp;
  int gate = finite && isfinite(cp) && cp > 0.0;
  int k = kMinK;
  if (gate) {
    int ex = 0;
    const double m = frexp(2.0 * cp, &ex);    // 2cp = m 2^ex, m in [0.5, 1)
    const int kc = (m == 0.5) ? ex - 1 : ex;  // ceil(log2(2cp))
    k = kc > kMinK ? kc : kMinK;
  }
  int lg = 0;
  while ((1 << lg) < D) ++lg;
  const int gamma = k + 1 + lg - 23;  // partial sums of the high part stay below 2^(gamma + 23)
  const int alpha = k - 11;           // ah: 11 bits below |a| <= 2^k
  const int beta = gamma - alpha;     // vh: the grid that puts ah vh on 2^gamma
  const double low = D * (ldexp(1.0, k + beta - 1) + ldexp(1.0, k - 12));
  if (!(low <= kMaxLow)) gate = 0;
  // (largest power of two, grid) of each piece, as exponents
  const int ahM = k, ahQ = alpha, vhM = 0, vhQ = beta, vl1M = beta - 1, vl1Q = beta - 12, vl2M = beta - 13,
            vl2Q = beta - 24, al1M = alpha - 1, al1Q = alpha - 12, al2M = alpha - 13, al2Q = alpha - 24,
            smM = gamma - 1, smQ = gamma - 12, bh1M = gamma + 21, bh1Q = gamma + 11, bh2M = gamma + 10,
            bh2Q = gamma;
  const int rowM[kSlots] = {ahM, 0, 0, ahM, ahM, al1M, al2M, al1M, smM, 0};
  const int rowQ[kSlots] = {ahQ, 0, 0, ahQ, ahQ, al1Q, al2Q, al1Q, smQ, 0};
  const int colM[kSlots] = {vhM, bh1M, bh2M, vl1M, vl2M, vhM, vhM, vl1M, 0, smM};
  const int colQ[kSlots] = {vhQ, bh1Q, bh2Q, vl1Q, vl2Q, vhQ, vhQ, vl1Q, 0, smQ};
  for (int s = 0; s < kSlots; ++s) {
    // fp16 holds magnitudes up to 2^15 and grids down to 2^-24
    const int lo = max(rowM[s] - 15, -24 - colQ[s]);
    const int hi = min(rowQ[s] + 24, 15 - colM[s]);
    const int want = (int)floor(0.25 * (double)(rowM[s] + rowQ[s] - colM[s] - colQ[s]) + 0.5);
    if (lo > hi) gate = 0;
    P.sh[s] = want < lo ? lo : (want > hi ? hi : want);
  }
  P.alpha = alpha;
  P.beta = beta;
  P.gamma = gamma;
  P.gate = gate;
}

// v 2^s as fp16; clears ok when that is not exact.
__device__ __forceinline__ _Float16 piece(double v, int s, bool& ok) {
  const double w = ldexp(v, s);
  const _Float16 r = (_Float16)w;
  ok = ok && ((double)r == w);
  return r;
}

// the first 8 W pieces of v (which may hold more)
template <int W, int L>
__device__ __forceinline__ void store_first(half8* __restrict__ dst, const _Float16 (&v)[L]) {
  static_assert(8 * W <= L, "enough pieces");
#pragma unroll
  for (int m = 0; m < W; ++m) {
    half8 h;
#pragma unroll
    for (int k = 0; k < 8; ++k) h[k] = v[8 * m + k];
    dst[m] = h;
  }
}

template <int W>
__device__ __forceinline__ void store_pieces(half8* __restrict__ dst, const _Float16 (&v)[8 * W]) {
#pragma unroll
  for (int m = 0; m < W; ++m) {
    half8 h;
#pragma unroll
    for (int k = 0; k < 8; ++k) h[k] = v[8 * m + k];
    dst[m] = h;
  }
}

// Operand preparation, one thread per row (workgroups [0, rb)) or per column (the rest):
//   rows     rhi[i] (8 NH fp16), rlo[i] (32 NL fp16), rA[i] = Ah_i
//   sq       (NH = NL = 1, D <= 3, no gradient) the 32 x 32 tile layout instead: rhi[i] with Ah1, Ah2
//            after the high products, rlo[i] (16 fp16: the low part without Al1), rA[i] = Al1_i;
//            chi[j] with two ones after Bh1, Bh2, clo[j] (16 fp16)
//   columns  chi[j], clo[j] and bpad[j] = b[j][0..C) for j < Npad (b = null: no weights; zero
//            past N; padding columns get an exponent that underflows), and (cols not null) the
//            float64 column table cols[j] = (y_j - y_0, -c2 |y_j - y_0|^2) of the float64 sweep
//   with_y   (the one-channel gradient) the weight moves into the exponent: two more low-part
//            products add L_j = log2 |b_j| (as Lh on a 2^-6 grid plus Ll on a 2^-17 grid, so
//            to 2^-18; |L_j| >= 32 does not convert exactly and sends the call to the float32
//            sweep), and the column record is bpad[j] = (s_j, -s_j y_j[0..D)) with s_j the sign
//            of b_j (0 for b_j = 0), so the sweep forms s_j (x_i - y_j) with one FMA per
//            coordinate and needs no product with the weight.
// Each workgroup reduces the bounds records and derives the parameters itself (identically);
// workgroup 0 publishes them. A piece that does not convert exactly sets P->bad.
template <int NH, int NL>
__global__ void __launch_bounds__(kBlock)
mf_prep_kernel(const float* __restrict__ x, const float* __restrict__ y, const float* __restrict__ b, int C,
               int with_y, double* __restrict__ cols, half8* __restrict__ rhi, half8* __restrict__ rlo, float* __restrict__ rA,
               half8* __restrict__ chi, half8* __restrict__ clo, float* __restrict__ bpad,
               const unsigned int* __restrict__ parts, const float* __restrict__ samples, int nsamples, int nparts,
               int64_t M, int64_t N, int64_t Npad, int D, double c2, int64_t rb, int set_aside, int sq,
               int32_t* __restrict__ aside_rows, int32_t* __restrict__ aside_cols, MfParams* __restrict__ P) {
  __shared__ unsigned int red[kBlock / 64][2 * kMaxLowD];
  __shared__ unsigned int smm[2 * kMaxLowD];
  __shared__ float ssort[kMaxAside];
  __shared__ double smed[kMaxLowD];
  __shared__ int swide;
  __shared__ MfParams sp;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int t = 0; t < 2 * kMaxLowD; ++t) {
    unsigned int v = t < kMaxLowD ? 0xffffffffu : 0u;
    if ((int)threadIdx.x < nparts) v = parts[threadIdx.x * 2 * kMaxLowD + t];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const unsigned int u = __shfl_xor(v, m);
      v = t < kMaxLowD ? (u < v ? u : v) : (u > v ? u : v);
    }
    if (lane == 0) red[wave][t] = v;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int t = 0; t < 2 * kMaxLowD; ++t) {
      unsigned int v = red[0][t];
      for (int w = 1; w < kBlock / 64; ++w) {
        const unsigned int u = red[w][t];
        v = t < kMaxLowD ? (u < v ? u : v) : (u > v ? u : v);
      }
      smm[t] = v;
    }
    double o[kMaxLowD];
    bool finite = true;
    const double h = box_of(smm, D, o, finite);
    swide = (set_aside && finite && too_wide(h, D, c2)) ? 1 : 0;
  }
  __syncthreads();
  if (swide) {
    // set-aside mode: the centre is the per-dimension median of the bounds pass's sample
    // (every workgroup sorts the same values, so all derive the same centre)
    for (int d = 0; d < D; ++d) {
      for (int t = threadIdx.x; t < kMaxAside; t += kBlock) ssort[t] = t < nsamples ? samples[d * kMaxAside + t] : INFINITY;
      __syncthreads();
      for (int k = 2; k <= kMaxAside; k <<= 1)
        for (int jstep = k >> 1; jstep > 0; jstep >>= 1) {
          for (int t = threadIdx.x; t < kMaxAside; t += kBlock) {
            const int q = t ^ jstep;
            if (q > t) {
              const bool up = (t & k) == 0;
              const float a = ssort[t], c = ssort[q];
              if ((a > c) == up) {
                ssort[t] = c;
                ssort[q] = a;
              }
            }
          }
          __syncthreads();
        }
      if (threadIdx.x == 0) smed[d] = (double)ssort[(nsamples - 1) / 2];
      __syncthreads();
    }
  }
  if (threadIdx.x == 0) {
    mf_params(smm, swide ? smed : nullptr, D, c2, sp);
    if (blockIdx.x == 0) {
      P->gate = sp.gate;
      P->robust = sp.robust;
      P->alpha = sp.alpha;
      P->beta = sp.beta;
      P->gamma = sp.gamma;
      for (int s = 0; s < kSlots; ++s) P->sh[s] = sp.sh[s];
    }
  }
  __syncthreads();
  const bool gate = sp.gate != 0;
  const double cp = sp.cp, inv_h = sp.inv_h;
  bool ok = true;
  if ((int64_t)blockIdx.x < rb) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= M || !gate) return;
    _Float16 hi[8 * NH], lo[32 * NL];
#pragma unroll
    for (int k = 0; k < 8 * NH; ++k) hi[k] = (_Float16)0.0f;
#pragma unroll
    for (int k = 0; k < 32 * NL; ++k) lo[k] = (_Float16)0.0f;
    if (sp.robust) {
      bool inside = true;
      for (int d = 0; d < D; ++d) inside = inside && fabs(((double)x[i * D + d] - sp.o[d]) * inv_h) <= 1.0;
      if (!inside) {  // set aside: zero pieces here, summed over all columns afterwards
        const int slot = atomicAdd(&P->nbr, 1);
        if (slot < kMaxAside) aside_rows[slot] = (int32_t)i;
        else P->bad = 1;
        store_pieces<NH>(rhi + i * NH, hi);
        if (sq) store_first<2>(rlo + i * 2, lo);
        else store_pieces<4 * NL>(rlo + i * 4 * NL, lo);
        rA[i] = 0.0f;
        return;
      }
    }
    double nrm = 0.0;
#pragma unroll
    for (int d = 0; d < kMaxLowD; ++d) {
      if (d >= D) break;
      const double u = ((double)x[i * D + d] - sp.o[d]) * inv_h;
      nrm = fma(u, u, nrm);
      const double a = 2.0 * cp * u;
      const double ah = rnd(a, sp.alpha);
      const double al1 = rnd(a - ah, sp.alpha - 12);
      const double al2 = rnd(a - ah - al1, sp.alpha - 24);
      hi[d] = piece(ah, -sp.sh[kAhVh], ok);
      lo[5 * d + 0] = piece(ah, -sp.sh[kAhVl1], ok);
      lo[5 * d + 1] = piece(ah, -sp.sh[kAhVl2], ok);
      lo[5 * d + 2] = piece(al1, -sp.sh[kAl1Vh], ok);
      lo[5 * d + 3] = piece(al2, -sp.sh[kAl2Vh], ok);
      lo[5 * d + 4] = piece(al1, -sp.sh[kAl1Vl1], ok);
    }
    hi[D] = piece(1.0, -sp.sh[kOneBh1], ok);
    hi[D + 1] = piece(1.0, -sp.sh[kOneBh2], ok);
    if (with_y) {
      lo[5 * D + 2] = (_Float16)1.0f;
      lo[5 * D + 3] = (_Float16)0x1p-10f;
    }
    const double A = -cp * nrm;
    const double Ah = rnd(A, sp.gamma);
    const double Al1 = rnd(A - Ah, sp.gamma - 12);
    if (sq) {
      // Ah as two products against column-side ones (shifts mirrored from the Bh pieces, which
      // have the same magnitudes), the low part without Al1, and Al1 itself for the row factor
      const double Ah1 = rnd(Ah, sp.gamma + 11);
      hi[D + 2] = piece(Ah1, sp.sh[kOneBh1], ok);
      hi[D + 3] = piece(Ah - Ah1, sp.sh[kOneBh2], ok);
      lo[5 * D] = piece(1.0, -sp.sh[kOneBl1], ok);
      const float Alf = (float)Al1;
      ok = ok && ((double)Alf == Al1);
      rA[i] = Alf;
      store_pieces<NH>(rhi + i * NH, hi);
      store_first<2>(rlo + i * 2, lo);
    } else {
      lo[5 * D] = piece(Al1, -sp.sh[kAl1One], ok);
      lo[5 * D + 1] = piece(1.0, -sp.sh[kOneBl1], ok);
      const float Ahf = (float)Ah;
      ok = ok && ((double)Ahf == Ah);
      rA[i] = Ahf;
      store_pieces<NH>(rhi + i * NH, hi);
      store_pieces<4 * NL>(rlo + i * 4 * NL, lo);
    }
  } else {
    const int64_t j = ((int64_t)blockIdx.x - rb) * kBlock + threadIdx.x;
    if (j >= Npad) return;
    const int W = C + (with_y ? D : 0);
    if (with_y) {  // (s_j, -s_j y_j), C = 1
      const float bj = (b && j < N) ? b[j] : 0.0f;
      const float sj = bj > 0.0f ? 1.0f : (bj < 0.0f ? -1.0f : 0.0f);
      bpad[j * W] = sj;
      for (int d = 0; d < D; ++d) bpad[j * W + 1 + d] = j < N ? -(sj * y[j * D + d]) : 0.0f;
    } else if (b) {
      for (int c = 0; c < C; ++c) bpad[j * W + c] = j < N ? b[j * C + c] : 0.0f;
    }
    if (cols && j < N) {  // float64 column table
      const int P64 = col_stride(D);
      double s = 0.0;
      for (int d = 0; d < D; ++d) {
        const double v = (double)y[j * D + d] - (double)y[d];
        cols[j * P64 + d] = v;
        s = fma(v, v, s);
      }
      cols[j * P64 + D] = -c2 * s;
      for (int d = D + 1; d < P64; ++d) cols[j * P64 + d] = 0.0;
    }
    if (!gate) return;
    _Float16 hi[8 * NH], lo[32 * NL];
#pragma unroll
    for (int k = 0; k < 8 * NH; ++k) hi[k] = (_Float16)0.0f;
#pragma unroll
    for (int k = 0; k < 32 * NL; ++k) lo[k] = (_Float16)0.0f;
    bool inside = true;
    if (j < N && sp.robust) {
      for (int d = 0; d < D; ++d) inside = inside && fabs(((double)y[j * D + d] - sp.o[d]) * inv_h) <= 1.0;
      if (!inside) {  // set aside: the padding record here, its terms added to every row afterwards
        const int slot = atomicAdd(&P->nbc, 1);
        if (slot < kMaxAside) aside_cols[slot] = (int32_t)j;
        else P->bad = 1;
      }
    }
    if (j < N && inside) {
      double nrm = 0.0;
#pragma unroll
      for (int d = 0; d < kMaxLowD; ++d) {
        if (d >= D) break;
        const double v = ((double)y[j * D + d] - sp.o[d]) * inv_h;
        nrm = fma(v, v, nrm);
        const double vh = rnd(v, sp.beta);
        const double vl1 = rnd(v - vh, sp.beta - 12);
        const double vl2 = rnd(v - vh - vl1, sp.beta - 24);
        hi[d] = piece(vh, sp.sh[kAhVh], ok);
        lo[5 * d + 0] = piece(vl1, sp.sh[kAhVl1], ok);
        lo[5 * d + 1] = piece(vl2, sp.sh[kAhVl2], ok);
        lo[5 * d + 2] = piece(vh, sp.sh[kAl1Vh], ok);
        lo[5 * d + 3] = piece(vh, sp.sh[kAl2Vh], ok);
        lo[5 * d + 4] = piece(vl1, sp.sh[kAl1Vl1], ok);
      }
      const double Bv = -cp * nrm;
      const double Bh = rnd(Bv, sp.gamma);
      const double Bh1 = rnd(Bh, sp.gamma + 11);
      hi[D] = piece(Bh1, sp.sh[kOneBh1], ok);
      hi[D + 1] = piece(Bh - Bh1, sp.sh[kOneBh2], ok);
      if (sq) {
        hi[D + 2] = piece(1.0, -sp.sh[kOneBh1], ok);
        hi[D + 3] = piece(1.0, -sp.sh[kOneBh2], ok);
        lo[5 * D] = piece(rnd(Bv - Bh, sp.gamma - 12), sp.sh[kOneBl1], ok);
      } else {
        lo[5 * D] = piece(1.0, sp.sh[kAl1One], ok);
        lo[5 * D + 1] = piece(rnd(Bv - Bh, sp.gamma - 12), sp.sh[kOneBl1], ok);
      }
      if (with_y) {
        const double bj = b ? (double)b[j] : 0.0;
        const double L = bj != 0.0 ? log2(fabs(bj)) : 0.0;
        const double Lh = rnd(L, -6);
        lo[5 * D + 2] = piece(Lh, 0, ok);
        lo[5 * D + 3] = piece(rnd(L - Lh, -17), 10, ok);
      }
    } else {
      // padding column: e = A_i - 65504 2^-s, far below every real exponent (those are at least
      // -2^(gamma+23)), so 2^e is exactly 0 and no reduction sees it
      hi[D] = (_Float16)-65504.0f;
    }
    store_pieces<NH>(chi + j * NH, hi);
    if (sq) store_first<2>(clo + j * 2, lo);
    else store_pieces<4 * NL>(clo + j * 4 * NL, lo);
  }
  if (!ok) P->bad = 1;
}

// out[i][c] = sum_j 2^{e_ij} b[j][c] over the columns [j0, j1) of this split (times rscale[i]
// with one split), else partial[split][i][c]. A wave holds RT tiles of 16 rows; lane (g, l)
// (g = lane / 16, l = lane % 16) feeds row l and features 8g..8g+7 of each tile to the MFMA and
// gets back e for rows 4g..4g+3 against column l of the current 16-column tile. Lanes keep
// per-column partial sums (folded into the totals every kChunk columns); the 16 lanes of a
// row group add theirs at the end. The next tile's operands are loaded while the current one
// is reduced.
// Waves per SIMD the register allocation must leave room for: 4 for the narrow single-channel
// form with 4 row tiles (it then fits 128 VGPRs without spilling), else no constraint.
template <int C, int RT, int NH>
constexpr int sweep_waves() { return (NH == 1 && C == 1 && RT == 4) ? 4 : 1; }

template <int C, int RT, int NH, int NL>
__global__ void __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(sweep_waves<C, RT, NH>())))
gauss_sum_mf_kernel(const half8* __restrict__ rhi, const half8* __restrict__ rlo, const float* __restrict__ rA,
                    const half8* __restrict__ chi, const half8* __restrict__ clo, const float* __restrict__ bpad,
                    float* __restrict__ out, const float* __restrict__ rscale, const MfParams* __restrict__ P,
                    int64_t M, int64_t N, int64_t cps, int64_t row_blocks, int64_t splits, int64_t pair0) {
  if (!P->gate || P->bad) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  // Workgroups go to the chip's 8 XCDs round-robin by id. Renumber them so that each XCD takes a
  // contiguous run of (split, row block) pairs, split-major: the workgroups resident on one XCD
  // then sweep the same split's column table, which stays in that XCD's L2. (This launch covers
  // pairs [pair0, pair0 + gridDim.x).)
  const uint32_t wg = blockIdx.x, total = gridDim.x;
  const uint32_t per = total / kXcds, extra = total % kXcds, xcd = wg % kXcds;
  const int64_t pair = pair0 + xcd * per + (xcd < extra ? xcd : extra) + wg / kXcds;
  const int64_t split = pair / row_blocks;
  const int64_t j0 = split * cps;
  const int64_t j1 = (j0 + cps < N) ? j0 + cps : N;
  const int64_t base = ((int64_t)(pair % row_blocks) * (kBlock / 64) + wave) * 16 * RT;
  const half8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};

  half8 ahi[RT], alo[RT][NL];
  f32x4 cinit[RT];
  float acc[RT][4][C], part[RT][4][C];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    int64_t i = base + r * 16 + l16;
    i = i < M ? i : M - 1;
    ahi[r] = g < NH ? rhi[i * NH + g] : zero8;
#pragma unroll
    for (int m = 0; m < NL; ++m) alo[r][m] = rlo[i * 4 * NL + m * 4 + g];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int64_t ii = base + r * 16 + 4 * g + q;
      ii = ii < M ? ii : M - 1;
      cinit[r][q] = rA[ii];
#pragma unroll
      for (int c = 0; c < C; ++c) acc[r][q][c] = part[r][q][c] = 0.0f;
    }
  }
  // Per-lane element offsets into a 16-column tile; the tile bases are wave-uniform.
  const int ochi = l16 * NH + (g < NH ? g : 0), oclo = l16 * 4 * NL + g, ob = l16 * C;
  struct Ops {
    half8 h, l[NL];
    float w[C];
  };
  auto load = [&](int64_t jt, Ops& o) {
    const half8* ph = chi + jt * NH;
    const half8* pl = clo + jt * 4 * NL;
    const float* pw = bpad + jt * C;
    o.h = ph[ochi];
#pragma unroll
    for (int m = 0; m < NL; ++m) o.l[m] = pl[oclo + 4 * m];
#pragma unroll
    for (int c = 0; c < C; ++c) o.w[c] = pw[ob + c];
  };
  auto tile = [&](const Ops& o) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      f32x4 e = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[r], o.h, cinit[r], 0, 0, 0);
#pragma unroll
      for (int m = 0; m < NL; ++m) e = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[r][m], o.l[m], e, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float k = exp2_hw(e[q]);
#pragma unroll
        for (int c = 0; c < C; ++c) part[r][q][c] = fmaf(k, o.w[c], part[r][q][c]);
      }
    }
  };
  // Two tiles per trip with alternating operand sets: each load is issued one tile ahead of its
  // use, and the sets never need copying. Column ranges are whole pairs of tiles (splits are
  // multiples of 32 columns and the tables are zero-padded to a multiple of 32).
  const int64_t ntiles = j1 > j0 ? 2 * ((j1 - j0 + 31) / 32) : 0;
  Ops A, B;
  if (ntiles > 0) load(j0, A);
  int tiles = 0;
  for (int64_t t = 0; t < ntiles; t += 2) {
    const int64_t ja = j0 + t * 16;
    load(ja + 16, B);
    tile(A);
    load(t + 2 < ntiles ? ja + 32 : ja, A);
    tile(B);
    tiles += 2;
    if (tiles == kChunkTiles) {
      tiles = 0;
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int c = 0; c < C; ++c) {
            acc[r][q][c] += part[r][q][c];
            part[r][q][c] = 0.0f;
          }
    }
  }
  // fold the last chunk, then add the 16 per-column partials of each row (lanes 16g .. 16g+15)
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int c = 0; c < C; ++c) {
        float v = acc[r][q][c] + part[r][q][c];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 8);
        acc[r][q][c] = v;
      }
  float* dst = out + split * M * C;
  const bool scaled = rscale && splits == 1;
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t i = base + r * 16 + 4 * g + q;
      if (l16 == q && i < M) {
        const float sc = scaled ? rscale[i] : 1.0f;
#pragma unroll
        for (int c = 0; c < C; ++c) dst[i * C + c] = sc * acc[r][q][c];
      }
    }
}

// The sum on 32 x 32 tiles (operands in the sq layout of mf_prep_kernel), C <= 4 channels:
// out[i][c] = 2^{Al1_i} sum_j 2^{e_ij - Al1_i} b[j][c] over the columns [j0, j1) of this split
// (times rscale[i] with one split), else partial[split][i][c]. A wave holds RT tiles of 32 rows;
// lane (g, l) (g = lane / 32, l = lane % 32) feeds row l and K slots 8g..8g+7 of each tile to the
// MFMA and gets back the exponents of rows 8(q / 4) + 4g + q % 4 (q < 16) against column l of
// the current 32-column tile. Lanes keep per-column partial sums (folded into the totals every
// kChunk columns); the 32 lanes of a row group add theirs at the end.
typedef float f32x16 __attribute__((ext_vector_type(16)));

template <int RT, int C>
__global__ void __launch_bounds__(kBlock)
gauss_sum_mf32_kernel(const half8* __restrict__ rhi, const half8* __restrict__ rlo, const float* __restrict__ rrem,
                      const half8* __restrict__ chi, const half8* __restrict__ clo, const float* __restrict__ bpad,
                      float* __restrict__ out, const float* __restrict__ rscale, const MfParams* __restrict__ P,
                      int64_t M, int64_t N, int64_t cps, int64_t row_blocks, int64_t splits, int64_t pair0) {
  if (!P->gate || P->bad) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  // XCD-aware renumbering, as in gauss_sum_mf_kernel
  const uint32_t wg = blockIdx.x, total = gridDim.x;
  const uint32_t per = total / kXcds, extra = total % kXcds, xcd = wg % kXcds;
  const int64_t pair = pair0 + xcd * per + (xcd < extra ? xcd : extra) + wg / kXcds;
  const int64_t split = pair / row_blocks;
  const int64_t j0 = split * cps;
  const int64_t j1 = (j0 + cps < N) ? j0 + cps : N;
  const int64_t base = ((int64_t)(pair % row_blocks) * (kBlock / 64) + wave) * 32 * RT;
  const half8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};

  // With one channel the chunk totals live in LDS, each lane in its own slots (32 KB per
  // workgroup at RT = 2): with them in registers the sweep needs 149 VGPRs and runs three waves
  // per SIMD, with them here 112 VGPRs and four (1M sum 93.4 -> 91.9 ms). With more channels
  // (one row tile) they stay in registers.
  constexpr bool kLds = C == 1;
  half8 ahi[RT], alo[RT];
  float part[RT][16][C];
  float acc[kLds ? 1 : RT][kLds ? 1 : 16][C];
  __shared__ float sacc[kBlock / 64][kLds ? RT : 1][kLds ? 16 : 1][64];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    int64_t i = base + r * 32 + l32;
    i = i < M ? i : M - 1;
    ahi[r] = g == 0 ? rhi[i] : zero8;
    alo[r] = rlo[i * 2 + g];
#pragma unroll
    for (int q = 0; q < 16; ++q)
#pragma unroll
      for (int c = 0; c < C; ++c) {
        part[r][q][c] = 0.0f;
        if constexpr (kLds) sacc[wave][r][q][lane] = 0.0f;
        else acc[r][q][c] = 0.0f;
      }
  }
  struct Ops {
    half8 h, l;
    float w[C];
  };
  auto load = [&](int64_t jt, Ops& o) {
    o.h = chi[jt + l32];
    o.l = clo[(jt + l32) * 2 + g];
#pragma unroll
    for (int c = 0; c < C; ++c) o.w[c] = bpad[(jt + l32) * C + c];
  };
  const f32x16 zero16 = {};
  auto tile = [&](const Ops& o) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      f32x16 e = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[r], o.h, zero16, 0, 0, 0);
      e = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[r], o.l, e, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float k = exp2_hw(e[q]);
#pragma unroll
        for (int c = 0; c < C; ++c) part[r][q][c] = fmaf(k, o.w[c], part[r][q][c]);
      }
    }
  };
  auto fold = [&]() {
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int q = 0; q < 16; ++q)
#pragma unroll
        for (int c = 0; c < C; ++c) {
          if constexpr (kLds) sacc[wave][r][q][lane] += part[r][q][c];
          else acc[r][q][c] += part[r][q][c];
          part[r][q][c] = 0.0f;
        }
  };
  // Two tiles per trip with alternating operand sets, each load one tile ahead of its use. The
  // column range is whole 32-column tiles (splits are multiples of 32 columns and the tables are
  // padded to a multiple of 32); an odd last tile is reduced after the loop.
  constexpr int kChunkTiles32 = kChunk / 32;
  const int64_t ntiles = j1 > j0 ? (j1 - j0 + 31) / 32 : 0;
  Ops A, B;
  if (ntiles > 0) load(j0, A);
  int tiles = 0;
  int64_t t = 0;
  for (; t + 2 <= ntiles; t += 2) {
    const int64_t ja = j0 + t * 32;
    load(ja + 32, B);
    tile(A);
    load(t + 2 < ntiles ? ja + 64 : ja, A);
    tile(B);
    tiles += 2;
    if (tiles == kChunkTiles32) {
      tiles = 0;
      fold();
    }
  }
  if (t < ntiles) tile(A);
  fold();
  // add the 32 per-column partials of each row (the lanes of one half-wave)
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int q = 0; q < 16; ++q)
#pragma unroll
      for (int c = 0; c < C; ++c) {
        float v;
        if constexpr (kLds) v = sacc[wave][r][q][lane];
        else v = acc[r][q][c];
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 8);
        v += __shfl_xor(v, 16);
        part[r][q][c] = v;
      }
  float* dst = out + split * M * C;
  const bool scaled = rscale && splits == 1;
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int64_t i = base + r * 32 + 8 * (q / 4) + 4 * g + (q % 4);
      if (l32 == q && i < M) {
        const float sc = (scaled ? rscale[i] : 1.0f) * exp2f(rrem[i]);
#pragma unroll
        for (int c = 0; c < C; ++c) dst[i * C + c] = sc * part[r][q][c];
      }
    }
}

// out_i = ln sum_j 2^{e_ij} over the columns [j0, j1) of this split with one split, else the
// split's (m, l) pair. Same tiles and lanes as the sum; per lane and row slot a running shift
// m (an integer, base 2) and l = sum 2^{e - m} over the lane's columns. m is raised, for every
// slot of the wave at once, only in a tile where some lane's term would exceed 2^kLseSlack
// (from -inf in the first tile); the 16 lanes of a row merge their (m, l) at the end.
// A slot is settled once m >= kLseSettled (-64): the exponent is never positive (its computed
// value exceeds 0 by a rounding far below 1), so the plain terms 2^e cannot overflow, and the
// ones that underflow float32 (below 2^-126) are negligible against the row's largest term
// (at least 2^(m - 1) >= 2^-65). Once every slot of the wave is settled, each slot's sum is
// rescaled to the plain scale, l 2^m with m = 0 from then on (m an integer: exact, and
// l 2^m >= 2^-81 stays normal), and the loop adds the plain terms 2^e with no shift and no
// test.
template <int RT, int NH, int NL>
__global__ void __launch_bounds__(kBlock)
lse_mf_kernel(const half8* __restrict__ rhi, const half8* __restrict__ rlo, const float* __restrict__ rA,
              const half8* __restrict__ chi, const half8* __restrict__ clo, float* __restrict__ out,
              LsePartial* __restrict__ partial, const MfParams* __restrict__ P, int64_t M, int64_t N, int64_t cps,
              int64_t row_blocks, int64_t splits, int64_t pair0) {
  if (!P->gate || P->bad) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const uint32_t wg = blockIdx.x, total = gridDim.x;
  const uint32_t per = total / kXcds, extra = total % kXcds, xcd = wg % kXcds;
  const int64_t pair = pair0 + xcd * per + (xcd < extra ? xcd : extra) + wg / kXcds;
  const int64_t split = pair / row_blocks;
  const int64_t j0 = split * cps;
  const int64_t j1 = (j0 + cps < N) ? j0 + cps : N;
  const int64_t base = ((int64_t)(pair % row_blocks) * (kBlock / 64) + wave) * 16 * RT;
  const half8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};

  half8 ahi[RT], alo[RT][NL];
  f32x4 cinit[RT];
  float m[RT][4], l[RT][4];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    int64_t i = base + r * 16 + l16;
    i = i < M ? i : M - 1;
    ahi[r] = g < NH ? rhi[i * NH + g] : zero8;
#pragma unroll
    for (int n = 0; n < NL; ++n) alo[r][n] = rlo[i * 4 * NL + n * 4 + g];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int64_t ii = base + r * 16 + 4 * g + q;
      ii = ii < M ? ii : M - 1;
      cinit[r][q] = rA[ii];
      m[r][q] = -INFINITY;
      l[r][q] = 0.0f;
    }
  }
  const int ochi = l16 * NH + (g < NH ? g : 0), oclo = l16 * 4 * NL + g;
  struct Ops {
    half8 h, l[NL];
  };
  auto load = [&](int64_t jt, Ops& o) {
    const half8* ph = chi + jt * NH;
    const half8* pl = clo + jt * 4 * NL;
    o.h = ph[ochi];
#pragma unroll
    for (int n = 0; n < NL; ++n) o.l[n] = pl[oclo + 4 * n];
  };
  // While the shift is tracked, the high and low parts of the exponent stay in separate
  // accumulators: eh is exact (a multiple of 2^gamma), so eh - m is exact for every term within
  // 2^(gamma+24) >= 64 of the shift, and d = (eh - m) + el rounds relative to the small shifted
  // exponent instead of to |e|. Rows far from every column (|e| in the thousands, where one
  // float32 rounding of e alone is 2^-11 or more) then keep their log-sum-exp to a few 1e-7.
  auto tile = [&](const Ops& o) {
    float eh[RT][4], el[RT][4], d[RT][4];
    float dmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      const f32x4 th = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[r], o.h, cinit[r], 0, 0, 0);
      f32x4 tl = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int n = 0; n < NL; ++n) tl = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[r][n], o.l[n], tl, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        eh[r][q] = th[q];
        el[r][q] = tl[q];
        d[r][q] = (th[q] - m[r][q]) + tl[q];
        dmax = fmaxf(dmax, d[r][q]);
      }
    }
    if (__any(dmax > kLseSlack)) {
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float mn = fmaxf(m[r][q], ceilf(eh[r][q] + el[r][q]));
          l[r][q] *= exp2_hw(m[r][q] - mn);
          m[r][q] = mn;
          d[r][q] = (eh[r][q] - mn) + el[r][q];
        }
    }
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q) l[r][q] += exp2_hw(d[r][q]);
  };
  auto tile_settled = [&](const Ops& o) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[r], o.h, cinit[r], 0, 0, 0);
#pragma unroll
      for (int n = 0; n < NL; ++n) t = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[r][n], o.l[n], t, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) l[r][q] += exp2_hw(t[q]);
    }
  };
  constexpr float kLseSettled = -64.0f;
  auto all_settled = [&]() {
    bool ok = true;
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q) ok = ok && m[r][q] >= kLseSettled;
    return __all(ok);
  };
  const int64_t ntiles = j1 > j0 ? 2 * ((j1 - j0 + 31) / 32) : 0;
  Ops A, B;
  if (ntiles > 0) load(j0, A);
  bool settled = false;
  int64_t t = 0;
  for (; t < ntiles && !settled; t += 2) {
    const int64_t ja = j0 + t * 16;
    load(ja + 16, B);
    tile(A);
    load(t + 2 < ntiles ? ja + 32 : ja, A);
    tile(B);
    settled = all_settled();
  }
  if (settled) {
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        l[r][q] *= exp2_hw(m[r][q]);
        m[r][q] = 0.0f;
      }
  }
  for (; t < ntiles; t += 2) {
    const int64_t ja = j0 + t * 16;
    load(ja + 16, B);
    tile_settled(A);
    load(t + 2 < ntiles ? ja + 32 : ja, A);
    tile_settled(B);
  }

  // merge the 16 lanes of each row: m = max, l = sum l 2^(m_lane - m)
  const bool last = splits == 1;
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float mm = m[r][q];
#pragma unroll
      for (int s = 1; s < 16; s <<= 1) mm = fmaxf(mm, __shfl_xor(mm, s));
      float ll = m[r][q] == -INFINITY ? 0.0f : l[r][q] * exp2_hw(m[r][q] - mm);
#pragma unroll
      for (int s = 1; s < 16; s <<= 1) ll += __shfl_xor(ll, s);
      const int64_t i = base + r * 16 + 4 * g + q;
      if (l16 == q && i < M) {
        if (last) {
          out[i] = (float)(((double)mm + (double)log2f(ll)) * M_LN2);
        } else {
          LsePartial pp;
          pp.m = (double)mm;
          pp.l = ll;
          pp.pad = 0.0f;
          partial[split * M + i] = pp;
        }
      }
    }
}

// The log-sum-exp on 32 x 32 tiles (operands in the sq layout), with no running shift:
// l_i = sum_j 2^{e_ij - Al1_i} over the columns [j0, j1) of this split, written as
// ln(2^{Al1_i} l_i) with one split, else as the split's pair (m, l) = (Al1_i, l_i). The
// exponent is never positive (its computed value exceeds 0 by a rounding far below 1), so no
// term overflows; what underflows float32 is negligible for every row whose sum is at least
// 2^-64 (at most N 2^-126 against it). Rows below that, or with no term at all, are far from
// every column: lse_fix_kernel recomputes them afterwards. Same tiles and lanes as
// gauss_sum_mf32_kernel; per 1024 pairs a wave issues 2 MFMAs, 16 exponentials and 16 adds.
template <int RT>
__global__ void __launch_bounds__(kBlock)
lse_mf32_kernel(const half8* __restrict__ rhi, const half8* __restrict__ rlo, const float* __restrict__ rrem,
                const half8* __restrict__ chi, const half8* __restrict__ clo, float* __restrict__ out,
                LsePartial* __restrict__ partial, const MfParams* __restrict__ P, int64_t M, int64_t N, int64_t cps,
                int64_t row_blocks, int64_t splits, int64_t pair0) {
  if (!P->gate || P->bad) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const uint32_t wg = blockIdx.x, total = gridDim.x;
  const uint32_t per = total / kXcds, extra = total % kXcds, xcd = wg % kXcds;
  const int64_t pair = pair0 + xcd * per + (xcd < extra ? xcd : extra) + wg / kXcds;
  const int64_t split = pair / row_blocks;
  const int64_t j0 = split * cps;
  const int64_t j1 = (j0 + cps < N) ? j0 + cps : N;
  const int64_t base = ((int64_t)(pair % row_blocks) * (kBlock / 64) + wave) * 32 * RT;
  const half8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};

  half8 ahi[RT], alo[RT];
  float l[RT][16];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    int64_t i = base + r * 32 + l32;
    i = i < M ? i : M - 1;
    ahi[r] = g == 0 ? rhi[i] : zero8;
    alo[r] = rlo[i * 2 + g];
#pragma unroll
    for (int q = 0; q < 16; ++q) l[r][q] = 0.0f;
  }
  struct Ops {
    half8 h, l;
  };
  auto load = [&](int64_t jt, Ops& o) {
    o.h = chi[jt + l32];
    o.l = clo[(jt + l32) * 2 + g];
  };
  const f32x16 zero16 = {};
  auto tile = [&](const Ops& o) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      f32x16 e = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[r], o.h, zero16, 0, 0, 0);
      e = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[r], o.l, e, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 16; ++q) l[r][q] += exp2_hw(e[q]);
    }
  };
  const int64_t ntiles = j1 > j0 ? (j1 - j0 + 31) / 32 : 0;
  Ops A, B;
  if (ntiles > 0) load(j0, A);
  int64_t t = 0;
  for (; t + 2 <= ntiles; t += 2) {
    const int64_t ja = j0 + t * 32;
    load(ja + 32, B);
    tile(A);
    load(t + 2 < ntiles ? ja + 64 : ja, A);
    tile(B);
  }
  if (t < ntiles) tile(A);
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      float v = l[r][q];
      v += __shfl_xor(v, 1);
      v += __shfl_xor(v, 2);
      v += __shfl_xor(v, 4);
      v += __shfl_xor(v, 8);
      v += __shfl_xor(v, 16);
      l[r][q] = v;
    }
  const bool last = splits == 1;
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int64_t i = base + r * 32 + 8 * (q / 4) + 4 * g + (q % 4);
      if (l32 == q && i < M) {
        if (last) {
          out[i] = (float)(((double)rrem[i] + (double)log2f(l[r][q])) * M_LN2);
        } else {
          LsePartial pp;
          pp.m = (double)rrem[i];
          pp.l = l[r][q];
          pp.pad = 0.0f;
          partial[split * M + i] = pp;
        }
      }
    }
}

// After lse_mf32_kernel (and the split combine): rows whose log-sum-exp came out below
// 64 ln 2 (sum below 2^-64), or not finite, are recomputed from a float64 exponent. Each
// workgroup looks at its 256 rows and, for each row flagged, all its threads take a fixed stride
// of the columns with a running maximum (float64), merged in a fixed tree:
// out_i = ln sum_j exp(-c2 ln 2 |x_i - y_j|^2) exactly in float64 arithmetic up to the final
// rounding. With no far row every workgroup returns after reading its rows.
template <int D>
__global__ void __launch_bounds__(kBlock)
lse_fix_kernel(const float* __restrict__ x, const float* __restrict__ y, float* __restrict__ out,
               const MfParams* __restrict__ P, int64_t M, int64_t N, double c2) {
  if (!P->gate || P->bad) return;
  __shared__ int rows[kBlock];
  __shared__ int nflag;
  __shared__ double rm[kBlock], rl[kBlock];
  const float kFloor = (float)(-64.0 * M_LN2);
  if (threadIdx.x == 0) nflag = 0;
  __syncthreads();
  const int64_t i0 = (int64_t)blockIdx.x * kBlock;
  {
    const int64_t i = i0 + threadIdx.x;
    if (i < M && !(out[i] >= kFloor)) rows[atomicAdd(&nflag, 1)] = (int)threadIdx.x;
  }
  __syncthreads();
  const int nf = nflag;
  if (nf == 0) return;
  // (the rows are recorded in an arbitrary order; each row's result does not depend on it)
  for (int k = 0; k < nf; ++k) {
    const int64_t i = i0 + rows[k];
    double xi[D];
#pragma unroll
    for (int d = 0; d < D; ++d) xi[d] = (double)x[i * D + d];
    double m = -INFINITY, lv = 0.0;
    for (int64_t j = threadIdx.x; j < N; j += kBlock) {
      double d2 = 0.0;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const double t = xi[d] - (double)y[j * D + d];
        d2 = fma(t, t, d2);
      }
      const double e = -c2 * d2;  // base 2
      if (!(e > -INFINITY)) continue;  // no contribution
      if (e > m) {
        lv = lv * exp2(m - e) + 1.0;
        m = e;
      } else {
        lv += exp2(e - m);
      }
    }
    rm[threadIdx.x] = m;
    rl[threadIdx.x] = lv;
    __syncthreads();
    for (int h = kBlock / 2; h > 0; h >>= 1) {
      if ((int)threadIdx.x < h) {
        const double ma = rm[threadIdx.x], mb = rm[threadIdx.x + h];
        const double mm = ma > mb ? ma : mb;
        const double la = ma == -INFINITY ? 0.0 : rl[threadIdx.x] * exp2(ma - mm);
        const double lb = mb == -INFINITY ? 0.0 : rl[threadIdx.x + h] * exp2(mb - mm);
        rm[threadIdx.x] = mm;
        rl[threadIdx.x] = la + lb;
      }
      __syncthreads();
    }
    if (threadIdx.x == 0) out[i] = (float)((rm[0] + log2(rl[0])) * M_LN2);
    __syncthreads();
  }
}

// Gradient with respect to x, one channel ("Kernel Operations on the GPU, with Autodiff, without
// Memory Overflows": the derivative of a reduction is a reduction over the same pairs):
//   out_i = -(g_i / sigma^2) sum_j k_ij b_j (x_i - y_j)
// The exponent carries log2 |b_j| (see the preparation), so 2^e = k_ij |b_j|; the record
// bw[j] = (s_j, -s_j y_j) gives s_j (x_i - y_j) = fma(s_j, x_i, -s_j y_j), which rounds exactly
// as x_i - y_j does (s_j = +-1 or 0): per pair one exp and 2 D FMAs, the differences taken in
// float32 from the original coordinates (no x_i sum - sum y cancellation).
// Lanes keep per-column partials for their 4 rows per tile, folded every kChunk columns and
// across the 16 lanes of a row at the end.
template <int D, int RT, int NH, int NL>
__global__ void __launch_bounds__(kBlock)
grad_mf_kernel(const half8* __restrict__ rhi, const half8* __restrict__ rlo, const float* __restrict__ rA,
               const half8* __restrict__ chi, const half8* __restrict__ clo, const float* __restrict__ bw,
               const float* __restrict__ x, const float* __restrict__ g, float* __restrict__ out, float inv_sigma2,
               const MfParams* __restrict__ P, int64_t M, int64_t N, int64_t cps, int64_t row_blocks,
               int64_t splits, int64_t pair0) {
  if (!P->gate || P->bad) return;
  constexpr int W = 1 + D;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const uint32_t wg = blockIdx.x, total = gridDim.x;
  const uint32_t per = total / kXcds, extra = total % kXcds, xcd = wg % kXcds;
  const int64_t pair = pair0 + xcd * per + (xcd < extra ? xcd : extra) + wg / kXcds;
  const int64_t split = pair / row_blocks;
  const int64_t j0 = split * cps;
  const int64_t j1 = (j0 + cps < N) ? j0 + cps : N;
  const int64_t base = ((int64_t)(pair % row_blocks) * (kBlock / 64) + wave) * 16 * RT;
  const half8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};

  half8 ahi[RT], alo[RT][NL];
  f32x4 cinit[RT];
  float xr[RT][4][D], acc[RT][4][D], part[RT][4][D];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    int64_t i = base + r * 16 + l16;
    i = i < M ? i : M - 1;
    ahi[r] = g4 < NH ? rhi[i * NH + g4] : zero8;
#pragma unroll
    for (int n = 0; n < NL; ++n) alo[r][n] = rlo[i * 4 * NL + n * 4 + g4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int64_t ii = base + r * 16 + 4 * g4 + q;
      ii = ii < M ? ii : M - 1;
      cinit[r][q] = rA[ii];
#pragma unroll
      for (int d = 0; d < D; ++d) {
        xr[r][q][d] = x[ii * D + d];
        acc[r][q][d] = part[r][q][d] = 0.0f;
      }
    }
  }
  const int ochi = l16 * NH + (g4 < NH ? g4 : 0), oclo = l16 * 4 * NL + g4, ow = l16 * W;
  struct Ops {
    half8 h, l[NL];
    float w[W];
  };
  auto load = [&](int64_t jt, Ops& o) {
    const half8* ph = chi + jt * NH;
    const half8* pl = clo + jt * 4 * NL;
    const float* pw = bw + jt * W;
    o.h = ph[ochi];
#pragma unroll
    for (int n = 0; n < NL; ++n) o.l[n] = pl[oclo + 4 * n];
#pragma unroll
    for (int c = 0; c < W; ++c) o.w[c] = pw[ow + c];
  };
  auto tile = [&](const Ops& o) {
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      f32x4 e = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[r], o.h, cinit[r], 0, 0, 0);
#pragma unroll
      for (int n = 0; n < NL; ++n) e = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[r][n], o.l[n], e, 0, 0, 0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float kw = exp2_hw(e[q]);
#pragma unroll
        for (int d = 0; d < D; ++d) part[r][q][d] = fmaf(kw, fmaf(o.w[0], xr[r][q][d], o.w[1 + d]), part[r][q][d]);
      }
    }
  };
  const int64_t ntiles = j1 > j0 ? 2 * ((j1 - j0 + 31) / 32) : 0;
  Ops A, B;
  if (ntiles > 0) load(j0, A);
  int tiles = 0;
  for (int64_t t = 0; t < ntiles; t += 2) {
    const int64_t ja = j0 + t * 16;
    load(ja + 16, B);
    tile(A);
    load(t + 2 < ntiles ? ja + 32 : ja, A);
    tile(B);
    tiles += 2;
    if (tiles == kChunkTiles) {
      tiles = 0;
#pragma unroll
      for (int r = 0; r < RT; ++r)
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int d = 0; d < D; ++d) {
            acc[r][q][d] += part[r][q][d];
            part[r][q][d] = 0.0f;
          }
    }
  }
  float* dst = out + split * M * D;
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[D];
#pragma unroll
      for (int d = 0; d < D; ++d) {
        float t = acc[r][q][d] + part[r][q][d];
        t += __shfl_xor(t, 1);
        t += __shfl_xor(t, 2);
        t += __shfl_xor(t, 4);
        t += __shfl_xor(t, 8);
        v[d] = t;
      }
      const int64_t i = base + r * 16 + 4 * g4 + q;
      if (l16 == q && i < M) {
        const float sc = -inv_sigma2 * g[i];
#pragma unroll
        for (int d = 0; d < D; ++d) dst[i * D + d] = sc * v[d];
      }
    }
}

// Sorts kMaxAside indices in LDS ascending (bitonic network; every thread of the workgroup
// takes part).
__device__ void sort_aside(int32_t* list) {
  for (int k = 2; k <= kMaxAside; k <<= 1)
    for (int jstep = k >> 1; jstep > 0; jstep >>= 1) {
      for (int t = threadIdx.x; t < kMaxAside; t += kBlock) {
        const int o = t ^ jstep;
        if (o > t) {
          const bool up = (t & k) == 0;
          const int32_t a = list[t], c = list[o];
          if ((a > c) == up) {
            list[t] = c;
            list[o] = a;
          }
        }
      }
      __syncthreads();
    }
}

// 2^{-c2 |x_i - y_j|^2} from the float64 squared distance of the float32 inputs, rounded to
// float32 before the exponential.
template <int D>
__device__ __forceinline__ double aside_term(const double (&xi)[D], const float* __restrict__ yj, double c2) {
  double d2 = 0.0;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    const double t = xi[d] - (double)yj[d];
    d2 = fma(t, t, d2);
  }
  return (double)exp2_hw((float)(-c2 * d2));
}

// The Gauss sum's last step, after either sweep: the first row_wgs workgroups combine the S
// column splits of their rows in increasing order (S > 1, from partial [S][M][C]; with S = 1 the
// sweep has written out itself) and apply rscale; the kMaxAside workgroups after them handle the
// set-aside rows. When the preparation set points aside (matrix-core path only):
//   - every row that is not set aside gets rscale[i] sum_j 2^{-c2 |x_i - y_j|^2} b[j][c] over the
//     set-aside columns j in increasing order added (terms in float64, then to the float32 sum;
//     each workgroup sorts the recorded indices itself, so the order does not depend on the
//     order in which they were recorded);
//   - each set-aside row is summed by one workgroup over all columns (each thread a fixed
//     stride of columns in float64, then a fixed tree) and written as rscale[i] times that.
template <int D, int C>
__global__ void __launch_bounds__(kBlock)
finish_sum_kernel(const float* __restrict__ partial, float* __restrict__ out, const float* __restrict__ x,
                  const float* __restrict__ y, const float* __restrict__ b, const float* __restrict__ rscale,
                  const int32_t* __restrict__ aside, const MfParams* __restrict__ P, int64_t M, int64_t N,
                  int64_t S, int64_t row_wgs, double c2) {
  __shared__ int32_t rows_l[kMaxAside];
  __shared__ int32_t cols_l[kMaxAside];
  __shared__ double red[C][kBlock];
  const bool robust = P->gate && !P->bad && P->robust;
  const int nr = robust ? (P->nbr < kMaxAside ? P->nbr : kMaxAside) : 0;
  const int nc = robust ? (P->nbc < kMaxAside ? P->nbc : kMaxAside) : 0;
  if ((int64_t)blockIdx.x >= row_wgs) {  // a set-aside row
    const int w = (int)((int64_t)blockIdx.x - row_wgs);
    if (w >= nr) return;
    const int64_t i = aside[w];
    double xi[D], acc[C];
#pragma unroll
    for (int d = 0; d < D; ++d) xi[d] = (double)x[i * D + d];
#pragma unroll
    for (int c = 0; c < C; ++c) acc[c] = 0.0;
    for (int64_t j = threadIdx.x; j < N; j += kBlock) {
      const double k = aside_term<D>(xi, y + j * D, c2);
#pragma unroll
      for (int c = 0; c < C; ++c) acc[c] = fma(k, (double)b[j * C + c], acc[c]);
    }
#pragma unroll
    for (int c = 0; c < C; ++c) red[c][threadIdx.x] = acc[c];
    __syncthreads();
    for (int h = kBlock / 2; h > 0; h >>= 1) {
      if ((int)threadIdx.x < h)
#pragma unroll
        for (int c = 0; c < C; ++c) red[c][threadIdx.x] += red[c][threadIdx.x + h];
      __syncthreads();
    }
    if (threadIdx.x < C) {
      const double sc = rscale ? (double)rscale[i] : 1.0;
      out[i * C + threadIdx.x] = (float)(sc * red[threadIdx.x][0]);
    }
    return;
  }
  if (nr > 0 || nc > 0) {
    for (int t = threadIdx.x; t < kMaxAside; t += kBlock) {
      rows_l[t] = t < nr ? aside[t] : 0x7fffffff;
      cols_l[t] = t < nc ? aside[kMaxAside + t] : 0x7fffffff;
    }
    __syncthreads();
    if (nr > 0) sort_aside(rows_l);
    if (nc > 0) sort_aside(cols_l);
  }
  const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (i >= M) return;
  if (nr > 0) {  // a set-aside row is written by its own workgroup
    int lo = 0, hi = nr;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (rows_l[mid] < i) lo = mid + 1;
      else hi = mid;
    }
    if (lo < nr && rows_l[lo] == i) return;
  }
  float v[C];
  const float sc = rscale ? rscale[i] : 1.0f;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    if (S > 1) {
      float t = 0.0f;
      for (int64_t k = 0; k < S; ++k) t += partial[(k * M + i) * C + c];
      v[c] = rscale ? t * sc : t;
    } else {
      v[c] = out[i * C + c];
    }
  }
  if (nc > 0) {
    double xi[D], acc[C];
#pragma unroll
    for (int d = 0; d < D; ++d) xi[d] = (double)x[i * D + d];
#pragma unroll
    for (int c = 0; c < C; ++c) acc[c] = 0.0;
    for (int e = 0; e < nc; ++e) {
      const int64_t j = cols_l[e];
      const double k = aside_term<D>(xi, y + j * D, c2);
#pragma unroll
      for (int c = 0; c < C; ++c) acc[c] = fma(k, (double)b[j * C + c], acc[c]);
    }
#pragma unroll
    for (int c = 0; c < C; ++c) v[c] += (float)((double)sc * acc[c]);
  }
  if (S > 1 || nc > 0) {
#pragma unroll
    for (int c = 0; c < C; ++c) out[i * C + c] = v[c];
  }
}

// Byte offsets of the operand region: parameters, bounds records, row operands, column
// operands, padded weights.
struct MfLayout {
  int NH, NL;
  int64_t Npad;
  size_t parts, samples, aside, rhi, rlo, rA, chi, clo, bpad, total;
};

// W: floats per padded column record (the weights, and for the gradient also y_j); grad: the
// gradient's two extra low-part products. The sweeps take (NH, NL) = (1, 1) or (2, 2).
MfLayout mf_layout(int64_t M, int64_t N, int D, int W, bool grad = false) {
  MfLayout L;
  const bool narrow = D + 2 <= 8 && 5 * D + 2 + (grad ? 2 : 0) <= 32;
  L.NH = narrow ? 1 : 2;
  L.NL = narrow ? 1 : 2;
  L.Npad = ceil_div(N, 32) * 32;
  size_t off = align_up(sizeof(MfParams));
  L.parts = off;
  off += align_up((size_t)kBoundBlocks * 2 * kMaxLowD * sizeof(unsigned int));
  L.samples = off;
  off += align_up((size_t)kMaxLowD * kMaxAside * sizeof(float));
  L.aside = off;  // set-aside rows, then set-aside columns
  off += align_up((size_t)2 * kMaxAside * sizeof(int32_t));
  L.rhi = off;
  off += align_up((size_t)M * 16 * L.NH);
  L.rlo = off;
  off += align_up((size_t)M * 64 * L.NL);
  L.rA = off;
  off += align_up((size_t)M * sizeof(float));
  L.chi = off;
  off += align_up((size_t)L.Npad * 16 * L.NH);
  L.clo = off;
  off += align_up((size_t)L.Npad * 64 * L.NL);
  L.bpad = off;
  off += align_up((size_t)L.Npad * W * sizeof(float));
  L.total = off;
  return L;
}

template <int C, int RT, int NH, int NL>
hipError_t sweep(char* r, const MfLayout& L, float* dst, const float* rscale, int64_t M, int64_t N, const Plan& p,
                 hipStream_t s) {
  // one launch per 2^30 workgroups (a launch's grid is limited to 2^31 - 1)
  const int64_t pairs = p.mf_row_blocks * p.splits;
  for (int64_t pair0 = 0; pair0 < pairs; pair0 += kMaxLaunch) {
    const int64_t n = pairs - pair0 < kMaxLaunch ? pairs - pair0 : kMaxLaunch;
    gauss_sum_mf_kernel<C, RT, NH, NL><<<(unsigned)n, kBlock, 0, s>>>(
        reinterpret_cast<const half8*>(r + L.rhi), reinterpret_cast<const half8*>(r + L.rlo),
        reinterpret_cast<const float*>(r + L.rA), reinterpret_cast<const half8*>(r + L.chi),
        reinterpret_cast<const half8*>(r + L.clo), reinterpret_cast<const float*>(r + L.bpad), dst, rscale,
        reinterpret_cast<const MfParams*>(r), M, N, p.cols_per_split, p.mf_row_blocks, p.splits, pair0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Row tiles per wave: 4 for C <= 2, 2 for C <= 4, else 1 (register budgets); fewer for few rows.
constexpr int max_rt(int C) { return C <= 2 ? 4 : (C <= 4 ? 2 : 1); }

template <int C, int NH, int NL>
hipError_t sweep_rt(char* r, const MfLayout& L, float* dst, const float* rscale, int64_t M, int64_t N, const Plan& p,
                    hipStream_t s) {
  if constexpr (max_rt(C) >= 4)
    if (p.mf_rt == 4) return sweep<C, 4, NH, NL>(r, L, dst, rscale, M, N, p, s);
  if constexpr (max_rt(C) >= 2)
    if (p.mf_rt == 2) return sweep<C, 2, NH, NL>(r, L, dst, rscale, M, N, p, s);
  if (p.mf_rt == 1) return sweep<C, 1, NH, NL>(r, L, dst, rscale, M, N, p, s);
  return hipErrorInvalidValue;
}

template <int C, int RT, int NH, int NL>
int occupancy_of() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gauss_sum_mf_kernel<C, RT, NH, NL>, kBlock, 0) != hipSuccess ||
      n < 1)
    n = 4;
  return n;
}

template <int C, int NH, int NL>
int occupancy_rt(int rt) {
  if constexpr (max_rt(C) >= 4)
    if (rt == 4) return occupancy_of<C, 4, NH, NL>();
  if constexpr (max_rt(C) >= 2)
    if (rt == 2) return occupancy_of<C, 2, NH, NL>();
  return occupancy_of<C, 1, NH, NL>();
}

template <int C>
int occupancy_c(bool wide, int rt) {
  return wide ? occupancy_rt<C, 2, 2>(rt) : occupancy_rt<C, 1, 1>(rt);
}

template <int C>
hipError_t sweep_c(char* r, const MfLayout& L, float* dst, const float* rscale, int64_t M, int64_t N, const Plan& p,
                   hipStream_t s) {
  if (L.NH == 1 && L.NL == 1) return sweep_rt<C, 1, 1>(r, L, dst, rscale, M, N, p, s);
  return sweep_rt<C, 2, 2>(r, L, dst, rscale, M, N, p, s);
}

// The 32 x 32 form: RT32 tiles of 32 rows per wave, i.e. rt / 2 in units of 16 rows.
template <int RT32, int C>
hipError_t sweep32(char* r, const MfLayout& L, float* dst, const float* rscale, int64_t M, int64_t N, const Plan& p,
                   hipStream_t s) {
  const int64_t pairs = p.mf_row_blocks * p.splits;
  for (int64_t pair0 = 0; pair0 < pairs; pair0 += kMaxLaunch) {
    const int64_t n = pairs - pair0 < kMaxLaunch ? pairs - pair0 : kMaxLaunch;
    gauss_sum_mf32_kernel<RT32, C><<<(unsigned)n, kBlock, 0, s>>>(
        reinterpret_cast<const half8*>(r + L.rhi), reinterpret_cast<const half8*>(r + L.rlo),
        reinterpret_cast<const float*>(r + L.rA), reinterpret_cast<const half8*>(r + L.chi),
        reinterpret_cast<const half8*>(r + L.clo), reinterpret_cast<const float*>(r + L.bpad), dst, rscale,
        reinterpret_cast<const MfParams*>(r), M, N, p.cols_per_split, p.mf_row_blocks, p.splits, pair0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int RT32>
hipError_t sweep32_lse(char* r, const MfLayout& L, float* out, LsePartial* part, int64_t M, int64_t N, const Plan& p,
                       hipStream_t s) {
  const int64_t pairs = p.mf_row_blocks * p.splits;
  for (int64_t pair0 = 0; pair0 < pairs; pair0 += kMaxLaunch) {
    const int64_t n = pairs - pair0 < kMaxLaunch ? pairs - pair0 : kMaxLaunch;
    lse_mf32_kernel<RT32><<<(unsigned)n, kBlock, 0, s>>>(
        reinterpret_cast<const half8*>(r + L.rhi), reinterpret_cast<const half8*>(r + L.rlo),
        reinterpret_cast<const float*>(r + L.rA), reinterpret_cast<const half8*>(r + L.chi),
        reinterpret_cast<const half8*>(r + L.clo), out, part, reinterpret_cast<const MfParams*>(r), M, N,
        p.cols_per_split, p.mf_row_blocks, p.splits, pair0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int RT32>
int occupancy32_lse() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, lse_mf32_kernel<RT32>, kBlock, 0) != hipSuccess || n < 1) n = 4;
  return n;
}

template <int RT32, int C>
int occupancy32() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gauss_sum_mf32_kernel<RT32, C>, kBlock, 0) != hipSuccess || n < 1)
    n = 4;
  return n;
}

template <int RT, int NH, int NL>
hipError_t sweep_lse(char* r, const MfLayout& L, float* out, LsePartial* part, int64_t M, int64_t N, const Plan& p,
                     hipStream_t s) {
  const int64_t pairs = p.mf_row_blocks * p.splits;
  for (int64_t pair0 = 0; pair0 < pairs; pair0 += kMaxLaunch) {
    const int64_t n = pairs - pair0 < kMaxLaunch ? pairs - pair0 : kMaxLaunch;
    lse_mf_kernel<RT, NH, NL><<<(unsigned)n, kBlock, 0, s>>>(
        reinterpret_cast<const half8*>(r + L.rhi), reinterpret_cast<const half8*>(r + L.rlo),
        reinterpret_cast<const float*>(r + L.rA), reinterpret_cast<const half8*>(r + L.chi),
        reinterpret_cast<const half8*>(r + L.clo), out, part, reinterpret_cast<const MfParams*>(r), M, N,
        p.cols_per_split, p.mf_row_blocks, p.splits, pair0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int NH, int NL>
hipError_t sweep_lse_rt(char* r, const MfLayout& L, float* out, LsePartial* part, int64_t M, int64_t N,
                        const Plan& p, hipStream_t s) {
  switch (p.mf_rt) {
    case 4: return sweep_lse<4, NH, NL>(r, L, out, part, M, N, p, s);
    case 2: return sweep_lse<2, NH, NL>(r, L, out, part, M, N, p, s);
    case 1: return sweep_lse<1, NH, NL>(r, L, out, part, M, N, p, s);
  }
  return hipErrorInvalidValue;
}

template <int RT, int NH, int NL>
int occupancy_lse() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, lse_mf_kernel<RT, NH, NL>, kBlock, 0) != hipSuccess || n < 1)
    n = 4;
  return n;
}

// Row tiles per wave of the gradient sweep: the per-row coordinates and accumulators take
// 12 D registers per tile.
constexpr int grad_rt(int D) { return D <= 4 ? 2 : 1; }

template <int D>
hipError_t sweep_grad(char* r, const MfLayout& L, const float* x, const float* g, float* dst, float inv_sigma2,
                      int64_t M, int64_t N, const Plan& p, hipStream_t s) {
  const int64_t pairs = p.mf_row_blocks * p.splits;
  for (int64_t pair0 = 0; pair0 < pairs; pair0 += kMaxLaunch) {
    const int64_t n = pairs - pair0 < kMaxLaunch ? pairs - pair0 : kMaxLaunch;
#define KEOPS_MF_GRAD_LAUNCH(NHv)                                                                            \
  grad_mf_kernel<D, grad_rt(D), NHv, NHv><<<(unsigned)n, kBlock, 0, s>>>(                                    \
      reinterpret_cast<const half8*>(r + L.rhi), reinterpret_cast<const half8*>(r + L.rlo),                   \
      reinterpret_cast<const float*>(r + L.rA), reinterpret_cast<const half8*>(r + L.chi),                    \
      reinterpret_cast<const half8*>(r + L.clo), reinterpret_cast<const float*>(r + L.bpad), x, g, dst,       \
      inv_sigma2, reinterpret_cast<const MfParams*>(r), M, N, p.cols_per_split, p.mf_row_blocks, p.splits, pair0)
    if (L.NH == 1 && L.NL == 1)
      KEOPS_MF_GRAD_LAUNCH(1);
    else
      KEOPS_MF_GRAD_LAUNCH(2);
#undef KEOPS_MF_GRAD_LAUNCH
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int D>
int occupancy_grad(bool wide) {
  int n = 0;
  const hipError_t e = wide ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, grad_mf_kernel<D, grad_rt(D), 2, 2>,
                                                                            kBlock, 0)
                            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, grad_mf_kernel<D, grad_rt(D), 1, 1>,
                                                                            kBlock, 0);
  return (e != hipSuccess || n < 1) ? 4 : n;
}

}  // namespace
}  // namespace lowd

size_t mf_region_bytes(int64_t M, int64_t N, int D, int W, bool grad) {
  return lowd::mf_layout(M, N, D, W, grad).total;
}

const int* mf_decision(const void* region) { return &static_cast<const lowd::MfParams*>(region)->gate; }

bool mf_sum_square(int D, int C, int rt) {
  return D >= 1 && D <= 3 && ((C == 1 && (rt == 2 || rt == 4)) || (C >= 2 && C <= 4 && rt == 2));
}
bool mf_lse_square(int D, int rt) { return D >= 1 && D <= 3 && (rt == 2 || rt == 4); }

int mf_rows_per_lane(int op, int D, int C) {
  if (op == 3) return lowd::grad_rt(D);
  if (op == 0 && D <= 3 && C >= 2 && C <= 4) return 2;  // one 32-row tile of the 32 x 32 form
  return lowd::max_rt(op == 1 ? 0 : C);
}

int mf_occupancy(int op, int D, int C, int rt) {
  // resident workgroups per CU of the sweep instance, from its register use (cached per
  // instance; 4 when the runtime cannot say)
  static std::atomic<int> cache[2][kMaxLowC + 1][5];
  static std::atomic<int> cache_grad[kMaxLowD + 1];
  const int wide = lowd::mf_layout(1, 1, D, 1, op == 3).NH == 2 ? 1 : 0;
  int dev = 0;
  if (op == 1) C = 0;  // the log-sum-exp sweep
  if (D < 1 || D > kMaxLowD || C < 0 || C > kMaxLowC || (rt != 1 && rt != 2 && rt != 4) ||
      hipGetDevice(&dev) != hipSuccess)
    return 4;
  if (op == 3) {
    int n = cache_grad[D].load(std::memory_order_relaxed);
    if (n > 0) return n;
#define KEOPS_MF_OG(Dv) n = lowd::occupancy_grad<Dv>(wide != 0)
    switch (D) {
      case 1: KEOPS_MF_OG(1); break;
      case 2: KEOPS_MF_OG(2); break;
      case 3: KEOPS_MF_OG(3); break;
      case 4: KEOPS_MF_OG(4); break;
      case 5: KEOPS_MF_OG(5); break;
      case 6: KEOPS_MF_OG(6); break;
      case 7: KEOPS_MF_OG(7); break;
      case 8: KEOPS_MF_OG(8); break;
    }
#undef KEOPS_MF_OG
    cache_grad[D].store(n, std::memory_order_relaxed);
    return n;
  }
  if ((op == 0 && mf_sum_square(D, C, rt)) || (op == 1 && mf_lse_square(D, rt))) {
    static std::atomic<int> cache32[2][5][5];
    const int cc = op == 0 ? C : 0;
    int n = cache32[op][rt][cc].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (op == 0)
      n = C == 1 ? (rt == 4 ? lowd::occupancy32<2, 1>() : lowd::occupancy32<1, 1>())
                 : (C == 2 ? lowd::occupancy32<1, 2>() : (C == 3 ? lowd::occupancy32<1, 3>() : lowd::occupancy32<1, 4>()));
    else n = rt == 4 ? lowd::occupancy32_lse<2>() : lowd::occupancy32_lse<1>();
    cache32[op][rt][cc].store(n, std::memory_order_relaxed);
    return n;
  }
  std::atomic<int>& slot = cache[wide][C][rt];
  int n = slot.load(std::memory_order_relaxed);
  if (n > 0) return n;
  auto query = [&]() -> int {
    if (C == 0) {
      if (rt == 4) return wide ? lowd::occupancy_lse<4, 2, 2>() : lowd::occupancy_lse<4, 1, 1>();
      if (rt == 2) return wide ? lowd::occupancy_lse<2, 2, 2>() : lowd::occupancy_lse<2, 1, 1>();
      return wide ? lowd::occupancy_lse<1, 2, 2>() : lowd::occupancy_lse<1, 1, 1>();
    }
#define KEOPS_MF_OCC(Cv) lowd::occupancy_c<Cv>(wide != 0, rt)
    switch (C) {
      case 1: return KEOPS_MF_OCC(1);
      case 2: return KEOPS_MF_OCC(2);
      case 3: return KEOPS_MF_OCC(3);
      case 4: return KEOPS_MF_OCC(4);
      case 5: return KEOPS_MF_OCC(5);
      case 6: return KEOPS_MF_OCC(6);
      case 7: return KEOPS_MF_OCC(7);
      case 8: return KEOPS_MF_OCC(8);
    }
#undef KEOPS_MF_OCC
    return 4;
  };
  n = query();
  slot.store(n, std::memory_order_relaxed);
  return n;
}

hipError_t launch_mf_prepare(const float* x, const float* y, const float* b, bool with_y, double* cols, void* region,
                             int64_t M, int64_t N, int D, int C, double c2, hipStream_t s, bool set_aside, bool square) {
  using namespace lowd;
  char* r = static_cast<char*>(region);
  const MfLayout L = mf_layout(M, N, D, C + (with_y ? D : 0), with_y);
  MfParams* P = reinterpret_cast<MfParams*>(r);
  unsigned int* parts = reinterpret_cast<unsigned int*>(r + L.parts);
  float* samples = reinterpret_cast<float*>(r + L.samples);
  int32_t* aside = reinterpret_cast<int32_t*>(r + L.aside);
  const int64_t n = M > N ? M : N;
  int64_t nb = ceil_div(n, kBlock);
  if (nb > kBoundBlocks) nb = kBoundBlocks;
  const int spw = kMaxAside / (int)nb;  // samples per bounds workgroup (nb <= kMaxAside)
  mf_bounds_kernel<<<(unsigned)nb, kBlock, 0, s>>>(x, y, M, N, D, parts, samples, spw, P);
  const int64_t rb = ceil_div(M, kBlock), cb = ceil_div(L.Npad, kBlock);
  half8* rhi = reinterpret_cast<half8*>(r + L.rhi);
  half8* rlo = reinterpret_cast<half8*>(r + L.rlo);
  float* rA = reinterpret_cast<float*>(r + L.rA);
  half8* chi = reinterpret_cast<half8*>(r + L.chi);
  half8* clo = reinterpret_cast<half8*>(r + L.clo);
  float* bpad = reinterpret_cast<float*>(r + L.bpad);
  const int sq = (square && L.NH == 1 && L.NL == 1 && !with_y && D <= 3) ? 1 : 0;
  if (L.NH == 1 && L.NL == 1)
    mf_prep_kernel<1, 1><<<(unsigned)(rb + cb), kBlock, 0, s>>>(
        x, y, b, C, with_y ? 1 : 0, cols, rhi, rlo, rA, chi, clo, bpad, parts, samples, (int)nb * spw, (int)nb, M, N, L.Npad, D, c2, rb,
        set_aside ? 1 : 0, sq, aside, aside + kMaxAside, P);
  else
    mf_prep_kernel<2, 2><<<(unsigned)(rb + cb), kBlock, 0, s>>>(
        x, y, b, C, with_y ? 1 : 0, cols, rhi, rlo, rA, chi, clo, bpad, parts, samples, (int)nb * spw, (int)nb, M, N, L.Npad, D, c2, rb,
        set_aside ? 1 : 0, 0, aside, aside + kMaxAside, P);
  return hipGetLastError();
}

hipError_t launch_mf_finish(const float* partial, float* out, const float* x, const float* y, const float* b,
                            const float* rscale, void* region, int64_t M, int64_t N, int D, int C, int64_t S,
                            double c2, hipStream_t s) {
  using namespace lowd;
  char* r = static_cast<char*>(region);
  const MfLayout L = mf_layout(M, N, D, C);
  const MfParams* P = reinterpret_cast<const MfParams*>(r);
  const int32_t* aside = reinterpret_cast<const int32_t*>(r + L.aside);
  const int64_t row_wgs = ceil_div(M, kBlock);
  auto run = [&](auto dt, auto ct) -> hipError_t {
    constexpr int Dv = decltype(dt)::value, Cv = decltype(ct)::value;
    finish_sum_kernel<Dv, Cv><<<(unsigned)(row_wgs + kMaxAside), kBlock, 0, s>>>(partial, out, x, y, b, rscale, aside,
                                                                               P, M, N, S, row_wgs, c2);
    return hipGetLastError();
  };
#define KEOPS_FIN_C(Dv, Cv) return run(std::integral_constant<int, Dv>{}, std::integral_constant<int, Cv>{})
#define KEOPS_FIN_D(Dv)                  \
  switch (C) {                           \
    case 1: KEOPS_FIN_C(Dv, 1);          \
    case 2: KEOPS_FIN_C(Dv, 2);          \
    case 3: KEOPS_FIN_C(Dv, 3);          \
    case 4: KEOPS_FIN_C(Dv, 4);          \
    case 5: KEOPS_FIN_C(Dv, 5);          \
    case 6: KEOPS_FIN_C(Dv, 6);          \
    case 7: KEOPS_FIN_C(Dv, 7);          \
    case 8: KEOPS_FIN_C(Dv, 8);          \
  }                                      \
  return hipErrorInvalidValue;
  switch (D) {
    case 1: KEOPS_FIN_D(1)
    case 2: KEOPS_FIN_D(2)
    case 3: KEOPS_FIN_D(3)
    case 4: KEOPS_FIN_D(4)
    case 5: KEOPS_FIN_D(5)
    case 6: KEOPS_FIN_D(6)
    case 7: KEOPS_FIN_D(7)
    case 8: KEOPS_FIN_D(8)
  }
#undef KEOPS_FIN_D
#undef KEOPS_FIN_C
  return hipErrorInvalidValue;
}

hipError_t launch_mf_lse(float* out, void* partial, void* region, int64_t M, int64_t N, int D, const Plan& p,
                         hipStream_t s) {
  using namespace lowd;
  char* r = static_cast<char*>(region);
  const MfLayout L = mf_layout(M, N, D, 0);
  LsePartial* part = static_cast<LsePartial*>(partial);
  if (mf_lse_square(D, p.mf_rt))
    return p.mf_rt == 4 ? sweep32_lse<2>(r, L, out, part, M, N, p, s) : sweep32_lse<1>(r, L, out, part, M, N, p, s);
  if (L.NH == 1 && L.NL == 1) return sweep_lse_rt<1, 1>(r, L, out, part, M, N, p, s);
  return sweep_lse_rt<2, 2>(r, L, out, part, M, N, p, s);
}

hipError_t launch_mf_lse_fix(const float* x, const float* y, float* out, void* region, int64_t M, int64_t N, int D,
                             double c2, const Plan& p, hipStream_t s) {
  using namespace lowd;
  if (!mf_lse_square(D, p.mf_rt) || M <= 0) return hipSuccess;
  const MfParams* P = static_cast<const MfParams*>(region);
  const unsigned nb = (unsigned)ceil_div(M, kBlock);
  switch (D) {
    case 1: lse_fix_kernel<1><<<nb, kBlock, 0, s>>>(x, y, out, P, M, N, c2); break;
    case 2: lse_fix_kernel<2><<<nb, kBlock, 0, s>>>(x, y, out, P, M, N, c2); break;
    case 3: lse_fix_kernel<3><<<nb, kBlock, 0, s>>>(x, y, out, P, M, N, c2); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_mf_grad(const float* x, const float* g, float* dst, float inv_sigma2, void* region, int64_t M,
                          int64_t N, int D, const Plan& p, hipStream_t s) {
  using namespace lowd;
  char* r = static_cast<char*>(region);
  const MfLayout L = mf_layout(M, N, D, 1 + D, true);
#define KEOPS_MF_G(Dv) sweep_grad<Dv>(r, L, x, g, dst, inv_sigma2, M, N, p, s)
  KEOPS_SWITCH_D(D, KEOPS_MF_G)
#undef KEOPS_MF_G
}

hipError_t launch_mf_sum(const float* rscale, float* dst, void* region, int64_t M, int64_t N, int D, int C,
                         const Plan& p, hipStream_t s) {
  using namespace lowd;
  char* r = static_cast<char*>(region);
  const MfLayout L = mf_layout(M, N, D, C);
  if (mf_sum_square(D, C, p.mf_rt)) {
    switch (C) {
      case 1: return p.mf_rt == 4 ? sweep32<2, 1>(r, L, dst, rscale, M, N, p, s) : sweep32<1, 1>(r, L, dst, rscale, M, N, p, s);
      case 2: return sweep32<1, 2>(r, L, dst, rscale, M, N, p, s);
      case 3: return sweep32<1, 3>(r, L, dst, rscale, M, N, p, s);
      case 4: return sweep32<1, 4>(r, L, dst, rscale, M, N, p, s);
    }
  }
#define KEOPS_MF_C(Cv) sweep_c<Cv>(r, L, dst, rscale, M, N, p, s)
  KEOPS_SWITCH_C(C, KEOPS_MF_C)
#undef KEOPS_MF_C
}

}  // namespace keops
