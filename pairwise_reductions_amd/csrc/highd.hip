// Host side of the matrix-core (fp16) batched Gauss sums: column and row preparation
// kernels, launch plans and the launchers declared in internal.h. The sweeps themselves live
// in highd_fwd.h and highd_grad.h and are compiled once per padded feature width
// (highd_d32.hip ... highd_d128.hip).
//
// Column preparation, general form. For a column weight vector w_j (the values b_j times an
// optional per-column scale c_j, read as fp16 or fp32) with norm n_j = |w_j|_2 and the batch
// maximum n_max, the sweep sees
//   beta_j = -|k_j|^2/2 + log2(n_j / n_max) / cs      (the log clamped below at kLogFloor),
//   w'_j   = w_j / n_j   (fp16, unit norm),
// and the output is multiplied back by n_max. Since n_j / n_max <= 1 the tracked exponent is
// still never positive, so the sweep's settled-row rule holds, and no fp16 value can
// overflow whatever the magnitude of the weights. The fast path (fp16 weights, no scales)
// copies the weights unchanged.
#include "highd_common.h"

#include <math.h>

namespace keops {
namespace {

using hd::hd_ceil_div;
using hd::key_slot;

template <typename T>
__device__ inline float to_f32(T v) { return (float)v; }

// Fast path: beta_j = -|k_j|^2/2 (-inf past N); vp[t][j/32][c][key_slot(j%32)] = v[t][j][c]
// for c < C, zero for padded keys and for the padding channels C <= c < Cp.
__global__ void __launch_bounds__(256)
fwd_prep_kernel(const _Float16* __restrict__ k, const _Float16* __restrict__ v, float* __restrict__ beta,
                _Float16* __restrict__ vp, int64_t N, int64_t Npad, int D, int C, int Cp) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t = blockIdx.y;
  if (j >= Npad) return;
  const _Float16* kr = k + (t * N + j) * D;
  const _Float16* vr = v + (t * N + j) * C;
  float s = 0.0f;
  if (j < N) {
    for (int d = 0; d < D; ++d) {
      const float kv = (float)kr[d];
      s = fmaf(kv, kv, s);
    }
  }
  beta[t * Npad + j] = (j < N) ? -0.5f * s : -INFINITY;
  _Float16* dst = vp + (t * Npad + (j / 32) * 32) * Cp + key_slot((int)(j % 32));
  for (int c = 0; c < Cp; ++c) dst[(int64_t)c * 32] = (j < N && c < C) ? vr[c] : (_Float16)0.0f;
}

// |c_j w_j|_2 of column j of batch t (c = 1 when cscale is null).
template <typename T>
__device__ inline float weight_norm(const T* __restrict__ w, const float* __restrict__ cscale, int64_t t, int64_t j,
                                    int64_t N, int C) {
  const T* wr = w + (t * N + j) * C;
  float s = 0.0f;
  for (int c = 0; c < C; ++c) {
    const float v = to_f32(wr[c]);
    s = fmaf(v, v, s);
  }
  const float sc = cscale ? fabsf(cscale[t * N + j]) : 1.0f;
  return sc * sqrtf(s);
}

// nmax[t] = max_j |c_j w_j|_2. nmax must hold +0 before the launch (float bits of
// non-negative values order like unsigned integers, so an integer max gives the float max).
template <typename T>
__global__ void __launch_bounds__(256)
weight_norm_max_kernel(const T* __restrict__ w, const float* __restrict__ cscale, int64_t N, int C,
                       float* __restrict__ nmax) {
  __shared__ float red[256];
  const int64_t t = blockIdx.y;
  float m = 0.0f;
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < N; j += (int64_t)gridDim.x * 256)
    m = fmaxf(m, weight_norm(w, cscale, t, j, N, C));
  red[threadIdx.x] = m;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + h]);
    __syncthreads();
  }
  if (threadIdx.x == 0) atomicMax(reinterpret_cast<unsigned int*>(nmax + t), __float_as_uint(red[0]));
}

// General column preparation (see the file comment). kGrad selects the table layout:
//   forward:  wp[t][j/32][c][key_slot(j%32)] for c < Cw (key-permuted, the A operand of O^T)
//   gradient: wp[t][j][c] for c < Cw (row-major, the A operand of dP^T), plus
//             yp[t][j/32][ch][key_slot(j%32)] = k[t][j][ch] for ch < D, 1 at ch = Dp, else 0.
template <typename T, bool kGrad>
__global__ void __launch_bounds__(256)
col_prep_kernel(const _Float16* __restrict__ k, const T* __restrict__ w, const float* __restrict__ cscale,
                const float* __restrict__ nmax, float* __restrict__ beta, _Float16* __restrict__ wp,
                _Float16* __restrict__ yp, int64_t N, int64_t Npad, int D, int Dp, int C, int Cw, float cs) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t = blockIdx.y;
  if (j >= Npad) return;
  const bool live = j < N;
  const _Float16* kr = k + (t * N + j) * D;
  const T* wr = w + (t * N + j) * C;
  float bj = -INFINITY, inv = 0.0f, sc = 1.0f;
  if (live) {
    float s = 0.0f;
    for (int d = 0; d < D; ++d) {
      const float kv = (float)kr[d];
      s = fmaf(kv, kv, s);
    }
    const float n = weight_norm(w, cscale, t, j, N, C);
    const float nm = nmax[t];
    const float ratio = nm > 0.0f ? n / nm : 0.0f;
    const float lw = fmaxf(log2f(ratio), hd::kLogFloor);
    bj = -0.5f * s + lw / cs;
    inv = n > 0.0f ? 1.0f / n : 0.0f;
    sc = cscale ? cscale[t * N + j] : 1.0f;
  }
  beta[t * Npad + j] = bj;
  if constexpr (kGrad) {
    _Float16* dst = wp + (t * Npad + j) * Cw;
    for (int c = 0; c < Cw; ++c) dst[c] = (live && c < C) ? (_Float16)(to_f32(wr[c]) * sc * inv) : (_Float16)0.0f;
    const int YC = Dp + 16;
    _Float16* yd = yp + (t * Npad + (j / 32) * 32) * YC + key_slot((int)(j % 32));
    for (int ch = 0; ch < YC; ++ch) {
      _Float16 v = (_Float16)0.0f;
      if (live && ch < D) v = kr[ch];
      if (live && ch == Dp) v = (_Float16)1.0f;
      yd[(int64_t)ch * 32] = v;
    }
  } else {
    _Float16* dst = wp + (t * Npad + (j / 32) * 32) * Cw + key_slot((int)(j % 32));
    for (int c = 0; c < Cw; ++c)
      dst[(int64_t)c * 32] = (live && c < C) ? (_Float16)(to_f32(wr[c]) * sc * inv) : (_Float16)0.0f;
  }
}

// Row weights of the gradient sweep: ap[t][i][c] = a_i[c] / |a_i| (zero past C), rho = |a_i|.
template <typename T>
__global__ void __launch_bounds__(256)
row_prep_kernel(const T* __restrict__ a, _Float16* __restrict__ ap, float* __restrict__ rho, int64_t M, int C,
                int Ck) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t t = blockIdx.y;
  if (i >= M) return;
  const T* ar = a + (t * M + i) * C;
  float s = 0.0f;
  for (int c = 0; c < C; ++c) {
    const float v = to_f32(ar[c]);
    s = fmaf(v, v, s);
  }
  const float n = sqrtf(s);
  const float inv = n > 0.0f ? 1.0f / n : 0.0f;
  rho[t * M + i] = n;
  _Float16* dst = ap + (t * M + i) * Ck;
  for (int c = 0; c < Ck; ++c) dst[c] = c < C ? (_Float16)(to_f32(ar[c]) * inv) : (_Float16)0.0f;
}

__global__ void __launch_bounds__(256)
combine_kernel(const float* __restrict__ partial, float* __restrict__ out, int64_t n, int64_t S) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  for (int64_t k = 0; k < S; ++k) s += partial[k * n + i];
  out[i] = s;
}

// ---- plans --------------------------------------------------------------------------------
struct Split {
  int64_t Npad, row_blocks, splits, kps;
};

// Column splits: enough workgroups for kSplitTarget per CU, each split >= 4 * kKeyPad keys and
// a multiple of kKeyPad (so split boundaries fall on stage boundaries).
Split plan_split(int64_t B, int64_t M, int64_t N, int rows_per_block, int num_cus) {
  Split p;
  p.Npad = hd::padded_keys(N);
  p.row_blocks = hd_ceil_div(M, rows_per_block);
  const int64_t blocks = p.row_blocks * B;
  const int64_t target = (int64_t)num_cus * hd::kSplitTarget;
  int64_t S = blocks < target ? hd_ceil_div(target, blocks) : 1;
  const int64_t max_split = p.Npad / (4 * hd::kKeyPad) > 1 ? p.Npad / (4 * hd::kKeyPad) : 1;
  if (S > max_split) S = max_split;
  const int64_t kps = hd_ceil_div(hd_ceil_div(N, S), hd::kKeyPad) * hd::kKeyPad;
  p.splits = hd_ceil_div(N, kps);
  p.kps = kps;
  return p;
}

// Workspace carving: sections in order, each aligned to kAlign.
struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t at = off;
    off += align_up(bytes);
    return at;
  }
};

struct FwdLayout {
  Split sp;
  size_t nmax, beta, vp, part, total;
};

FwdLayout fwd_layout(int64_t B, int64_t M, int64_t N, int D, int C, bool general, int num_cus) {
  FwdLayout L;
  const int Cp = hd::padded_channels(C);
  L.sp = plan_split(B, M, N, hd::kWaves * hd::fwd_query_tiles(hd::padded_features(D), Cp) * 16, num_cus);
  Carve c;
  L.nmax = c.take(general ? (size_t)B * sizeof(float) : 0);
  L.beta = c.take((size_t)B * L.sp.Npad * sizeof(float));
  L.vp = c.take((size_t)B * L.sp.Npad * Cp * sizeof(_Float16));
  L.part = c.take(L.sp.splits > 1 ? (size_t)L.sp.splits * B * M * C * sizeof(float) : 0);
  L.total = c.off;
  return L;
}

struct GradLayout {
  Split sp;
  size_t nmax, beta, bvp, yp, ap, rho, part, total;
};

GradLayout grad_layout(int64_t B, int64_t M, int64_t N, int D, int C, int num_cus) {
  GradLayout L;
  const int Dp = hd::padded_features(D), Ck = hd::padded_k_channels(C);
  L.sp = plan_split(B, M, N, hd::kWaves * hd::grad_query_tiles(Dp) * 16, num_cus);
  Carve c;
  L.nmax = c.take((size_t)B * sizeof(float));
  L.beta = c.take((size_t)B * L.sp.Npad * sizeof(float));
  L.bvp = c.take((size_t)B * L.sp.Npad * Ck * sizeof(_Float16));
  L.yp = c.take((size_t)B * L.sp.Npad * (Dp + 16) * sizeof(_Float16));
  L.ap = c.take((size_t)B * M * Ck * sizeof(_Float16));
  L.rho = c.take((size_t)B * M * sizeof(float));
  L.part = c.take(L.sp.splits > 1 ? (size_t)L.sp.splits * B * M * D * sizeof(float) : 0);
  L.total = c.off;
  return L;
}

float cs_of(float sigma) {
  const double s = (double)sigma;
  return (float)(1.4426950408889634 / (s * s));  // tau log2(e)
}

hipError_t fwd_dispatch(const hd::FwdArgs& a) {
  switch (hd::padded_features(a.D)) {
    case 32: return hd::fwd_launch<32>(a);
    case 64: return hd::fwd_launch<64>(a);
    case 96: return hd::fwd_launch<96>(a);
    case 128: return hd::fwd_launch<128>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t grad_dispatch(const hd::GradArgs& a) {
  switch (hd::padded_features(a.D)) {
    case 32: return hd::grad_launch<32>(a);
    case 64: return hd::grad_launch<64>(a);
    case 96: return hd::grad_launch<96>(a);
    case 128: return hd::grad_launch<128>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t combine(const float* part, float* out, int64_t n, int64_t S, hipStream_t s) {
  combine_kernel<<<(unsigned)hd_ceil_div(n, 256), 256, 0, s>>>(part, out, n, S);
  return hipGetLastError();
}

// nmax[t] = max_j |c_j w_j| for every batch t.
template <typename T>
hipError_t weight_norm_max(const T* w, const float* cscale, float* nmax, int64_t B, int64_t N, int C, hipStream_t s) {
  hipError_t e = launch_fill(nmax, B, 0.0f, s);
  if (e != hipSuccess) return e;
  int64_t blocks = hd_ceil_div(N, 256);
  if (blocks > 256) blocks = 256;
  weight_norm_max_kernel<T><<<dim3((unsigned)blocks, (unsigned)B), 256, 0, s>>>(w, cscale, N, C, nmax);
  return hipGetLastError();
}

}  // namespace

bool highd_supported(int D, int C) { return D >= 16 && D <= 128 && D % 16 == 0 && C >= 1 && C <= 64; }

size_t highd_workspace_bytes(int64_t B, int64_t M, int64_t N, int D, int C, bool general) {
  if (B == 0 || M == 0 || N == 0) return 0;
  return fwd_layout(B, M, N, D, C, general, device_cus()).total;
}

size_t highd_grad_workspace_bytes(int64_t B, int64_t M, int64_t N, int D, int C) {
  if (B == 0 || M == 0 || N == 0) return 0;
  return grad_layout(B, M, N, D, C, device_cus()).total;
}

hipError_t launch_gauss_sum_highd(const void* x, const void* y, const void* b, bool b_f32, const float* rscale,
                                  const float* cscale, float* out, void* workspace, int64_t B, int64_t M, int64_t N,
                                  int D, int C, float sigma, hipStream_t s) {
  const bool general = b_f32 || cscale != nullptr;
  const FwdLayout L = fwd_layout(B, M, N, D, C, general, device_cus());
  char* ws = static_cast<char*>(workspace);
  float* nmax = reinterpret_cast<float*>(ws + L.nmax);
  float* beta = reinterpret_cast<float*>(ws + L.beta);
  _Float16* vp = reinterpret_cast<_Float16*>(ws + L.vp);
  float* part = reinterpret_cast<float*>(ws + L.part);
  const _Float16* k = static_cast<const _Float16*>(y);
  const float cs = cs_of(sigma);
  const int Cp = hd::padded_channels(C);
  const dim3 pgrid((unsigned)hd_ceil_div(L.sp.Npad, 256), (unsigned)B);
  hipError_t e;
  if (!general) {
    fwd_prep_kernel<<<pgrid, 256, 0, s>>>(k, static_cast<const _Float16*>(b), beta, vp, N, L.sp.Npad, D, C, Cp);
    e = hipGetLastError();
  } else if (b_f32) {
    const float* w = static_cast<const float*>(b);
    e = weight_norm_max(w, cscale, nmax, B, N, C, s);
    if (e != hipSuccess) return e;
    col_prep_kernel<float, false><<<pgrid, 256, 0, s>>>(k, w, cscale, nmax, beta, vp, nullptr, N, L.sp.Npad, D, 0, C,
                                                        Cp, cs);
    e = hipGetLastError();
  } else {
    const _Float16* w = static_cast<const _Float16*>(b);
    e = weight_norm_max(w, cscale, nmax, B, N, C, s);
    if (e != hipSuccess) return e;
    col_prep_kernel<_Float16, false><<<pgrid, 256, 0, s>>>(k, w, cscale, nmax, beta, vp, nullptr, N, L.sp.Npad, D, 0,
                                                           C, Cp, cs);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  hd::FwdArgs a;
  a.q = static_cast<const _Float16*>(x);
  a.k = k;
  a.beta = beta;
  a.vp = vp;
  a.out = L.sp.splits > 1 ? part : out;
  a.rscale = rscale;
  a.oscale = general ? nmax : nullptr;
  a.M = M;
  a.N = N;
  a.Npad = L.sp.Npad;
  a.kps = L.sp.kps;
  a.cs = cs;
  a.D = D;
  a.C = C;
  a.grid = dim3((unsigned)L.sp.row_blocks, (unsigned)L.sp.splits, (unsigned)B);
  a.stream = s;
  e = fwd_dispatch(a);
  if (e != hipSuccess || L.sp.splits == 1) return e;
  return combine(part, out, B * M * C, L.sp.splits, s);
}

hipError_t launch_gauss_sum_grad_highd(const void* x, const void* y, const void* a, bool a_f32, const void* bv,
                                       bool bv_f32, float* out, void* workspace, int64_t B, int64_t M, int64_t N,
                                       int D, int C, float sigma, hipStream_t s) {
  const GradLayout L = grad_layout(B, M, N, D, C, device_cus());
  char* ws = static_cast<char*>(workspace);
  float* nmax = reinterpret_cast<float*>(ws + L.nmax);
  float* beta = reinterpret_cast<float*>(ws + L.beta);
  _Float16* bvp = reinterpret_cast<_Float16*>(ws + L.bvp);
  _Float16* yp = reinterpret_cast<_Float16*>(ws + L.yp);
  _Float16* ap = reinterpret_cast<_Float16*>(ws + L.ap);
  float* rho = reinterpret_cast<float*>(ws + L.rho);
  float* part = reinterpret_cast<float*>(ws + L.part);
  const _Float16* k = static_cast<const _Float16*>(y);
  const float cs = cs_of(sigma);
  const int Dp = hd::padded_features(D), Ck = hd::padded_k_channels(C);
  const dim3 pgrid((unsigned)hd_ceil_div(L.sp.Npad, 256), (unsigned)B);
  hipError_t e;
  if (bv_f32) {
    const float* w = static_cast<const float*>(bv);
    e = weight_norm_max(w, nullptr, nmax, B, N, C, s);
    if (e != hipSuccess) return e;
    col_prep_kernel<float, true><<<pgrid, 256, 0, s>>>(k, w, nullptr, nmax, beta, bvp, yp, N, L.sp.Npad, D, Dp, C,
                                                       Ck, cs);
  } else {
    const _Float16* w = static_cast<const _Float16*>(bv);
    e = weight_norm_max(w, nullptr, nmax, B, N, C, s);
    if (e != hipSuccess) return e;
    col_prep_kernel<_Float16, true><<<pgrid, 256, 0, s>>>(k, w, nullptr, nmax, beta, bvp, yp, N, L.sp.Npad, D, Dp, C,
                                                          Ck, cs);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 rgrid((unsigned)hd_ceil_div(M, 256), (unsigned)B);
  if (a_f32)
    row_prep_kernel<float><<<rgrid, 256, 0, s>>>(static_cast<const float*>(a), ap, rho, M, C, Ck);
  else
    row_prep_kernel<_Float16><<<rgrid, 256, 0, s>>>(static_cast<const _Float16*>(a), ap, rho, M, C, Ck);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hd::GradArgs g;
  g.x = static_cast<const _Float16*>(x);
  g.y = k;
  g.ap = ap;
  g.rho = rho;
  g.beta = beta;
  g.bvp = bvp;
  g.yp = yp;
  g.oscale = nmax;
  g.out = L.sp.splits > 1 ? part : out;
  g.M = M;
  g.N = N;
  g.Npad = L.sp.Npad;
  g.kps = L.sp.kps;
  g.cs = cs;
  g.tau = (float)(1.0 / ((double)sigma * (double)sigma));
  g.D = D;
  g.Ck = Ck;
  g.grid = dim3((unsigned)L.sp.row_blocks, (unsigned)L.sp.splits, (unsigned)B);
  g.stream = s;
  e = grad_dispatch(g);
  if (e != hipSuccess || L.sp.splits == 1) return e;
  return combine(part, out, B * M * D, L.sp.splits, s);
}

}  // namespace keops
