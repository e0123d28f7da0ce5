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

#include <type_traits>

#include <math.h>

namespace keops {
namespace {

using hd::half8;
using hd::hd_ceil_div;
using hd::slot_key;

template <typename T>
__device__ inline float to_f32(T v) { return (float)v; }

typedef __bf16 bf16_t;

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

// Column tables, one workgroup per 32-key block of one batch. The block's keys and weights are
// staged through LDS so that every global read and write is contiguous.
//   kMode kCopy:    beta_j = -|k_j|^2/2, wp = the fp16 weights unchanged (fast forward path);
//   kMode kNormFwd: the general form of the file comment, forward layout;
//   kMode kNormGrad: the general form, gradient layout, plus the key-permuted columns yp and,
//                    when wpl is given, the weights key-permuted again for the fused second
//                    output of the gradient sweep.
// Layouts: forward wp[t][j/32][c][key_slot(j%32)] for c < Cw (the A operand of O^T; with
// perm32 the slot32_key() order of the 32x32 tiles instead);
// gradient wp[t][j][c] for c < Cw (the A operand of dP^T) and yp[t][j/32][ch][key_slot(j%32)]
// = k[t][j][ch] for ch < D, 1 at ch = Dp, else 0. Keys past N get beta = -inf and zeros.
enum { kCopy = 0, kNormFwd = 1, kNormGrad = 2 };
constexpr int kMaxPrepD = 128;
constexpr int kMaxPrepC = 64;

template <typename TK, typename T, int kMode>
__global__ void __launch_bounds__(256)
col_prep_kernel(const TK* __restrict__ k, const T* __restrict__ w, const float* __restrict__ cscale,
                const float* __restrict__ nmax, float* __restrict__ beta, _Float16* __restrict__ wp,
                _Float16* __restrict__ wpl, _Float16* __restrict__ yp, int64_t N, int64_t Npad, int D, int Dp, int C,
                int Cw, float cs, int perm32) {
  __shared__ float sk[32][kMaxPrepD + 1];
  __shared__ float sw[32][kMaxPrepC + 1];
  __shared__ float sinv[32];
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.y;
  const int64_t j0 = (int64_t)blockIdx.x * 32;
  const int live = N - j0 >= 32 ? 32 : (N > j0 ? (int)(N - j0) : 0);

  // keys, contiguous in global memory, in 16-byte vectors (D is a multiple of 16)
  constexpr int EV = 16 / (int)sizeof(TK);
  typedef TK vec_t __attribute__((ext_vector_type(EV)));
  for (int c = tid; c < 32 * D / EV; c += 256) {
    const int key = (c * EV) / D, d = (c * EV) % D;
    vec_t v = vec_t{};
    if (key < live) v = *reinterpret_cast<const vec_t*>(k + (t * N + j0) * D + c * EV);
#pragma unroll
    for (int u = 0; u < EV; ++u) sk[key][d + u] = to_f32(v[u]);
  }
  // weights, times the column scale (fp16 rows of a multiple of 8 channels in 16-byte vectors)
  if (std::is_same<T, _Float16>::value && C % 8 == 0) {
    typedef T t8 __attribute__((ext_vector_type(8)));
    for (int c8 = tid; c8 < 32 * C / 8; c8 += 256) {
      const int key = (8 * c8) / C, c = (8 * c8) % C;
      t8 v = t8{};
      float sc = 1.0f;
      if (key < live) {
        v = *reinterpret_cast<const t8*>(w + (t * N + j0) * C + 8 * c8);
        if (cscale) sc = cscale[t * N + j0 + key];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) sw[key][c + u] = to_f32(v[u]) * sc;
    }
  } else {
    for (int e = tid; e < 32 * C; e += 256) {
      const int key = e / C, c = e % C;
      float v = 0.0f;
      if (key < live) {
        v = to_f32(w[(t * N + j0) * C + e]);
        if (cscale) v *= cscale[t * N + j0 + key];
      }
      sw[key][c] = v;
    }
  }
  __syncthreads();

  // squared key norms and weight norms: 8 lanes per key
  {
    const int key = tid >> 3, part = tid & 7;
    float kn = 0.0f, wn = 0.0f;
    for (int d = part; d < D; d += 8) kn = fmaf(sk[key][d], sk[key][d], kn);
    for (int c = part; c < C; c += 8) wn = fmaf(sw[key][c], sw[key][c], wn);
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      kn += __shfl_xor(kn, o, 8);
      wn += __shfl_xor(wn, o, 8);
    }
    if (part == 0) {
      float bj = -INFINITY, inv = 0.0f;
      if (key < live) {
        bj = -0.5f * kn;
        inv = 1.0f;
        if constexpr (kMode != kCopy) {
          const float n = sqrtf(wn);
          const float nm = nmax[t];
          const float ratio = nm > 0.0f ? n / nm : 0.0f;
          bj += fmaxf(log2f(ratio), hd::kLogFloor) / cs;
          inv = n > 0.0f ? 1.0f / n : 0.0f;
        }
      }
      beta[t * Npad + j0 + key] = bj;
      sinv[key] = inv;
    }
  }
  __syncthreads();

  if constexpr (kMode == kNormGrad) {
    _Float16* dst = wp + (t * Npad + j0) * Cw;
    for (int e = tid; e < 32 * Cw; e += 256) {
      const int key = e / Cw, c = e % Cw;
      dst[e] = (_Float16)(c < C ? sw[key][c] * sinv[key] : 0.0f);
    }
    if (wpl) {  // the same unit weights key-permuted over hd::kFusedWeightChannels channels
      constexpr int CF = hd::kFusedWeightChannels;
      _Float16* d2 = wpl + (t * Npad + j0) * CF;
      for (int e = tid; e < 32 * CF; e += 256) {
        const int c = e / 32, key = slot_key(e % 32);
        d2[e] = (_Float16)(c < C ? sw[key][c] * sinv[key] : 0.0f);
      }
    }
    const int YC = Dp + 16;
    _Float16* yd = yp + (t * Npad + j0) * YC;
    for (int e = tid; e < 32 * YC; e += 256) {
      const int ch = e / 32, key = slot_key(e % 32);
      _Float16 v = (_Float16)0.0f;
      if (ch < D) v = (_Float16)sk[key][ch];
      else if (ch == Dp && key < live) v = (_Float16)1.0f;
      yd[e] = v;
    }
  } else {
    // forward layout, 8 slots per 16-byte store; with wpl the fp16 lo parts of float32 weights
    // as well
    _Float16* dst = wp + (t * Npad + j0) * Cw;
    _Float16* dsl = wpl ? wpl + (t * Npad + j0) * Cw : nullptr;
    for (int e8 = tid; e8 < 4 * Cw; e8 += 256) {
      const int c = e8 / 4, s0 = (e8 % 4) * 8;
      hd::half8 h8, l8;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int key = perm32 ? hd::slot32_key(s0 + u) : slot_key(s0 + u);
        const float v = c < C ? sw[key][c] * sinv[key] : 0.0f;
        h8[u] = (_Float16)v;
        l8[u] = (_Float16)(v - (float)h8[u]);
      }
      *reinterpret_cast<hd::half8*>(dst + 8 * e8) = h8;
      if (dsl) *reinterpret_cast<hd::half8*>(dsl + 8 * e8) = l8;
    }
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

// out[r][d] = in[r][d] for d < D and 0 for D <= d < Dp (element bits copied unchanged; the
// all-zero pattern is +0 in every input format).
template <typename T>
__global__ void __launch_bounds__(256)
pad_rows_kernel(const T* __restrict__ in, T* __restrict__ out, int64_t rows, int D, int Dp) {
  const int64_t n = rows * Dp;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int64_t r = e / Dp;
    const int d = (int)(e - r * Dp);
    out[e] = d < D ? in[r * D + d] : T(0);
  }
}

// out[r][d] = in[r][d] for d < D, from rows of Dp values.
__global__ void __launch_bounds__(256)
narrow_rows_kernel(const float* __restrict__ in, float* __restrict__ out, int64_t rows, int Dp, int D) {
  const int64_t n = rows * D;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n; e += (int64_t)gridDim.x * 256) {
    const int64_t r = e / D;
    out[e] = in[r * Dp + (e - r * D)];
  }
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

// Column splits: enough workgroups for kSplitTarget workgroups of kWaves waves per CU (fewer
// when a workgroup has more waves), each split >= 4 * kKeyPad keys and a multiple of kKeyPad (so
// split boundaries fall on stage boundaries).
Split plan_split(int64_t B, int64_t M, int64_t N, int rows_per_block, int num_cus, int waves = hd::kWaves) {
  Split p;
  p.Npad = hd::padded_keys(N);
  p.row_blocks = hd_ceil_div(M, rows_per_block);
  const int64_t blocks = p.row_blocks * B;
  const int64_t target = (int64_t)num_cus * hd::kSplitTarget * hd::kWaves / waves;
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
  size_t nmax, beta, vp, vpl, part, total;
};

FwdLayout fwd_layout(int64_t B, int64_t M, int64_t N, int D, int C, ElemType xy, bool general, int num_cus) {
  FwdLayout L;
  const int Cp = hd::padded_channels(C);
  const bool split = xy == kElemF32;
  const int Dp = hd::padded_features(D);
  const int W = hd::fwd_waves(Dp, Cp, split);
  L.sp = plan_split(B, M, N, W * hd::fwd_query_tiles(Dp, Cp, split) * 16, num_cus, W);
  Carve c;
  const size_t table = (size_t)B * L.sp.Npad * Cp * sizeof(_Float16);
  L.nmax = c.take(general ? (size_t)B * sizeof(float) : 0);
  L.beta = c.take((size_t)B * L.sp.Npad * sizeof(float));
  L.vp = c.take(table);
  L.vpl = c.take(split ? table : 0);
  L.part = c.take(L.sp.splits > 1 ? (size_t)L.sp.splits * B * M * C * sizeof(float) : 0);
  L.total = c.off;
  return L;
}

struct GradLayout {
  Split sp;
  size_t nmax, beta, bvp, yp, ap, rho, part, gp, part2, total;
};

GradLayout grad_layout(int64_t B, int64_t M, int64_t N, int D, int C, bool fused, int num_cus) {
  GradLayout L;
  const int Dp = hd::padded_features(D), Ck = hd::padded_k_channels(C);
  L.sp = plan_split(B, M, N,
                    hd::grad_waves(Dp) * hd::grad_query_tiles(Dp, Ck, fused ? hd::kFusedWeightChannels : 0) * 16,
                    num_cus, hd::grad_waves(Dp));
  Carve c;
  L.nmax = c.take((size_t)B * sizeof(float));
  L.beta = c.take((size_t)B * L.sp.Npad * sizeof(float));
  L.bvp = c.take((size_t)B * L.sp.Npad * Ck * sizeof(_Float16));
  L.yp = c.take((size_t)B * L.sp.Npad * (Dp + 16) * sizeof(_Float16));
  L.ap = c.take((size_t)B * M * Ck * sizeof(_Float16));
  L.rho = c.take((size_t)B * M * sizeof(float));
  L.part = c.take(L.sp.splits > 1 ? (size_t)L.sp.splits * B * M * D * sizeof(float) : 0);
  L.gp = c.take(fused ? (size_t)B * L.sp.Npad * hd::kFusedWeightChannels * sizeof(_Float16) : 0);
  L.part2 = c.take(fused && L.sp.splits > 1 ? (size_t)L.sp.splits * B * M * C * sizeof(float) : 0);
  L.total = c.off;
  return L;
}

float cs_of(float sigma) {
  const double s = (double)sigma;
  return (float)(1.4426950408889634 / (s * s));  // tau log2(e)
}

template <typename TIn>
hipError_t fwd_dispatch_t(const hd::FwdArgs& a) {
  switch (hd::padded_features(a.D)) {
    case 32: return hd::fwd_launch<TIn, 32>(a);
    case 64: return hd::fwd_launch<TIn, 64>(a);
    case 96: return hd::fwd_launch<TIn, 96>(a);
    case 128: return hd::fwd_launch<TIn, 128>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t fwd_dispatch(const hd::FwdArgs& a, ElemType xy) {
  switch (xy) {
    case kElemF16: return fwd_dispatch_t<_Float16>(a);
    case kElemBF16: return fwd_dispatch_t<bf16_t>(a);
    case kElemF32: return fwd_dispatch_t<float>(a);
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

int hd_fused_weight_channels() { return hd::kFusedWeightChannels; }

bool highd_supported(int D, int C) { return D >= 1 && D <= 128 && C >= 1 && C <= 64; }

int highd_stored_features(int D) { return (D + 15) / 16 * 16; }

namespace {
int64_t grid_stride_blocks(int64_t n) {
  const int64_t b = hd_ceil_div(n, 256);
  return b < 1 ? 1 : (b > 65536 ? 65536 : b);
}
}  // namespace

hipError_t launch_pad_rows(const void* in, void* out, int64_t rows, int D, int Dp, int elem_bytes, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const unsigned blocks = (unsigned)grid_stride_blocks(rows * Dp);
  if (elem_bytes == 2)
    pad_rows_kernel<uint16_t><<<blocks, 256, 0, s>>>(static_cast<const uint16_t*>(in), static_cast<uint16_t*>(out),
                                                     rows, D, Dp);
  else if (elem_bytes == 4)
    pad_rows_kernel<uint32_t><<<blocks, 256, 0, s>>>(static_cast<const uint32_t*>(in), static_cast<uint32_t*>(out),
                                                     rows, D, Dp);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_narrow_rows(const float* in, float* out, int64_t rows, int Dp, int D, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  narrow_rows_kernel<<<(unsigned)grid_stride_blocks(rows * D), 256, 0, s>>>(in, out, rows, Dp, D);
  return hipGetLastError();
}

bool highd_general(ElemType xy, ElemType bt, bool col_scaled) {
  return xy != kElemF16 || bt != kElemF16 || col_scaled;
}

size_t highd_workspace_bytes(int64_t B, int64_t M, int64_t N, int D, int C, ElemType xy, bool general) {
  if (B == 0 || M == 0 || N == 0) return 0;
  return fwd_layout(B, M, N, D, C, xy, general, device_cus()).total;
}

size_t highd_grad_workspace_bytes(int64_t B, int64_t M, int64_t N, int D, int C, bool fused) {
  if (B == 0 || M == 0 || N == 0) return 0;
  return grad_layout(B, M, N, D, C, fused, device_cus()).total;
}

namespace {

// Column tables of the general forward form for keys of type TK and weights of type T.
template <typename TK, typename T>
hipError_t fwd_prep_general(const TK* k, const T* w, const float* cscale, float* nmax, float* beta, _Float16* vp,
                            _Float16* vpl, int64_t B, int64_t N, int64_t Npad, int D, int C, int Cp, float cs,
                            int perm32, hipStream_t s) {
  hipError_t e = weight_norm_max(w, cscale, nmax, B, N, C, s);
  if (e != hipSuccess) return e;
  col_prep_kernel<TK, T, kNormFwd><<<dim3((unsigned)(Npad / 32), (unsigned)B), 256, 0, s>>>(
      k, w, cscale, nmax, beta, vp, vpl, nullptr, N, Npad, D, 0, C, Cp, cs, perm32);
  return hipGetLastError();
}

template <typename TK>
hipError_t fwd_prep_general_w(const TK* k, const void* w, ElemType bt, const float* cscale, float* nmax, float* beta,
                              _Float16* vp, _Float16* vpl, int64_t B, int64_t N, int64_t Npad, int D, int C, int Cp,
                              float cs, int perm32, hipStream_t s) {
  switch (bt) {
    case kElemF16:
      return fwd_prep_general(k, static_cast<const _Float16*>(w), cscale, nmax, beta, vp, vpl, B, N, Npad, D, C, Cp,
                              cs, perm32, s);
    case kElemBF16:
      return fwd_prep_general(k, static_cast<const bf16_t*>(w), cscale, nmax, beta, vp, vpl, B, N, Npad, D, C, Cp,
                              cs, perm32, s);
    case kElemF32:
      return fwd_prep_general(k, static_cast<const float*>(w), cscale, nmax, beta, vp, vpl, B, N, Npad, D, C, Cp, cs,
                              perm32, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gauss_sum_highd(const void* x, const void* y, ElemType xy, const void* b, ElemType bt,
                                  const float* rscale, const float* cscale, float* out, void* workspace, int64_t B,
                                  int64_t M, int64_t N, int D, int C, float sigma, hipStream_t s) {
  const bool general = highd_general(xy, bt, cscale != nullptr);
  const FwdLayout L = fwd_layout(B, M, N, D, C, xy, general, device_cus());
  char* ws = static_cast<char*>(workspace);
  float* nmax = reinterpret_cast<float*>(ws + L.nmax);
  float* beta = reinterpret_cast<float*>(ws + L.beta);
  _Float16* vp = reinterpret_cast<_Float16*>(ws + L.vp);
  _Float16* vpl = xy == kElemF32 ? reinterpret_cast<_Float16*>(ws + L.vpl) : nullptr;
  float* part = reinterpret_cast<float*>(ws + L.part);
  const float cs = cs_of(sigma);
  const int Cp = hd::padded_channels(C);
  const int sq = hd::fwd_square(xy == kElemF32, hd::padded_features(D), Cp) ? 1 : 0;
  hipError_t e;
  if (!general) {
    col_prep_kernel<_Float16, _Float16, kCopy><<<dim3((unsigned)(L.sp.Npad / 32), (unsigned)B), 256, 0, s>>>(
        static_cast<const _Float16*>(y), static_cast<const _Float16*>(b), nullptr, nullptr, beta, vp, nullptr,
        nullptr, N, L.sp.Npad, D, 0, C, Cp, cs, sq);
    e = hipGetLastError();
  } else if (xy == kElemF16) {
    e = fwd_prep_general_w(static_cast<const _Float16*>(y), b, bt, cscale, nmax, beta, vp, vpl, B, N, L.sp.Npad, D,
                           C, Cp, cs, sq, s);
  } else if (xy == kElemBF16) {
    e = fwd_prep_general_w(static_cast<const bf16_t*>(y), b, bt, cscale, nmax, beta, vp, vpl, B, N, L.sp.Npad, D, C,
                           Cp, cs, sq, s);
  } else {
    e = fwd_prep_general_w(static_cast<const float*>(y), b, bt, cscale, nmax, beta, vp, vpl, B, N, L.sp.Npad, D, C,
                           Cp, cs, sq, s);
  }
  if (e != hipSuccess) return e;
  hd::FwdArgs a;
  a.q = x;
  a.k = y;
  a.beta = beta;
  a.vp = vp;
  a.vpl = vpl;
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
  sweep_event(s, true);
  if (sq) e = xy == kElemF16 ? hd::fwd32_launch<_Float16>(a) : hd::fwd32_launch<bf16_t>(a);
  else e = fwd_dispatch(a, xy);
  sweep_event(s, false);
  if (e != hipSuccess || L.sp.splits == 1) return e;
  return combine(part, out, B * M * C, L.sp.splits, s);
}

hipError_t launch_gauss_sum_grad_highd(const void* x, const void* y, const void* a, bool a_f32, const void* bv,
                                       bool bv_f32, float* out, float* out2, void* workspace, int64_t B, int64_t M,
                                       int64_t N, int D, int C, float sigma, hipStream_t s) {
  const bool fused = out2 != nullptr;
  if (fused && C > hd::kFusedWeightChannels) return hipErrorInvalidValue;
  const GradLayout L = grad_layout(B, M, N, D, C, fused, device_cus());
  char* ws = static_cast<char*>(workspace);
  float* nmax = reinterpret_cast<float*>(ws + L.nmax);
  float* beta = reinterpret_cast<float*>(ws + L.beta);
  _Float16* bvp = reinterpret_cast<_Float16*>(ws + L.bvp);
  _Float16* yp = reinterpret_cast<_Float16*>(ws + L.yp);
  _Float16* ap = reinterpret_cast<_Float16*>(ws + L.ap);
  float* rho = reinterpret_cast<float*>(ws + L.rho);
  float* part = reinterpret_cast<float*>(ws + L.part);
  _Float16* gp = fused ? reinterpret_cast<_Float16*>(ws + L.gp) : nullptr;
  float* part2 = reinterpret_cast<float*>(ws + L.part2);
  const _Float16* k = static_cast<const _Float16*>(y);
  const float cs = cs_of(sigma);
  const int Dp = hd::padded_features(D), Ck = hd::padded_k_channels(C);
  const dim3 pgrid((unsigned)(L.sp.Npad / 32), (unsigned)B);
  hipError_t e;
  if (bv_f32) {
    const float* w = static_cast<const float*>(bv);
    e = weight_norm_max(w, nullptr, nmax, B, N, C, s);
    if (e != hipSuccess) return e;
    col_prep_kernel<_Float16, float, kNormGrad><<<pgrid, 256, 0, s>>>(k, w, nullptr, nmax, beta, bvp, gp, yp, N,
                                                                      L.sp.Npad, D, Dp, C, Ck, cs, 0);
  } else {
    const _Float16* w = static_cast<const _Float16*>(bv);
    e = weight_norm_max(w, nullptr, nmax, B, N, C, s);
    if (e != hipSuccess) return e;
    col_prep_kernel<_Float16, _Float16, kNormGrad><<<pgrid, 256, 0, s>>>(k, w, nullptr, nmax, beta, bvp, gp, yp,
                                                                         N, L.sp.Npad, D, Dp, C, Ck, cs, 0);
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
  g.gp = gp;
  g.out2 = fused ? (L.sp.splits > 1 ? part2 : out2) : nullptr;
  g.C2 = C;
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
  e = combine(part, out, B * M * D, L.sp.splits, s);
  if (e != hipSuccess || !fused) return e;
  return combine(part2, out2, B * M * C, L.sp.splits, s);
}

}  // namespace keops
