// Matrix-core (fp16) batched Gauss sum for gfx950:
//   out[t][i][c] = sum_j exp(-tau/2 ||q_i - k_j||^2) v[j][c],  tau = 1/sigma^2,
// the Gauss sum with signed weights of "Fast Gauss Sums via Flash Attention" (its eq. (1)),
// evaluated with the squared-norm expansion ||q - k||^2 = ||q||^2 + ||k||^2 - 2 q.k so that
// the O(N M D) part is a dense contraction on the matrix cores.
//
// Per wave: 2 tiles of 32 query rows. Per 32-key subtile:
//   S^T = K Q^T + B      two v_mfma_f32_32x32x16_f16 per D=32; the accumulator starts from
//                        B[j] = -|k_j|^2 / 2, so S'_ij = q_i.k_j - |k_j|^2/2 comes out whole;
//   a_ij = c S'_ij + alpha_i,  c = tau log2(e),  alpha_i = -c |q_i|^2 / 2 - m_i   (one FMA);
//   P = 2^a rounded to fp16; O^T += V^T P^T       two MFMAs per 32 channels.
// The accumulator layout of S^T gives each lane one query row and 16 keys; those 16 values
// are exactly the lane's fp16 operand of the P^T product once the keys of every subtile are
// visited in the order slot_key() (V is stored pre-permuted the same way), so P never moves
// between lanes. m_i is a running base-2 shift: set by the first subtile, raised only when a
// subtile would produce a term above 2^kSlack (then O is rescaled), so P stays in fp16 range.
#include "internal.h"

#include <math.h>

namespace keops {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;          // waves per workgroup
constexpr int kQT = 2;             // 32-row query tiles per wave
constexpr int kRowsPerBlock = kWaves * kQT * 32;
constexpr int kStage = 64;         // keys per LDS stage (two 32-key subtiles)
constexpr float kSlack = 8.0f;     // lazy rescale threshold, base-2 units

__device__ __forceinline__ float exp2_hw(float v) { return __builtin_amdgcn_exp2f(v); }

// Offset of the key held in fp16 operand slot `slot` (0..31) of a 32-key subtile:
// slot = 16*step + 8*half + s. It inverts the accumulator row map 8*(v/4) + 4*half + v%4.
__host__ __device__ inline int slot_key(int slot) {
  const int st = slot >> 4, h = (slot >> 3) & 1, s = slot & 7;
  return 16 * st + 4 * h + (s & 3) + 8 * (s >> 2);
}
__host__ __device__ inline int key_slot(int o) {
  const int st = o >> 4, rem = o & 15;
  const int h = (rem >> 2) & 1, s = (rem & 3) + 4 * (rem >> 3);
  return 16 * st + 8 * h + s;
}

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t padded_keys(int64_t N) { return ceil_div(N, kStage) * kStage; }

// beta[t][j] = -|k_j|^2 / 2 for j < N and -inf for N <= j < Npad;
// vp[t][j / 32][c][key_slot(j % 32)] = v[t][j][c] (zero for padded keys).
__global__ void __launch_bounds__(256)
highd_prep_kernel(const _Float16* __restrict__ k, const _Float16* __restrict__ v, float* __restrict__ beta,
                  _Float16* __restrict__ vp, int64_t N, int64_t Npad, int D, int C) {
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
  _Float16* dst = vp + (t * Npad + (j / 32) * 32) * C + key_slot((int)(j % 32));
  for (int c = 0; c < C; ++c) dst[(int64_t)c * 32] = (j < N) ? vr[c] : (_Float16)0.0f;
}

template <int D, int C>
__global__ void __launch_bounds__(256)
highd_kernel(const _Float16* __restrict__ q, const _Float16* __restrict__ k, const float* __restrict__ beta,
             const _Float16* __restrict__ vp, float* __restrict__ out, int64_t M, int64_t N, int64_t Npad,
             int64_t kps, float cs) {
  constexpr int DS = D / 16;     // K-steps of S^T
  constexpr int CT = C / 32;     // 32-channel output tiles
  constexpr int KP = D + 8;      // LDS row pitch of K, halves
  constexpr int VP = 32 + 8;     // LDS row pitch of V^T, halves
  __shared__ __attribute__((aligned(16))) _Float16 sK[2][kStage][KP];
  __shared__ __attribute__((aligned(16))) _Float16 sV[2][kStage / 32][C][VP];
  __shared__ __attribute__((aligned(16))) float sB[2][kStage];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t bt = blockIdx.z, split = blockIdx.y;
  const int64_t j0 = split * kps;
  const int64_t j1 = (j0 + kps < N) ? j0 + kps : N;
  const int64_t nstages = ceil_div(j1 - j0, kStage);
  const int64_t row_base = (int64_t)blockIdx.x * kRowsPerBlock + wave * (kQT * 32);

  const _Float16* qb = q + bt * M * D;
  const _Float16* kb = k + bt * N * D;
  const float* bb = beta + bt * Npad;
  const _Float16* vb = vp + bt * Npad * C;

  half8 qop[kQT][DS];
  float alpha[kQT], mrow[kQT];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    int64_t i = row_base + qt * 32 + l32;
    i = i < M ? i : M - 1;
    float nrm = 0.0f;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      qop[qt][ds] = *reinterpret_cast<const half8*>(qb + i * D + 16 * ds + 8 * h);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float qv = (float)qop[qt][ds][s];
        nrm = fmaf(qv, qv, nrm);
      }
    }
    nrm += __shfl_xor(nrm, 32);
    alpha[qt] = -0.5f * cs * nrm;
    mrow[qt] = 0.0f;
  }
  f32x16 O[kQT][CT];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int v = 0; v < 16; ++v) O[qt][ct][v] = 0.0f;

  auto load_stage = [&](int buf, int64_t st) {
    const int64_t jb = j0 + st * kStage;
    for (int c = tid; c < kStage * D / 8; c += 256) {
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      const int64_t j = jb + row;
      half8 val = {};
      if (j < j1) val = *reinterpret_cast<const half8*>(kb + j * D + col);
      *reinterpret_cast<half8*>(&sK[buf][row][col]) = val;
    }
    for (int c = tid; c < (kStage / 32) * C * 4; c += 256) {
      const int t = c / (C * 4), rem = c % (C * 4), ch = rem / 4, part = (rem % 4) * 8;
      const int64_t tile = jb / 32 + t;
      const half8 val = *reinterpret_cast<const half8*>(vb + (tile * C + ch) * 32 + part);
      *reinterpret_cast<half8*>(&sV[buf][t][ch][part]) = val;
    }
    for (int c = tid; c < kStage; c += 256) sB[buf][c] = bb[jb + c];
  };

  load_stage(0, 0);
  __syncthreads();
  bool first = true;
  for (int64_t st = 0; st < nstages; ++st) {
    const int buf = (int)(st & 1);
    if (st + 1 < nstages) load_stage(buf ^ 1, st + 1);
#pragma unroll
    for (int sub = 0; sub < kStage / 32; ++sub) {
      half8 kop[DS];
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) kop[ds] = *reinterpret_cast<const half8*>(&sK[buf][sub * 32 + l32][16 * ds + 8 * h]);
      f32x16 bc;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 t4 = *reinterpret_cast<const f32x4*>(&sB[buf][sub * 32 + 8 * g + 4 * h]);
        bc[4 * g + 0] = t4[0];
        bc[4 * g + 1] = t4[1];
        bc[4 * g + 2] = t4[2];
        bc[4 * g + 3] = t4[3];
      }
      half8 vop[CT][2];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
          vop[ct][s2] = *reinterpret_cast<const half8*>(&sV[buf][sub][32 * ct + l32][16 * s2 + 8 * h]);
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) {
        f32x16 S = __builtin_amdgcn_mfma_f32_32x32x16_f16(kop[0], qop[qt][0], bc, 0, 0, 0);
#pragma unroll
        for (int ds = 1; ds < DS; ++ds) S = __builtin_amdgcn_mfma_f32_32x32x16_f16(kop[ds], qop[qt][ds], S, 0, 0, 0);
        float mx = S[0];
#pragma unroll
        for (int v = 1; v < 16; ++v) mx = fmaxf(mx, S[v]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float amax = fmaf(mx, cs, alpha[qt]);
        if (first) {
          alpha[qt] -= amax;
          mrow[qt] += amax;
        } else if (amax > kSlack) {
          alpha[qt] -= amax;
          mrow[qt] += amax;
          const float sc = exp2_hw(-amax);
#pragma unroll
          for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int v = 0; v < 16; ++v) O[qt][ct][v] *= sc;
        }
        half8 pb[2];
#pragma unroll
        for (int v = 0; v < 16; ++v) pb[v >> 3][v & 7] = (_Float16)exp2_hw(fmaf(S[v], cs, alpha[qt]));
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2)
            O[qt][ct] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vop[ct][s2], pb[s2], O[qt][ct], 0, 0, 0);
      }
      first = false;
    }
    __syncthreads();
  }

  const int64_t BMC = (int64_t)gridDim.z * M * C;
  float* dst = out + split * BMC + bt * M * C;
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const int64_t i = row_base + qt * 32 + l32;
    if (i >= M) continue;
    const float scale = exp2_hw(mrow[qt]);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 o;
        o[0] = O[qt][ct][4 * g + 0] * scale;
        o[1] = O[qt][ct][4 * g + 1] * scale;
        o[2] = O[qt][ct][4 * g + 2] * scale;
        o[3] = O[qt][ct][4 * g + 3] * scale;
        *reinterpret_cast<f32x4*>(dst + i * C + 32 * ct + 8 * g + 4 * h) = o;
      }
  }
}

__global__ void __launch_bounds__(256)
highd_combine_kernel(const float* __restrict__ partial, float* __restrict__ out, int64_t n, int64_t S) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  for (int64_t k = 0; k < S; ++k) s += partial[k * n + i];
  out[i] = s;
}

struct HighdPlan {
  int64_t Npad, row_blocks, splits, kps;
  size_t beta_bytes, vp_bytes, part_bytes, total;
};

HighdPlan highd_plan(int64_t B, int64_t M, int64_t N, int D, int C, int num_cus) {
  (void)D;
  HighdPlan p;
  p.Npad = padded_keys(N);
  p.row_blocks = ceil_div(M, kRowsPerBlock);
  const int64_t blocks = p.row_blocks * B;
  const int64_t target = (int64_t)num_cus * 2;
  int64_t S = blocks < target ? ceil_div(target, blocks) : 1;
  const int64_t max_split = p.Npad / (4 * kStage) > 1 ? p.Npad / (4 * kStage) : 1;
  if (S > max_split) S = max_split;
  int64_t kps = ceil_div(ceil_div(N, S), kStage) * kStage;
  S = ceil_div(N, kps);
  p.splits = S;
  p.kps = kps;
  p.beta_bytes = align_up((size_t)B * p.Npad * sizeof(float));
  p.vp_bytes = align_up((size_t)B * p.Npad * C * sizeof(_Float16));
  p.part_bytes = S > 1 ? align_up((size_t)S * B * M * C * sizeof(float)) : 0;
  p.total = p.beta_bytes + p.vp_bytes + p.part_bytes;
  return p;
}

}  // namespace

bool highd_supported(int D, int C) { return (D == 32 || D == 64) && (C == 32 || C == 64); }

size_t highd_workspace_bytes(int64_t B, int64_t M, int64_t N, int D, int C) {
  if (B == 0 || M == 0 || N == 0) return 0;
  return highd_plan(B, M, N, D, C, device_cus()).total;
}

hipError_t launch_gauss_sum_highd(const void* x, const void* y, const void* b, float* out, void* workspace,
                                  int64_t B, int64_t M, int64_t N, int D, int C, float sigma, bool bf16,
                                  hipStream_t s) {
  if (bf16) return hipErrorNotSupported;
  const HighdPlan p = highd_plan(B, M, N, D, C, device_cus());
  char* ws = static_cast<char*>(workspace);
  float* beta = reinterpret_cast<float*>(ws);
  _Float16* vpm = reinterpret_cast<_Float16*>(ws + p.beta_bytes);
  float* part = reinterpret_cast<float*>(ws + p.beta_bytes + p.vp_bytes);
  const _Float16* q = static_cast<const _Float16*>(x);
  const _Float16* k = static_cast<const _Float16*>(y);
  const _Float16* v = static_cast<const _Float16*>(b);
  const double sd = (double)sigma;
  const float cs = (float)(1.4426950408889634 / (sd * sd));  // tau log2(e)
  highd_prep_kernel<<<dim3((unsigned)ceil_div(p.Npad, 256), (unsigned)B), 256, 0, s>>>(k, v, beta, vpm, N, p.Npad, D, C);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  float* dst = p.splits > 1 ? part : out;
  const dim3 grid((unsigned)p.row_blocks, (unsigned)p.splits, (unsigned)B);
  if (D == 32 && C == 32) highd_kernel<32, 32><<<grid, 256, 0, s>>>(q, k, beta, vpm, dst, M, N, p.Npad, p.kps, cs);
  else if (D == 32 && C == 64) highd_kernel<32, 64><<<grid, 256, 0, s>>>(q, k, beta, vpm, dst, M, N, p.Npad, p.kps, cs);
  else if (D == 64 && C == 32) highd_kernel<64, 32><<<grid, 256, 0, s>>>(q, k, beta, vpm, dst, M, N, p.Npad, p.kps, cs);
  else if (D == 64 && C == 64) highd_kernel<64, 64><<<grid, 256, 0, s>>>(q, k, beta, vpm, dst, M, N, p.Npad, p.kps, cs);
  else return hipErrorInvalidValue;
  e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const int64_t n = B * M * C;
  highd_combine_kernel<<<(unsigned)ceil_div(n, 256), 256, 0, s>>>(part, out, n, p.splits);
  return hipGetLastError();
}

}  // namespace keops
