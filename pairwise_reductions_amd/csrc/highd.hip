// Matrix-core (fp16) batched Gauss sum for gfx950:
//   out[t][i][c] = sum_j exp(-tau/2 ||q_i - k_j||^2) v[j][c],  tau = 1/sigma^2,
// the Gauss sum with signed weights of "Fast Gauss Sums via Flash Attention" (its eq. (1)),
// evaluated with the squared-norm expansion ||q - k||^2 = ||q||^2 + ||k||^2 - 2 q.k so that
// the O(N M D) part is a dense contraction on the matrix cores.
//
// Tiles are 16 queries x 32 keys on v_mfma_f32_16x16x32_f16. Per wave: QT query tiles.
//   S^T = K Q^T + B   one MFMA per 16 keys at D = 32; the accumulator starts from
//                     B[j] = -|k_j|^2 / 2, so S'_ij = q_i.k_j - |k_j|^2/2 comes out whole;
//   a_ij = c S'_ij + alpha_i,  c = tau log2(e),  alpha_i = -c |q_i|^2 / 2 - m_i   (one FMA);
//   P = 2^a rounded to fp16;  O^T += V^T P^T   one MFMA per 16 channels (K = 32 keys).
// In the accumulator of S^T a lane holds one query and 4 keys of each 16-key half; those 8
// values are exactly the lane's fp16 operand of the P^T product when the 32 keys of a
// subtile are visited in the order slot_key() (V is stored pre-permuted the same way), so P
// never moves between lanes. m_i is a running base-2 shift: set by the first subtile and
// raised only when a subtile would produce a term above 2^kSlack (then O is rescaled).
#include "internal.h"

#include <math.h>

#include <type_traits>

namespace keops {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;           // waves per workgroup
constexpr int kStageKeys = 64;      // keys per LDS stage (32-key subtiles staged together)
// Query tiles per wave and register budget. Measured on the B=4, 16384^2, D=C=32 workload,
// more independent query tiles per wave beat more resident waves: the matrix cores and the
// exp pipe overlap within a wave. Larger D or C take fewer tiles to stay within registers.
constexpr int query_tiles(int D, int C) { return (D == 32 && C <= 32) ? 8 : 4; }
// Channels are processed in tiles of 16; a call with C channels runs the kernel for
// padded_channels(C) and stores the first C.
constexpr int padded_channels(int C) { return C <= 16 ? 16 : (C <= 32 ? 32 : 64); }
constexpr int kMinBlocks = 1;       // workgroups per CU the register budget is sized for
constexpr int kSplitTarget = 2;     // column splits aim for this many workgroups per CU
constexpr int kKeyPad = 256;        // key counts are padded to a multiple of this
constexpr float kSlack = 8.0f;      // kernel values may reach 2^kSlack before a rescale

__device__ __forceinline__ float exp2_hw(float v) { return __builtin_amdgcn_exp2f(v); }

// Key offset (0..31 within a subtile) held in fp16 operand slot `slot` = 8*g + s, where g is
// the lane's 16-lane group: slots 0..3 are keys 4g..4g+3 of the first 16-key half, slots
// 4..7 the same of the second half. key_slot() is the inverse.
__host__ __device__ inline int slot_key(int slot) {
  const int g = slot >> 3, s = slot & 7;
  return 4 * g + (s & 3) + 16 * (s >> 2);
}
__host__ __device__ inline int key_slot(int o) {
  const int half = o >> 4, rem = o & 15;
  return 8 * (rem >> 2) + 4 * half + (rem & 3);
}

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t padded_keys(int64_t N) { return ceil_div(N, kKeyPad) * kKeyPad; }

// beta[t][j] = -|k_j|^2 / 2 for j < N and -inf for N <= j < Npad;
// vp[t][j / 32][c][key_slot(j % 32)] = v[t][j][c] for c < C, zero for padded keys and for the
// padding channels C <= c < Cp.
__global__ void __launch_bounds__(256)
highd_prep_kernel(const _Float16* __restrict__ k, const _Float16* __restrict__ v, float* __restrict__ beta,
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

template <int D, int C, int QT, int kMinB, int kStage, bool kPipe>
__global__ void __launch_bounds__(256, kMinB)
highd_kernel(const _Float16* __restrict__ q, const _Float16* __restrict__ k, const float* __restrict__ beta,
             const _Float16* __restrict__ vp, float* __restrict__ out, int64_t M, int64_t N, int64_t Npad,
             int64_t kps, float cs, int Cout) {
  constexpr int DS = D / 32;     // K-steps of S^T
  constexpr int CT = C / 16;     // 16-channel output tiles
  constexpr int KP = D + 8;      // LDS row pitch of K, halves
  constexpr int VP = 32 + 8;     // LDS row pitch of V^T, halves
  constexpr int NSUB = kStage / 32;
  constexpr int kRowsPerBlock = kWaves * QT * 16;
  __shared__ __attribute__((aligned(16))) _Float16 sK[2][kStage][KP];
  __shared__ __attribute__((aligned(16))) _Float16 sV[2][NSUB][C][VP];
  __shared__ __attribute__((aligned(16))) float sB[2][kStage];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t bt = blockIdx.z, split = blockIdx.y;
  const int64_t j0 = split * kps;
  const int64_t j1 = (j0 + kps < N) ? j0 + kps : N;
  const int64_t nstages = ceil_div(j1 - j0, kStage);
  const int64_t row_base = (int64_t)blockIdx.x * kRowsPerBlock + wave * (QT * 16);

  const _Float16* qb = q + bt * M * D;
  const _Float16* kb = k + bt * N * D;
  const float* bb = beta + bt * Npad;
  const _Float16* vb = vp + bt * Npad * C;

  half8 qop[QT][DS];
  float alpha[QT], mrow[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    int64_t i = row_base + qt * 16 + l16;
    i = i < M ? i : M - 1;
    float nrm = 0.0f;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      qop[qt][ds] = *reinterpret_cast<const half8*>(qb + i * D + 32 * ds + 8 * g);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float qv = (float)qop[qt][ds][s];
        nrm = fmaf(qv, qv, nrm);
      }
    }
    nrm += __shfl_xor(nrm, 16);
    nrm += __shfl_xor(nrm, 32);
    alpha[qt] = -0.5f * cs * nrm;
    mrow[qt] = 0.0f;
  }
  f32x4 O[QT][CT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) O[qt][ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  // Stage loads: global -> registers (issued before the current stage is computed) and
  // registers -> LDS (after it), so global latency hides behind the matrix work.
  constexpr int KCH = kStage * D / 8 / 256;       // 16-byte K chunks per thread
  constexpr int kVChunks = NSUB * C * 4;          // 16-byte V chunks per stage
  constexpr int VCH = (kVChunks + 255) / 256;     // ... per thread (the last round may be partial)
  static_assert(KCH * 256 * 8 == kStage * D && kStage / 4 <= 256, "tile shapes");
  static_assert(kVChunks % 256 == 0 || VCH == 1, "tile shapes");
  half8 rk[KCH], rv[VCH];
  f32x4 rb = {};
  auto fetch = [&](int64_t st) {
    const int64_t jb = j0 + st * kStage;
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int c = tid + 256 * r;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      const int64_t j = jb + row;
      rk[r] = half8{};
      if (j < j1) rk[r] = *reinterpret_cast<const half8*>(kb + j * D + col);
    }
#pragma unroll
    for (int r = 0; r < VCH; ++r) {
      const int c = tid + 256 * r;
      const int t = c / (C * 4), rem = c % (C * 4), ch = rem / 4, part = (rem % 4) * 8;
      if (c < kVChunks) rv[r] = *reinterpret_cast<const half8*>(vb + ((jb / 32 + t) * C + ch) * 32 + part);
    }
    if (tid < kStage / 4) rb = *reinterpret_cast<const f32x4*>(bb + jb + 4 * tid);
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int c = tid + 256 * r;
      *reinterpret_cast<half8*>(&sK[buf][c / (D / 8)][(c % (D / 8)) * 8]) = rk[r];
    }
#pragma unroll
    for (int r = 0; r < VCH; ++r) {
      const int c = tid + 256 * r;
      const int t = c / (C * 4), rem = c % (C * 4);
      if (c < kVChunks) *reinterpret_cast<half8*>(&sV[buf][t][rem / 4][(rem % 4) * 8]) = rv[r];
    }
    if (tid < kStage / 4) *reinterpret_cast<f32x4*>(&sB[buf][4 * tid]) = rb;
  };

  // S'^T of one 32-key subtile for every query tile: S[qt][half] holds keys 16*half + 4g + v.
  auto scores = [&](int buf, int sub, f32x4 (&S)[QT][2]) {
    half8 kop[2][DS];
    f32x4 bc[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int ds = 0; ds < DS; ++ds)
        kop[hh][ds] = *reinterpret_cast<const half8*>(&sK[buf][sub * 32 + 16 * hh + l16][32 * ds + 8 * g]);
      bc[hh] = *reinterpret_cast<const f32x4*>(&sB[buf][sub * 32 + 16 * hh + 4 * g]);
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        S[qt][hh] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[hh][0], qop[qt][0], bc[hh], 0, 0, 0);
#pragma unroll
        for (int ds = 1; ds < DS; ++ds)
          S[qt][hh] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[hh][ds], qop[qt][ds], S[qt][hh], 0, 0, 0);
      }
  };
  // P = 2^(c S' + alpha) in fp16 and O^T += V^T P^T for one subtile.
  auto accumulate = [&](int buf, int sub, const f32x4 (&S)[QT][2]) {
    half8 vop[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) vop[ct] = *reinterpret_cast<const half8*>(&sV[buf][sub][16 * ct + l16][8 * g]);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      half8 pb;
#pragma unroll
      for (int s = 0; s < 8; ++s) pb[s] = (_Float16)exp2_hw(fmaf(S[qt][s >> 2][s & 3], cs, alpha[qt]));
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) O[qt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[ct], pb, O[qt][ct], 0, 0, 0);
    }
  };
  // A row is settled once its shift m >= -kSlack: every later kernel value is then at most
  // 2^-m <= 2^kSlack (the Gaussian exponent is never positive), so no row maximum is needed.
  // Until then each subtile raises the shifts where a term would exceed 2^kSlack (or sets
  // them, on the first subtile) and rescales O to match.
  bool first = true, settled = false;
  auto track_rows = [&](const f32x4 (&S)[QT][2]) {
    bool all_settled = true;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mx = fmaxf(fmaxf(fmaxf(S[qt][0][0], S[qt][0][1]), fmaxf(S[qt][0][2], S[qt][0][3])),
                       fmaxf(fmaxf(S[qt][1][0], S[qt][1][1]), fmaxf(S[qt][1][2], S[qt][1][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float amax = fmaf(mx, cs, alpha[qt]);
      const float delta = (first || amax > kSlack) ? amax : 0.0f;
      alpha[qt] -= delta;
      mrow[qt] += delta;
      const float sc = (first || delta == 0.0f) ? 1.0f : exp2_hw(-delta);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) O[qt][ct] *= sc;
      all_settled = all_settled && (mrow[qt] >= -kSlack);
    }
    settled = __all(all_settled);
    first = false;
  };
  // One stage; both phases execute one barrier per stage, so the workgroup stays in step.
  auto stage = [&](int64_t st, auto track) {
    constexpr bool kTrack = decltype(track)::value;
    const int buf = (int)(st & 1);
    if (st + 1 < nstages) fetch(st + 1);
    if constexpr (kTrack || !kPipe) {
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub) {
        f32x4 S[QT][2];
        scores(buf, sub, S);
        if constexpr (kTrack) track_rows(S);
        accumulate(buf, sub, S);
      }
    } else {
      // Software-pipelined: the scores of subtile n+1 are issued to the matrix cores before
      // the exponentials of subtile n.
      f32x4 Sa[QT][2], Sb[QT][2];
      scores(buf, 0, Sa);
#pragma unroll
      for (int sub = 0; sub < NSUB; sub += 2) {
        if (sub + 1 < NSUB) scores(buf, sub + 1, Sb);
        accumulate(buf, sub, Sa);
        if (sub + 1 < NSUB) {
          if (sub + 2 < NSUB) scores(buf, sub + 2, Sa);
          accumulate(buf, sub + 1, Sb);
        }
      }
    }
    if (st + 1 < nstages) commit(buf ^ 1);
    __syncthreads();
  };

  fetch(0);
  commit(0);
  __syncthreads();
  int64_t st = 0;
  for (; st < nstages && !settled; ++st) stage(st, std::true_type{});
  for (; st < nstages; ++st) stage(st, std::false_type{});

  // Store the first Cout channels (C here is Cout rounded up to a multiple of 16).
  const int64_t BMC = (int64_t)gridDim.z * M * Cout;
  float* dst = out + split * BMC + bt * M * Cout;
  const bool vec = (Cout % 4) == 0;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int64_t i = row_base + qt * 16 + l16;
    if (i >= M) continue;
    const float scale = exp2_hw(mrow[qt]);
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const int c0 = 16 * ct + 4 * g;
      const f32x4 o = O[qt][ct] * scale;
      if (vec && c0 + 4 <= Cout) {
        *reinterpret_cast<f32x4*>(dst + i * Cout + c0) = o;
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (c0 + v < Cout) dst[i * Cout + c0 + v] = o[v];
      }
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
  HighdPlan p;
  const int Cp = padded_channels(C);
  p.Npad = padded_keys(N);
  p.row_blocks = ceil_div(M, kWaves * query_tiles(D, Cp) * 16);
  const int64_t blocks = p.row_blocks * B;
  const int64_t target = (int64_t)num_cus * kSplitTarget;
  int64_t S = blocks < target ? ceil_div(target, blocks) : 1;
  const int64_t max_split = p.Npad / (4 * kKeyPad) > 1 ? p.Npad / (4 * kKeyPad) : 1;
  if (S > max_split) S = max_split;
  int64_t kps = ceil_div(ceil_div(N, S), kKeyPad) * kKeyPad;
  S = ceil_div(N, kps);
  p.splits = S;
  p.kps = kps;
  p.beta_bytes = align_up((size_t)B * p.Npad * sizeof(float));
  p.vp_bytes = align_up((size_t)B * p.Npad * Cp * sizeof(_Float16));
  p.part_bytes = S > 1 ? align_up((size_t)S * B * M * C * sizeof(float)) : 0;
  p.total = p.beta_bytes + p.vp_bytes + p.part_bytes;
  return p;
}

}  // namespace

bool highd_supported(int D, int C) { return (D == 32 || D == 64) && C >= 1 && C <= 64; }

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
  const int Cp = padded_channels(C);
  highd_prep_kernel<<<dim3((unsigned)ceil_div(p.Npad, 256), (unsigned)B), 256, 0, s>>>(k, v, beta, vpm, N, p.Npad, D, C,
                                                                                       Cp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  float* dst = p.splits > 1 ? part : out;
  const dim3 grid((unsigned)p.row_blocks, (unsigned)p.splits, (unsigned)B);
#define KEOPS_HD(Dv, Cv)                                                                          \
  highd_kernel<Dv, Cv, query_tiles(Dv, Cv), kMinBlocks, kStageKeys, false><<<grid, 256, 0, s>>>( \
      q, k, beta, vpm, dst, M, N, p.Npad, p.kps, cs, C)
  if (D == 32 && Cp == 16) KEOPS_HD(32, 16);
  else if (D == 32 && Cp == 32) KEOPS_HD(32, 32);
  else if (D == 32 && Cp == 64) KEOPS_HD(32, 64);
  else if (D == 64 && Cp == 16) KEOPS_HD(64, 16);
  else if (D == 64 && Cp == 32) KEOPS_HD(64, 32);
  else if (D == 64 && Cp == 64) KEOPS_HD(64, 64);
  else return hipErrorInvalidValue;
#undef KEOPS_HD
  e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const int64_t n = B * M * C;
  highd_combine_kernel<<<(unsigned)ceil_div(n, 256), 256, 0, s>>>(part, out, n, p.splits);
  return hipGetLastError();
}

}  // namespace keops
