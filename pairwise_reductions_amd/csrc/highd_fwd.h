// Forward matrix-core Gauss sum ("Fast Gauss Sums via Flash Attention", eq. (1), computed
// from the squared-norm expansion ||q - k||^2 = ||q||^2 + ||k||^2 - 2 q.k, so the O(M N D)
// part is a dense contraction on the matrix cores). Included by the per-feature-width
// sources, each of which instantiates fwd_launch<TIn, Dp> for one padded D.
//
// Tiles are 16 queries x 32 keys on 16x16x32 MFMAs. Per wave: QT query tiles.
//   S^T = K Q^T + B   one MFMA per 16 keys and 32 features; the accumulator starts from
//                     B[j] = beta_j, so S'_ij = q_i.k_j + beta_j comes out whole;
//   a_ij = cs S'_ij + alpha_i,  alpha_i = -cs |q_i|^2 / 2 - m_i   (one FMA);
//   P = 2^a rounded to fp16;  O^T += V^T P^T   one MFMA per 16 channels (K = 32 keys).
// P never moves between lanes (the key order of slot_key()); m_i is a running base-2 shift,
// set by the first subtile and raised only when a subtile would produce a term above
// 2^kSlack (then O is rescaled).
//
// Input types (TIn, the type of q and k):
//   _Float16  fp16 MFMAs throughout;
//   __bf16    S^T on bf16 MFMAs (exact products of the inputs), the weights arrive as a
//             normalised fp16 table, P and O as for fp16;
//   float     every operand is split into fp16 hi + lo parts (v = hi + lo to about 2^-22
//             relative) and each product takes three MFMAs, hi.hi + lo.hi + hi.lo (the lo.lo
//             term is below 2^-22); q and k are split as they are read, P in registers and
//             the weights by the column preparation. This keeps the matrix cores at float32
//             accuracy for the cost of three times the MFMA work.
#pragma once

#include "highd_common.h"

#include <math.h>

#include <type_traits>

namespace keops {
namespace hd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// One 8-feature slice of a point, as the S^T product consumes it.
template <typename TIn>
struct Op;
template <>
struct Op<_Float16> {
  half8 h;
};
template <>
struct Op<__bf16> {
  bf16x8 h;
};
template <>
struct Op<float> {
  half8 h, l;
};

template <typename TIn>
constexpr bool kSplit = std::is_same<TIn, float>::value;

// Read 8 consecutive elements at p (16-byte aligned) into an operand; with kNorm, add their
// squares to nrm in float32.
template <typename TIn, bool kNorm>
__device__ __forceinline__ Op<TIn> load_op(const TIn* p, float& nrm) {
  Op<TIn> o;
  if constexpr (kSplit<TIn>) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float v = s < 4 ? a[s] : b[s - 4];
      if constexpr (kNorm) nrm = fmaf(v, v, nrm);
      o.h[s] = (_Float16)v;
      o.l[s] = (_Float16)(v - (float)o.h[s]);
    }
  } else {
    if constexpr (std::is_same<TIn, _Float16>::value)
      o.h = *reinterpret_cast<const half8*>(p);
    else
      o.h = *reinterpret_cast<const bf16x8*>(p);
    if constexpr (kNorm) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float v = (float)o.h[s];
        nrm = fmaf(v, v, nrm);
      }
    }
  }
  return o;
}

template <typename TIn>
__device__ __forceinline__ Op<TIn> zero_op() {
  Op<TIn> o;
  if constexpr (kSplit<TIn>) {
    o.h = half8{};
    o.l = half8{};
  } else {
    o.h = decltype(o.h){};
  }
  return o;
}

// acc += k-slice (A operand, rows = keys) x q-slice (B operand, columns = queries)
template <typename TIn>
__device__ __forceinline__ f32x4 s_mfma(const Op<TIn>& k, const Op<TIn>& q, f32x4 acc) {
  if constexpr (kSplit<TIn>) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k.h, q.h, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(k.l, q.h, acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(k.h, q.l, acc, 0, 0, 0);
  } else if constexpr (std::is_same<TIn, _Float16>::value) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(k.h, q.h, acc, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(k.h, q.h, acc, 0, 0, 0);
  }
}

template <typename TIn, int D, int C, int QT, int kStage, bool kFused, int kW>
__global__ void __launch_bounds__(64 * kW, 1)
fwd_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const float* __restrict__ beta,
           const _Float16* __restrict__ vp, const _Float16* __restrict__ vpl, float* __restrict__ out,
           const float* __restrict__ rscale, const float* __restrict__ oscale, int64_t M, int64_t N, int64_t Npad,
           int64_t kps, float cs, int Din, int Cout) {
  constexpr bool SPLIT = kSplit<TIn>;
  constexpr int NP = SPLIT ? 2 : 1;  // operand parts kept in LDS (hi, lo)
  constexpr int DS = D / 32;         // K-steps of S^T
  constexpr int CT = C / 16;         // 16-channel output tiles
  constexpr int KP = D + 8;          // LDS row pitch of K, 16-bit elements
  constexpr int VP = 32 + 8;         // LDS row pitch of V^T, halves
  constexpr int NSUB = kStage / 32;
  constexpr int kRowsPerBlock = kW * QT * 16;
  constexpr int kThreads = 64 * kW;
  using Raw = typename std::conditional<std::is_same<TIn, __bf16>::value, __bf16, _Float16>::type;
  using Raw8 = decltype(Op<TIn>{}.h);
  __shared__ __attribute__((aligned(16))) Raw sK[NP][2][kStage][KP];
  __shared__ __attribute__((aligned(16))) _Float16 sV[NP][2][NSUB][C][VP];
  __shared__ __attribute__((aligned(16))) float sB[2][kStage];
  // fp16 inputs take the folded form of highd_common.h once a wave's rows are settled; cs beta
  // is kept beside beta for it
  constexpr bool kFoldable = std::is_same<TIn, _Float16>::value;
  __shared__ __attribute__((aligned(16))) float sBs[2][kFoldable ? kStage : 4];
  __shared__ float sKn[kW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t bt = blockIdx.z, split = blockIdx.y;
  const int64_t j0 = split * kps;
  const int64_t j1 = (j0 + kps < N) ? j0 + kps : N;
  const int64_t nstages = hd_ceil_div(j1 - j0, kStage);
  const int64_t row_base = (int64_t)blockIdx.x * kRowsPerBlock + wave * (QT * 16);

  // D is Din rounded up to a multiple of 32; the features Din <= d < D read as zero.
  const TIn* qb = q + bt * M * Din;
  const TIn* kb = k + bt * N * Din;
  const float* bb = beta + bt * Npad;
  const _Float16* vb[NP];
  vb[0] = vp + bt * Npad * C;
  if constexpr (SPLIT) vb[NP - 1] = vpl + bt * Npad * C;

  Op<TIn> qop[QT][DS];
  float alpha[QT], mrow[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    int64_t i = row_base + qt * 16 + l16;
    i = i < M ? i : M - 1;
    float nrm = 0.0f;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const int col = 32 * ds + 8 * g;
      qop[qt][ds] = col < Din ? load_op<TIn, true>(qb + i * Din + col, nrm) : zero_op<TIn>();
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
  // registers -> LDS (after it), so global latency hides behind the matrix work. Tables are
  // cut into 8-element chunks dealt round-robin to the workgroup's threads.
  constexpr int kKChunks = kStage * D / 8, KCH = (kKChunks + kThreads - 1) / kThreads;
  constexpr int kVChunks = NSUB * C * 4, VCH = (kVChunks + kThreads - 1) / kThreads;
  static_assert(kStage / 4 <= kThreads && kStage % 32 == 0, "tile shapes");
  Raw8 rk[NP][KCH];
  half8 rv[NP][VCH];
  f32x4 rb = {};
  auto fetch = [&](int64_t st) {
    const int64_t jb = j0 + st * kStage;
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int c = tid + kThreads * r;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      const int64_t j = jb + row;
      float unused = 0.0f;
      const Op<TIn> o = (c < kKChunks && j < j1 && col < Din) ? load_op<TIn, false>(kb + j * Din + col, unused)
                                                              : zero_op<TIn>();
      rk[0][r] = o.h;
      if constexpr (SPLIT) rk[NP - 1][r] = o.l;
    }
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int r = 0; r < VCH; ++r) {
        const int c = tid + kThreads * r;
        const int t = c / (C * 4), rem = c % (C * 4), ch = rem / 4, part = (rem % 4) * 8;
        if (c < kVChunks) rv[p][r] = *reinterpret_cast<const half8*>(vb[p] + ((jb / 32 + t) * C + ch) * 32 + part);
      }
    if (tid < kStage / 4) rb = *reinterpret_cast<const f32x4*>(bb + jb + 4 * tid);
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int p = 0; p < NP; ++p) {
#pragma unroll
      for (int r = 0; r < KCH; ++r) {
        const int c = tid + kThreads * r;
        if (c < kKChunks) *reinterpret_cast<Raw8*>(&sK[p][buf][c / (D / 8)][(c % (D / 8)) * 8]) = rk[p][r];
      }
#pragma unroll
      for (int r = 0; r < VCH; ++r) {
        const int c = tid + kThreads * r;
        const int t = c / (C * 4), rem = c % (C * 4);
        if (c < kVChunks) *reinterpret_cast<half8*>(&sV[p][buf][t][rem / 4][(rem % 4) * 8]) = rv[p][r];
      }
    }
    if (tid < kStage / 4) {
      *reinterpret_cast<f32x4*>(&sB[buf][4 * tid]) = rb;
      if constexpr (kFoldable) *reinterpret_cast<f32x4*>(&sBs[buf][4 * tid]) = rb * cs;
    }
  };

  // S'^T of one 32-key subtile for every query tile: S[qt][half] holds keys 16*half + 4g + v.
  auto scores = [&](int buf, int sub, f32x4 (&S)[QT][2], auto folded) {
    const float* srcb = decltype(folded)::value ? &sBs[buf][0] : &sB[buf][0];
    Op<TIn> kop[2][DS];
    f32x4 bc[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const int key = sub * 32 + 16 * hh + l16, col = 32 * ds + 8 * g;
        kop[hh][ds].h = *reinterpret_cast<const Raw8*>(&sK[0][buf][key][col]);
        if constexpr (SPLIT) kop[hh][ds].l = *reinterpret_cast<const half8*>(&sK[NP - 1][buf][key][col]);
      }
      bc[hh] = *reinterpret_cast<const f32x4*>(srcb + sub * 32 + 16 * hh + 4 * g);
    }
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        S[qt][hh] = s_mfma<TIn>(kop[hh][0], qop[qt][0], bc[hh]);
#pragma unroll
        for (int ds = 1; ds < DS; ++ds) S[qt][hh] = s_mfma<TIn>(kop[hh][ds], qop[qt][ds], S[qt][hh]);
      }
  };
  // P = 2^(c S' + alpha) in fp16 (hi and lo parts when split; 2^S' in the folded form) and
  // O^T += V^T P^T.
  auto accumulate = [&](int buf, int sub, const f32x4 (&S)[QT][2], auto folded) {
    half8 vop[NP][CT];
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        vop[p][ct] = *reinterpret_cast<const half8*>(&sV[p][buf][sub][16 * ct + l16][8 * g]);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      half8 ph, pl;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float e = S[qt][s >> 2][s & 3];
        const float pv = exp2_hw(decltype(folded)::value ? e : fmaf(e, cs, alpha[qt]));
        ph[s] = (_Float16)pv;
        if constexpr (SPLIT) pl[s] = (_Float16)(pv - (float)ph[s]);
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        O[qt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[0][ct], ph, O[qt][ct], 0, 0, 0);
        if constexpr (SPLIT) {
          O[qt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[NP - 1][ct], ph, O[qt][ct], 0, 0, 0);
          O[qt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[0][ct], pl, O[qt][ct], 0, 0, 0);
        }
      }
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
  // One stage, scores of every query tile first; both phases execute one barrier per stage,
  // so the workgroup stays in step.
  auto stage_batched = [&](int64_t st, auto track, auto folded) {
    constexpr bool kTrack = decltype(track)::value;
    const int buf = (int)(st & 1);
    if (st + 1 < nstages) fetch(st + 1);
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      f32x4 S[QT][2];
      scores(buf, sub, S, folded);
      if constexpr (kTrack) track_rows(S);
      accumulate(buf, sub, S, folded);
    }
    if (st + 1 < nstages) commit(buf ^ 1);
    __syncthreads();
  };

  // One stage. Per 32-key subtile the key and weight operands are read from LDS once, then
  // each query tile runs S'^T (two MFMAs per 32 features), the row-shift update while
  // tracking, P = 2^(cs S' + alpha) in fp16 and O^T += V^T P^T. Taking the tiles one at a
  // time keeps a single tile's scores live, which leaves room for two waves per SIMD at eight
  // tiles; both phases execute one barrier per stage, so the workgroup stays in step.
  auto stage_fused = [&](int64_t st, auto track) {
    constexpr bool kTrack = decltype(track)::value;
    const int buf = (int)(st & 1);
    if (st + 1 < nstages) fetch(st + 1);
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      Op<TIn> kop[2][DS];
      f32x4 bc[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
          const int key = sub * 32 + 16 * hh + l16, col = 32 * ds + 8 * g;
          kop[hh][ds].h = *reinterpret_cast<const Raw8*>(&sK[0][buf][key][col]);
          if constexpr (SPLIT) kop[hh][ds].l = *reinterpret_cast<const half8*>(&sK[NP - 1][buf][key][col]);
        }
        bc[hh] = *reinterpret_cast<const f32x4*>(&sB[buf][sub * 32 + 16 * hh + 4 * g]);
      }
      half8 vop[NP][CT];
#pragma unroll
      for (int p = 0; p < NP; ++p)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          vop[p][ct] = *reinterpret_cast<const half8*>(&sV[p][buf][sub][16 * ct + l16][8 * g]);
      bool all_settled = true;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        f32x4 S[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          S[hh] = s_mfma<TIn>(kop[hh][0], qop[qt][0], bc[hh]);
#pragma unroll
          for (int ds = 1; ds < DS; ++ds) S[hh] = s_mfma<TIn>(kop[hh][ds], qop[qt][ds], S[hh]);
        }
        if constexpr (kTrack) {
          float mx = fmaxf(fmaxf(fmaxf(S[0][0], S[0][1]), fmaxf(S[0][2], S[0][3])),
                           fmaxf(fmaxf(S[1][0], S[1][1]), fmaxf(S[1][2], S[1][3])));
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
        half8 ph, pl;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const float pv = exp2_hw(fmaf(S[s >> 2][s & 3], cs, alpha[qt]));
          ph[s] = (_Float16)pv;
          if constexpr (SPLIT) pl[s] = (_Float16)(pv - (float)ph[s]);
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          O[qt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[0][ct], ph, O[qt][ct], 0, 0, 0);
          if constexpr (SPLIT) {
            O[qt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[NP - 1][ct], ph, O[qt][ct], 0, 0, 0);
            O[qt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop[0][ct], pl, O[qt][ct], 0, 0, 0);
          }
        }
      }
      if constexpr (kTrack) {
        settled = __all(all_settled);
        first = false;
      }
    }
    if (st + 1 < nstages) commit(buf ^ 1);
    __syncthreads();
  };

  // Settled stages, software-pipelined over the stage's (subtile, query tile) units: the
  // scores of the next unit are issued on the matrix cores before the exponentials of the
  // current one (two score buffers alternate), and the next subtile's key, bias and weight
  // operands are read from LDS one subtile ahead (two operand sets alternate), so neither the
  // VALU nor the matrix cores wait on a result just requested.
  struct Operands {
    Op<TIn> k[2][DS];
    f32x4 b[2];
    half8 v[NP][CT];
  };
  auto read_operands = [&](int buf, int sub, Operands& o, auto folded) {
    const float* srcb = decltype(folded)::value ? &sBs[buf][0] : &sB[buf][0];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int ds = 0; ds < DS; ++ds) {
        const int key = sub * 32 + 16 * hh + l16, col = 32 * ds + 8 * g;
        o.k[hh][ds].h = *reinterpret_cast<const Raw8*>(&sK[0][buf][key][col]);
        if constexpr (SPLIT) o.k[hh][ds].l = *reinterpret_cast<const half8*>(&sK[NP - 1][buf][key][col]);
      }
      o.b[hh] = *reinterpret_cast<const f32x4*>(srcb + sub * 32 + 16 * hh + 4 * g);
    }
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        o.v[p][ct] = *reinterpret_cast<const half8*>(&sV[p][buf][sub][16 * ct + l16][8 * g]);
  };
  auto score_with = [&](const Operands& o, int qt, f32x4 (&S)[2]) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      S[hh] = s_mfma<TIn>(o.k[hh][0], qop[qt][0], o.b[hh]);
#pragma unroll
      for (int ds = 1; ds < DS; ++ds) S[hh] = s_mfma<TIn>(o.k[hh][ds], qop[qt][ds], S[hh]);
    }
  };
  auto stage_pipe = [&](int64_t st, auto folded) {
    const int buf = (int)(st & 1);
    if (st + 1 < nstages) fetch(st + 1);
    Operands ops[2];
    read_operands(buf, 0, ops[0], folded);
    f32x4 Sbuf[2][2];
    score_with(ops[0], 0, Sbuf[0]);
#pragma unroll
    for (int u = 0; u < NSUB * QT; ++u) {
      const int sub = u / QT, qt = u % QT;
      const Operands& cur = ops[sub & 1];
      if (qt == 0 && sub + 1 < NSUB) read_operands(buf, sub + 1, ops[(sub + 1) & 1], folded);
      if (u + 1 < NSUB * QT) {
        if (qt + 1 < QT)
          score_with(cur, qt + 1, Sbuf[(u + 1) & 1]);
        else
          score_with(ops[(sub + 1) & 1], 0, Sbuf[(u + 1) & 1]);
      }
      const f32x4(&S)[2] = Sbuf[u & 1];
      half8 ph, pl;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float e = S[s >> 2][s & 3];
        const float pv = exp2_hw(decltype(folded)::value ? e : fmaf(e, cs, alpha[qt]));
        ph[s] = (_Float16)pv;
        if constexpr (SPLIT) pl[s] = (_Float16)(pv - (float)ph[s]);
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        O[qt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur.v[0][ct], ph, O[qt][ct], 0, 0, 0);
        if constexpr (SPLIT) {
          O[qt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur.v[NP - 1][ct], ph, O[qt][ct], 0, 0, 0);
          O[qt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(cur.v[0][ct], pl, O[qt][ct], 0, 0, 0);
        }
      }
    }
    if (st + 1 < nstages) commit(buf ^ 1);
    __syncthreads();
  };

  if constexpr (kFoldable) fold_key_norm(bb, j0, j1, tid, kThreads, lane, wave, sKn);
  fetch(0);
  commit(0);
  __syncthreads();
  int64_t st = 0;
  if constexpr (kFused) {
    for (; st < nstages && !settled; ++st) stage_fused(st, std::true_type{});
  } else {
    for (; st < nstages && !settled; ++st) stage_batched(st, std::true_type{}, std::false_type{});
  }
  bool folded = false;
  if constexpr (kFoldable) {
    if (settled && st < nstages) {
      float kn2 = 0.0f;
#pragma unroll
      for (int w = 0; w < kW; ++w) kn2 = fmaxf(kn2, sKn[w]);
      float amin = alpha[0], amax = alpha[0], d2 = 0.0f;
      bool fits = true;  // every cs q_d rounds to a finite fp16 value
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        amin = fminf(amin, alpha[qt]);
        amax = fmaxf(amax, alpha[qt]);
        float dq = 0.0f;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) fold_rounding(qop[qt][ds].h, cs, dq, fits);
        dq += __shfl_xor(dq, 16);
        dq += __shfl_xor(dq, 32);
        d2 = fmaxf(d2, dq);
      }
      folded = fold_decide(amin, amax, d2, fits, kn2);
      if (folded) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) O[qt][ct] *= exp2_hw(-alpha[qt]);
          mrow[qt] += alpha[qt];
          alpha[qt] = 0.0f;
#pragma unroll
          for (int ds = 0; ds < DS; ++ds) qop[qt][ds].h = fold_scale(qop[qt][ds].h, cs);
        }
      }
    }
  }
  for (; st < nstages; ++st) {
    if constexpr (kFused) {
      if (kFoldable && folded)
        stage_pipe(st, std::true_type{});
      else
        stage_pipe(st, std::false_type{});
    } else {
      if (kFoldable && folded)
        stage_batched(st, std::false_type{}, std::true_type{});
      else
        stage_batched(st, std::false_type{}, std::false_type{});
    }
  }

  // Store the first Cout channels (C here is Cout rounded up to a multiple of 16).
  const int64_t BMC = (int64_t)gridDim.z * M * Cout;
  float* dst = out + split * BMC + bt * M * Cout;
  const bool vec = (Cout % 4) == 0;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int64_t i = row_base + qt * 16 + l16;
    if (i >= M) continue;
    float scale = exp2_hw(mrow[qt]);
    if (rscale) scale *= rscale[bt * M + i];
    if (oscale) scale *= oscale[bt];
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

}  // namespace

template <typename TIn, int Dp>
hipError_t fwd_launch(const FwdArgs& a) {
  const int Cp = padded_channels(a.C);
  const TIn* q = static_cast<const TIn*>(a.q);
  const TIn* k = static_cast<const TIn*>(a.k);
#define KEOPS_FWD(Cv)                                                                                       \
  fwd_kernel<TIn, Dp, Cv, fwd_query_tiles(Dp, Cv, kSplit<TIn>), fwd_stage(Dp, Cv, kSplit<TIn>),                 \
             fwd_fused(Dp, Cv, kSplit<TIn>),                                                                       \
             fwd_waves(Dp, Cv, kSplit<TIn>)>                                                                       \
      <<<a.grid, 64 * fwd_waves(Dp, Cv, kSplit<TIn>), 0, a.stream>>>(                                             \
      q, k, a.beta, a.vp, a.vpl, a.out, a.rscale, a.oscale, a.M, a.N, a.Npad, a.kps, a.cs, a.D, a.C)
  if (Cp == 16) {
    KEOPS_FWD(16);
  } else if (Cp == 32) {
    // fp16 and bf16 at D = C = 32 (padded) run as fwd32_kernel
    if constexpr (!kSplit<TIn> && Dp == 32) return hipErrorInvalidValue;
    else KEOPS_FWD(32);
  } else {
    KEOPS_FWD(64);
  }
#undef KEOPS_FWD
  return hipGetLastError();
}

}  // namespace hd
}  // namespace keops
