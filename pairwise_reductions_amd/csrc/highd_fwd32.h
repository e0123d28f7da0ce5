// Forward matrix-core Gauss sum on 32x32x16 tiles ("Fast Gauss Sums via Flash Attention",
// eq. (1)), for fp16 or bf16 inputs with D <= 32 and 17 <= C <= 32 (both padded to 32). The
// arithmetic is that of fwd_kernel in highd_fwd.h, on tiles of 32 queries x 32 keys:
//   S'^T = K Q^T + B   two 32x32x16 MFMAs (features 0-15, 16-31), the accumulator starting
//                      from beta of each lane's keys;
//   P = 2^(cs S' + alpha) rounded to fp16;  O^T += V^T P^T   two 32x32x16 MFMAs (keys 0-15,
//                      16-31), all 32 channels at once.
// Per 1024 pairs a wave issues 4 MFMAs where the 16x16x32 form issues 8 for the same matrix
// work; on this chip the smaller number interferes less with the exponentials issued beside
// them (a register-only replica of the unit costs 60.7 ns per 512 pairs at two waves per SIMD
// against 71.4 ns on 16x16x32 tiles).
// Lane (g, l) (g = lane / 32, l = lane % 32) holds, in S'^T and O^T, rows 8(v / 4) + 4g + v % 4
// (v < 16) of column l: keys of query l, and channels of query l. Its values v < 8 and v >= 8
// are then exactly its B operands of the two P^T products when each 32-key subtile's weights
// are stored in the slot32_key() order, so P never moves between lanes.
//
// fp16 inputs take the folded form of highd_common.h once a wave's rows are settled.
#pragma once

#include "highd_common.h"

#include <math.h>

#include <type_traits>

namespace keops {
namespace hd {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_32 __attribute__((ext_vector_type(8)));

template <typename TIn>
struct Raw8Of {
  using type = half8;
};
template <>
struct Raw8Of<__bf16> {
  using type = bf16x8_32;
};

template <typename TIn>
__device__ __forceinline__ f32x16 mfma32_s(const typename Raw8Of<TIn>::type& a, const typename Raw8Of<TIn>::type& b,
                                           const f32x16& c) {
  if constexpr (std::is_same<TIn, _Float16>::value)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <typename TIn, int QT, int kStage, int kW>
__global__ void __launch_bounds__(64 * kW, 1)
fwd32_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const float* __restrict__ beta,
             const _Float16* __restrict__ vp, float* __restrict__ out, const float* __restrict__ rscale,
             const float* __restrict__ oscale, int64_t M, int64_t N, int64_t Npad, int64_t kps, float cs, int Din,
             int Cout) {
  constexpr int D = 32, C = 32;
  constexpr int KP = D + 8;   // LDS row pitch of K, 16-bit elements
  constexpr int VP = 32 + 8;  // LDS row pitch of V^T, halves
  constexpr int NSUB = kStage / 32;
  constexpr int kRowsPerBlock = kW * QT * 32;
  constexpr int kThreads = 64 * kW;
  using Raw = typename std::conditional<std::is_same<TIn, __bf16>::value, __bf16, _Float16>::type;
  using Raw8 = typename Raw8Of<TIn>::type;
  __shared__ __attribute__((aligned(16))) Raw sK[2][kStage][KP];
  __shared__ __attribute__((aligned(16))) _Float16 sV[2][NSUB][C][VP];
  constexpr bool kFoldable = std::is_same<TIn, _Float16>::value;
  __shared__ __attribute__((aligned(16))) float sB[2][kStage];
  __shared__ __attribute__((aligned(16))) float sBs[2][kFoldable ? kStage : 4];  // cs beta
  __shared__ float sKn[kW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, l32 = lane & 31;
  const int64_t bt = blockIdx.z, split = blockIdx.y;
  const int64_t j0 = split * kps;
  const int64_t j1 = (j0 + kps < N) ? j0 + kps : N;
  const int64_t nstages = hd_ceil_div(j1 - j0, kStage);
  const int64_t row_base = (int64_t)blockIdx.x * kRowsPerBlock + wave * (QT * 32);

  const TIn* qb = q + bt * M * Din;
  const TIn* kb = k + bt * N * Din;
  const float* bb = beta + bt * Npad;
  const _Float16* vb = vp + bt * Npad * C;

  // query operands: features 16 kk + 8g .. 16 kk + 8g + 7 of query l (read as zero past Din)
  Raw8 qop[QT][2];
  float alpha[QT], mrow[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    int64_t i = row_base + qt * 32 + l32;
    i = i < M ? i : M - 1;
    float nrm = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int col = 16 * kk + 8 * g;
      Raw8 o = Raw8{};
      if (col < Din) o = *reinterpret_cast<const Raw8*>(qb + i * Din + col);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const float v = (float)o[s];
        nrm = fmaf(v, v, nrm);
      }
      qop[qt][kk] = o;
    }
    nrm += __shfl_xor(nrm, 32);
    alpha[qt] = -0.5f * cs * nrm;
    mrow[qt] = 0.0f;
  }
  f32x16 O[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) O[qt] = f32x16{};

  // Stage loads as in fwd_kernel: global -> registers before the current stage is computed,
  // registers -> LDS after it; 8-element chunks dealt round-robin to the workgroup's threads.
  constexpr int kKChunks = kStage * D / 8, KCH = (kKChunks + kThreads - 1) / kThreads;
  constexpr int kVChunks = NSUB * C * 4, VCH = (kVChunks + kThreads - 1) / kThreads;
  static_assert(kStage / 4 <= kThreads && kStage % 32 == 0, "tile shapes");
  Raw8 rk[KCH];
  half8 rv[VCH];
  f32x4 rb = {};
  auto fetch = [&](int64_t st) {
    const int64_t jb = j0 + st * kStage;
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int c = tid + kThreads * r;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      const int64_t j = jb + row;
      Raw8 o = Raw8{};
      if (c < kKChunks && j < j1 && col < Din) o = *reinterpret_cast<const Raw8*>(kb + j * Din + col);
      rk[r] = o;
    }
#pragma unroll
    for (int r = 0; r < VCH; ++r) {
      const int c = tid + kThreads * r;
      const int t = c / (C * 4), rem = c % (C * 4), ch = rem / 4, part = (rem % 4) * 8;
      if (c < kVChunks) rv[r] = *reinterpret_cast<const half8*>(vb + ((jb / 32 + t) * C + ch) * 32 + part);
    }
    if (tid < kStage / 4) rb = *reinterpret_cast<const f32x4*>(bb + jb + 4 * tid);
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int c = tid + kThreads * r;
      if (c < kKChunks) *reinterpret_cast<Raw8*>(&sK[buf][c / (D / 8)][(c % (D / 8)) * 8]) = rk[r];
    }
#pragma unroll
    for (int r = 0; r < VCH; ++r) {
      const int c = tid + kThreads * r;
      const int t = c / (C * 4), rem = c % (C * 4);
      if (c < kVChunks) *reinterpret_cast<half8*>(&sV[buf][t][rem / 4][(rem % 4) * 8]) = rv[r];
    }
    if (tid < kStage / 4) {
      *reinterpret_cast<f32x4*>(&sB[buf][4 * tid]) = rb;
      if constexpr (kFoldable) *reinterpret_cast<f32x4*>(&sBs[buf][4 * tid]) = rb * cs;
    }
  };

  // Operands of one 32-key subtile: key l's features (two K = 16 slices), beta of the lane's 16
  // keys, and the weights of channel l over the subtile's two 16-slot halves.
  struct Operands {
    Raw8 k[2];
    f32x16 b;
    half8 v[2];
  };
  auto read_operands = [&](int buf, int sub, Operands& o, auto folded) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) o.k[kk] = *reinterpret_cast<const Raw8*>(&sK[buf][sub * 32 + l32][16 * kk + 8 * g]);
    const float* srcb = decltype(folded)::value ? &sBs[buf][0] : &sB[buf][0];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(srcb + sub * 32 + 8 * w + 4 * g);
#pragma unroll
      for (int u = 0; u < 4; ++u) o.b[4 * w + u] = b4[u];
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) o.v[h] = *reinterpret_cast<const half8*>(&sV[buf][sub][l32][16 * h + 8 * g]);
  };
  auto score_with = [&](const Operands& o, int qt) -> f32x16 {
    f32x16 S = mfma32_s<TIn>(o.k[0], qop[qt][0], o.b);
    return mfma32_s<TIn>(o.k[1], qop[qt][1], S);
  };
  auto use = [&](const Operands& o, int qt, const f32x16& S, auto folded) {
    half8 pa, pb;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const _Float16 h = (_Float16)exp2_hw(decltype(folded)::value ? S[v] : fmaf(S[v], cs, alpha[qt]));
      if (v < 8) pa[v] = h;
      else pb[v - 8] = h;
    }
    O[qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(o.v[0], pa, O[qt], 0, 0, 0);
    O[qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(o.v[1], pb, O[qt], 0, 0, 0);
  };

  // Until every query of the wave is settled (shift m >= -kSlack: later kernel values are at
  // most 2^kSlack), each subtile raises the shifts where a term would exceed 2^kSlack (or sets
  // them, on the first subtile) and rescales O to match.
  bool first = true, settled = false;
  auto stage_track = [&](int64_t st) {
    const int buf = (int)(st & 1);
    if (st + 1 < nstages) fetch(st + 1);
#pragma unroll 1
    for (int sub = 0; sub < NSUB; ++sub) {
      Operands o;
      read_operands(buf, sub, o, std::false_type{});
      bool all_settled = true;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const f32x16 S = score_with(o, qt);
        float mx = S[0];
#pragma unroll
        for (int v = 1; v < 16; ++v) mx = fmaxf(mx, S[v]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float amax = fmaf(mx, cs, alpha[qt]);
        const float delta = (first || amax > kSlack) ? amax : 0.0f;
        alpha[qt] -= delta;
        mrow[qt] += delta;
        const float sc = (first || delta == 0.0f) ? 1.0f : exp2_hw(-delta);
        O[qt] *= sc;
        all_settled = all_settled && (mrow[qt] >= -kSlack);
        use(o, qt, S, std::false_type{});
      }
      settled = __all(all_settled);
      first = false;
    }
    if (st + 1 < nstages) commit(buf ^ 1);
    __syncthreads();
  };
  // Settled stages, software-pipelined over the stage's (subtile, query tile) units: the scores
  // of the next unit are issued before the exponentials of the current one, and the next
  // subtile's operands are read one subtile ahead (two sets alternate).
  auto stage_pipe = [&](int64_t st, auto folded) {
    const int buf = (int)(st & 1);
    if (st + 1 < nstages) fetch(st + 1);
    Operands ops[2];
    read_operands(buf, 0, ops[0], folded);
    f32x16 Sbuf[2];
    Sbuf[0] = score_with(ops[0], 0);
#pragma unroll
    for (int u = 0; u < NSUB * QT; ++u) {
      const int sub = u / QT, qt = u % QT;
      const Operands& cur = ops[sub & 1];
      if (qt == 0 && sub + 1 < NSUB) read_operands(buf, sub + 1, ops[(sub + 1) & 1], folded);
      if (u + 1 < NSUB * QT) {
        if (qt + 1 < QT)
          Sbuf[(u + 1) & 1] = score_with(cur, qt + 1);
        else
          Sbuf[(u + 1) & 1] = score_with(ops[(sub + 1) & 1], 0);
      }
      use(cur, qt, Sbuf[u & 1], folded);
    }
    if (st + 1 < nstages) commit(buf ^ 1);
    __syncthreads();
  };

  if constexpr (kFoldable) fold_key_norm(bb, j0, j1, tid, kThreads, lane, wave, sKn);
  fetch(0);
  commit(0);
  __syncthreads();
  int64_t st = 0;
  for (; st < nstages && !settled; ++st) stage_track(st);
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
        for (int kk = 0; kk < 2; ++kk) fold_rounding(qop[qt][kk], cs, dq, fits);
        dq += __shfl_xor(dq, 32);
        d2 = fmaxf(d2, dq);
      }
      folded = fold_decide(amin, amax, d2, fits, kn2);
      if (folded) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          O[qt] *= exp2_hw(-alpha[qt]);
          mrow[qt] += alpha[qt];
          alpha[qt] = 0.0f;
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) qop[qt][kk] = fold_scale(qop[qt][kk], cs);
        }
      }
    }
  }
  for (; st < nstages; ++st) {
    if (kFoldable && folded)
      stage_pipe(st, std::true_type{});
    else
      stage_pipe(st, std::false_type{});
  }

  // Store the first Cout channels: lane (g, l) holds channels 8w + 4g .. 8w + 4g + 3 of query l.
  const int64_t BMC = (int64_t)gridDim.z * M * Cout;
  float* dst = out + split * BMC + bt * M * Cout;
  const bool vec = (Cout % 4) == 0;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int64_t i = row_base + qt * 32 + l32;
    if (i >= M) continue;
    float scale = exp2_hw(mrow[qt]);
    if (rscale) scale *= rscale[bt * M + i];
    if (oscale) scale *= oscale[bt];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c0 = 8 * w + 4 * g;
      f32x4 o;
#pragma unroll
      for (int u = 0; u < 4; ++u) o[u] = O[qt][4 * w + u] * scale;
      if (vec && c0 + 4 <= Cout) {
        *reinterpret_cast<f32x4*>(dst + i * Cout + c0) = o;
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (c0 + u < Cout) dst[i * Cout + c0 + u] = o[u];
      }
    }
  }
}

}  // namespace

// Query tiles of 32 per wave, keys per LDS stage and waves per workgroup: 4 x 32 queries per
// wave and 8 waves share 128-key stages, the rows per workgroup of the 16x16 form at D = C = 32
// (so the column-split plan is the same).
template <typename TIn>
hipError_t fwd32_launch(const FwdArgs& a) {
  constexpr int kQT = 4, kStage = 128, kW = 8;
  fwd32_kernel<TIn, kQT, kStage, kW><<<a.grid, 64 * kW, 0, a.stream>>>(
      static_cast<const TIn*>(a.q), static_cast<const TIn*>(a.k), a.beta, a.vp, a.out, a.rscale, a.oscale, a.M, a.N,
      a.Npad, a.kps, a.cs, a.D, a.C);
  return hipGetLastError();
}

}  // namespace hd
}  // namespace keops
