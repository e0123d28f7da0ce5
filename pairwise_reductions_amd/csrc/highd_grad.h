// Matrix-core gradient sweep of the batched Gauss sum. Included by the per-feature-width
// sources, each of which instantiates grad_launch<Dp> for one padded D.
//
// For s_i = sum_j Phi_ij v_j ("Fast Gauss Sums via Flash Attention", eq. (1)) and an upstream
// gradient g_i = dL/ds_i, the chain rule through Phi_ij = exp(-tau/2 ||q_i - k_j||^2) gives
//   dL/dq_i = -tau sum_j W_ij (q_i - k_j),   W_ij = Phi_ij (g_i . v_j),
//   dL/dk_j = -tau sum_i W_ij (k_j - q_i),
// the second being the first with the roles of the two point sets (and of g and v) swapped.
// One kernel therefore serves both: rows x_i with weights a_i, columns y_j with weights bv_j,
//   G_i = -tau sum_j W_ij (x_i - y_j) = -tau (x_i sum_j W_ij - sum_j W_ij y_j).
// Per 32-key subtile and 16-row tile, on v_mfma_f32_16x16x32_f16:
//   S^T  = Y X^T + beta          (as in the forward kernel)
//   dP^T = Bv' A'^T              (K = the weight channels, padded to a multiple of 32)
//   W    = 2^(cs S' + alpha) * dP, rounded to fp16 in the lanes that computed it
//   O^T += Y'^T W^T              (Y' = the columns plus a channel of ones, so the row sums
//                                 sum_j W_ij come out of the same product)
// With CB > 0 the same sweep also accumulates the plain weighted sum O2^T += Bv'^T P^T over the
// kernel values P (before the dP factor), which in the y-gradient role (rows y, columns x,
// column weights g) is the gradient with respect to b, sum_i Phi_ij g_i, at the cost of one
// conversion per kernel value and CB/16 more MFMAs, with no further exponential.
// Overflow of W in fp16 is ruled out by scaling: a'_i = a_i/|a_i| and bv'_j = bv_j/|bv_j| have
// unit norm, so |a'.bv'| <= 1, and log2(|bv_j| / max_j |bv_j|) is folded into beta_j, so the
// tracked exponent still never exceeds zero before the shift. The epilogue restores
// |a_i| * max_j |bv_j| * 2^m_i.
#pragma once

#include "highd_common.h"

#include <math.h>

#include <type_traits>

namespace keops {
namespace hd {
namespace {

template <int D, int CK, int QT, int kStage, int CB, int kW>
__global__ void __launch_bounds__(64 * kW, 1)
grad_kernel(const _Float16* __restrict__ x, const _Float16* __restrict__ y, const _Float16* __restrict__ ap,
            const float* __restrict__ rho, const float* __restrict__ beta, const _Float16* __restrict__ bvp,
            const _Float16* __restrict__ yp, const _Float16* __restrict__ gp, const float* __restrict__ oscale,
            float* __restrict__ out, float* __restrict__ out2, int64_t M, int64_t N, int64_t Npad, int64_t kps,
            float cs, float tau, int Din, int Cout2) {
  constexpr int DS = D / 32;           // K-steps of S^T
  constexpr int KS = CK / 32;          // K-steps of dP^T
  constexpr int YC = D + 16;           // channels of Y': D features, then the ones tile
  constexpr int OT = YC / 16;          // 16-channel output tiles
  constexpr int KP = D + 8;            // LDS row pitches, halves
  constexpr int AP = CK + 8;
  constexpr int VP = 32 + 8;
  constexpr int NSUB = kStage / 32;
  constexpr int kRowsPerBlock = kW * QT * 16;
  constexpr int kThreads = 64 * kW;
  __shared__ __attribute__((aligned(16))) _Float16 sK[2][kStage][KP];
  __shared__ __attribute__((aligned(16))) _Float16 sA[2][kStage][AP];
  __shared__ __attribute__((aligned(16))) _Float16 sY[2][NSUB][YC][VP];
  __shared__ __attribute__((aligned(16))) float sB[2][kStage];
  constexpr int CBT = CB > 0 ? CB / 16 : 1;  // 16-channel tiles of the second output
  __shared__ __attribute__((aligned(16))) _Float16 sG[2][NSUB][CB > 0 ? CB : 1][VP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, l16 = lane & 15;
  const int64_t bt = blockIdx.z, split = blockIdx.y;
  const int64_t j0 = split * kps;
  const int64_t j1 = (j0 + kps < N) ? j0 + kps : N;
  const int64_t nstages = hd_ceil_div(j1 - j0, kStage);
  const int64_t row_base = (int64_t)blockIdx.x * kRowsPerBlock + wave * (QT * 16);

  const _Float16* xb = x + bt * M * Din;
  const _Float16* yb = y + bt * N * Din;
  const _Float16* ab = ap + bt * M * CK;
  const float* bb = beta + bt * Npad;
  const _Float16* vb = bvp + bt * Npad * CK;
  const _Float16* pb = yp + bt * Npad * YC;
  const _Float16* gb = CB > 0 ? gp + bt * Npad * CB : nullptr;

  half8 qop[QT][DS], aop[QT][KS];
  float alpha[QT], mrow[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    int64_t i = row_base + qt * 16 + l16;
    i = i < M ? i : M - 1;
    float nrm = 0.0f;
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      const int col = 32 * ds + 8 * g;
      qop[qt][ds] = half8{};
      if (col < Din) qop[qt][ds] = *reinterpret_cast<const half8*>(xb + i * Din + col);
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
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) aop[qt][ks] = *reinterpret_cast<const half8*>(ab + i * CK + 32 * ks + 8 * g);
  }
  f32x4 O[QT][OT], O2[QT][CBT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
    for (int ot = 0; ot < OT; ++ot) O[qt][ot] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int cb = 0; cb < CBT; ++cb) O2[qt][cb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // Stage loads, global -> registers before the current stage is computed, registers -> LDS
  // after it. Each table is cut into 16-byte chunks dealt round-robin to the workgroup's threads.
  constexpr int kKChunks = kStage * D / 8, KCH = (kKChunks + kThreads - 1) / kThreads;
  constexpr int kAChunks = kStage * CK / 8, ACH = (kAChunks + kThreads - 1) / kThreads;
  constexpr int kYChunks = NSUB * YC * 4, YCH = (kYChunks + kThreads - 1) / kThreads;
  constexpr int kGChunks = CB > 0 ? NSUB * CB * 4 : 0, GCH = kGChunks > 0 ? (kGChunks + kThreads - 1) / kThreads : 1;
  static_assert(kStage / 4 <= kThreads && kStage % 32 == 0, "tile shapes");
  half8 rk[KCH], ra[ACH], ry[YCH], rg[GCH];
  f32x4 rb = {};
  auto fetch = [&](int64_t st) {
    const int64_t jb = j0 + st * kStage;
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int c = tid + kThreads * r;
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      const int64_t j = jb + row;
      rk[r] = half8{};
      if (c < kKChunks && j < j1 && col < Din) rk[r] = *reinterpret_cast<const half8*>(yb + j * Din + col);
    }
#pragma unroll
    for (int r = 0; r < ACH; ++r) {
      const int c = tid + kThreads * r;
      const int row = c / (CK / 8), col = (c % (CK / 8)) * 8;
      if (c < kAChunks) ra[r] = *reinterpret_cast<const half8*>(vb + (jb + row) * CK + col);
    }
#pragma unroll
    for (int r = 0; r < YCH; ++r) {
      const int c = tid + kThreads * r;
      const int t = c / (YC * 4), rem = c % (YC * 4), ch = rem / 4, part = (rem % 4) * 8;
      if (c < kYChunks) ry[r] = *reinterpret_cast<const half8*>(pb + ((jb / 32 + t) * YC + ch) * 32 + part);
    }
    if constexpr (CB > 0) {
#pragma unroll
      for (int r = 0; r < GCH; ++r) {
        const int c = tid + kThreads * r;
        const int t = c / (CB * 4), rem = c % (CB * 4), ch = rem / 4, part = (rem % 4) * 8;
        if (c < kGChunks) rg[r] = *reinterpret_cast<const half8*>(gb + ((jb / 32 + t) * CB + ch) * 32 + part);
      }
    }
    if (tid < kStage / 4) rb = *reinterpret_cast<const f32x4*>(bb + jb + 4 * tid);
  };
  auto commit = [&](int buf) {
#pragma unroll
    for (int r = 0; r < KCH; ++r) {
      const int c = tid + kThreads * r;
      if (c < kKChunks) *reinterpret_cast<half8*>(&sK[buf][c / (D / 8)][(c % (D / 8)) * 8]) = rk[r];
    }
#pragma unroll
    for (int r = 0; r < ACH; ++r) {
      const int c = tid + kThreads * r;
      if (c < kAChunks) *reinterpret_cast<half8*>(&sA[buf][c / (CK / 8)][(c % (CK / 8)) * 8]) = ra[r];
    }
#pragma unroll
    for (int r = 0; r < YCH; ++r) {
      const int c = tid + kThreads * r;
      const int t = c / (YC * 4), rem = c % (YC * 4);
      if (c < kYChunks) *reinterpret_cast<half8*>(&sY[buf][t][rem / 4][(rem % 4) * 8]) = ry[r];
    }
    if constexpr (CB > 0) {
#pragma unroll
      for (int r = 0; r < GCH; ++r) {
        const int c = tid + kThreads * r;
        const int t = c / (CB * 4), rem = c % (CB * 4);
        if (c < kGChunks) *reinterpret_cast<half8*>(&sG[buf][t][rem / 4][(rem % 4) * 8]) = rg[r];
      }
    }
    if (tid < kStage / 4) *reinterpret_cast<f32x4*>(&sB[buf][4 * tid]) = rb;
  };

  // Row shifts, as in the forward kernel: once m_i >= -kSlack every later scaled kernel value
  // is at most 2^kSlack, so the tracking stops for the whole wave.
  bool first = true, settled = false;
  // One stage. Per 32-key subtile the key, weight and column operands are read from LDS once;
  // then each row tile runs S'^T and dP^T, the row-shift update while tracking,
  // W = 2^(cs S' + alpha) dP in fp16 and O^T += Y'^T W^T, one tile at a time so that only one
  // tile's products are live.
  auto stage = [&](int64_t st, auto track) {
    constexpr bool kTrack = decltype(track)::value;
    const int buf = (int)(st & 1);
    if (st + 1 < nstages) fetch(st + 1);
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      half8 kop[2][DS], bop[2][KS];
      f32x4 bc[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int key = sub * 32 + 16 * hh + l16;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) kop[hh][ds] = *reinterpret_cast<const half8*>(&sK[buf][key][32 * ds + 8 * g]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) bop[hh][ks] = *reinterpret_cast<const half8*>(&sA[buf][key][32 * ks + 8 * g]);
        bc[hh] = *reinterpret_cast<const f32x4*>(&sB[buf][sub * 32 + 16 * hh + 4 * g]);
      }
      half8 yop[OT], gop[CBT];
#pragma unroll
      for (int ot = 0; ot < OT; ++ot) yop[ot] = *reinterpret_cast<const half8*>(&sY[buf][sub][16 * ot + l16][8 * g]);
      if constexpr (CB > 0) {
#pragma unroll
        for (int cb = 0; cb < CBT; ++cb)
          gop[cb] = *reinterpret_cast<const half8*>(&sG[buf][sub][16 * cb + l16][8 * g]);
      }
      bool all_settled = true;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        f32x4 S[2], P[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          S[hh] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[hh][0], qop[qt][0], bc[hh], 0, 0, 0);
#pragma unroll
          for (int ds = 1; ds < DS; ++ds)
            S[hh] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop[hh][ds], qop[qt][ds], S[hh], 0, 0, 0);
          P[hh] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bop[hh][0], aop[qt][0], f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0,
                                                         0);
#pragma unroll
          for (int ks = 1; ks < KS; ++ks)
            P[hh] = __builtin_amdgcn_mfma_f32_16x16x32_f16(bop[hh][ks], aop[qt][ks], P[hh], 0, 0, 0);
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
          for (int ot = 0; ot < OT; ++ot) O[qt][ot] *= sc;
          if constexpr (CB > 0) {
#pragma unroll
            for (int cb = 0; cb < CBT; ++cb) O2[qt][cb] *= sc;
          }
          all_settled = all_settled && (mrow[qt] >= -kSlack);
        }
        half8 wb, pb8;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const float pv = exp2_hw(fmaf(S[s >> 2][s & 3], cs, alpha[qt]));
          wb[s] = (_Float16)(pv * P[s >> 2][s & 3]);
          if constexpr (CB > 0) pb8[s] = (_Float16)pv;
        }
#pragma unroll
        for (int ot = 0; ot < OT; ++ot)
          O[qt][ot] = __builtin_amdgcn_mfma_f32_16x16x32_f16(yop[ot], wb, O[qt][ot], 0, 0, 0);
        if constexpr (CB > 0) {
#pragma unroll
          for (int cb = 0; cb < CBT; ++cb)
            O2[qt][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(gop[cb], pb8, O2[qt][cb], 0, 0, 0);
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

  fetch(0);
  commit(0);
  __syncthreads();
  int64_t st = 0;
  for (; st < nstages && !settled; ++st) stage(st, std::true_type{});
  for (; st < nstages; ++st) stage(st, std::false_type{});

  // G_i = -tau 2^m_i |a_i| max|bv| (x_i * sum_j W'_ij - sum_j W'_ij y_j). The row sum is
  // channel D, held in element 0 by the lanes of group 0.
  float rsum[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) rsum[qt] = __shfl(O[qt][OT - 1][0], l16);
  const int64_t BMD = (int64_t)gridDim.z * M * Din;
  float* dst = out + split * BMD + bt * M * Din;
  const float osc = oscale[bt];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int64_t i = row_base + qt * 16 + l16;
    if (i >= M) continue;
    const float scale = -tau * exp2_hw(mrow[qt]) * rho[bt * M + i] * osc;
#pragma unroll
    for (int ot = 0; ot < OT - 1; ++ot) {
      const int d0 = 16 * ot + 4 * g;
      if (d0 >= Din) continue;  // Din is a multiple of 16, so d0 < Din means d0 + 4 <= Din
      const half4 xv = *reinterpret_cast<const half4*>(xb + i * Din + d0);
      f32x4 o;
#pragma unroll
      for (int v = 0; v < 4; ++v) o[v] = scale * fmaf((float)xv[v], rsum[qt], -O[qt][ot][v]);
      *reinterpret_cast<f32x4*>(dst + i * Din + d0) = o;
    }
  }
  // Second output: sum_j Phi_ij bv_j = 2^m_i max|bv| sum_j P'_ij bv'_j, first Cout2 channels.
  if constexpr (CB > 0) {
    float* dst2 = out2 + (split * gridDim.z + bt) * M * Cout2;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int64_t i = row_base + qt * 16 + l16;
      if (i >= M) continue;
      const float scale = exp2_hw(mrow[qt]) * osc;
#pragma unroll
      for (int cb = 0; cb < CBT; ++cb)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int c = 16 * cb + 4 * g + v;
          if (c < Cout2) dst2[i * Cout2 + c] = scale * O2[qt][cb][v];
        }
    }
  }
}

}  // namespace

template <int Dp>
hipError_t grad_launch(const GradArgs& a) {
  constexpr int kStage = grad_stage(Dp), kW = grad_waves(Dp);
#define KEOPS_GRAD(CKv, CBv)                                                                                     \
  grad_kernel<Dp, CKv, grad_query_tiles(Dp, CKv, CBv), kStage, CBv, kW><<<a.grid, 64 * kW, 0, a.stream>>>(       \
      a.x, a.y, a.ap, a.rho, a.beta, a.bvp, a.yp, a.gp, a.oscale, a.out, a.out2, a.M, a.N, a.Npad, a.kps, a.cs, \
      a.tau, a.D, a.C2)
  if (a.out2) {
    if (a.Ck == 32) KEOPS_GRAD(32, 16);
    else return hipErrorInvalidValue;
  } else if (a.Ck == 32) {
    KEOPS_GRAD(32, 0);
  } else {
    KEOPS_GRAD(64, 0);
  }
#undef KEOPS_GRAD
  return hipGetLastError();
}

}  // namespace hd
}  // namespace keops
