// Shared pieces of the matrix-core (fp16) Gauss-sum kernels: tile constants, the key order
// inside a 32-key subtile, and the argument blocks of the per-feature-width launchers.
// Internal to the library.
//
// Notation ("Fast Gauss Sums via Flash Attention", eq. (1)): queries q_i (rows), keys k_j
// (columns), Phi_ij = exp(-tau/2 ||q_i - k_j||^2), tau = 1/sigma^2, cs = tau log2(e).
#pragma once

#include "internal.h"

namespace keops {
namespace hd {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;           // waves per workgroup
constexpr int kStageKeys = 64;      // keys per LDS stage (two 32-key subtiles)
constexpr int kSplitTarget = 2;     // column splits aim for this many workgroups per CU
constexpr int kKeyPad = 256;        // key counts are padded to a multiple of this
constexpr float kSlack = 8.0f;      // scaled kernel values may reach 2^kSlack before a rescale
constexpr float kLogFloor = -60.0f; // log2 of the smallest column weight kept apart from zero

// Query tiles (16 rows each) per wave, forward kernel. Measured on B=4, 16384^2, D=C=32: more
// independent tiles per wave beat more resident waves, since the matrix cores and the exp
// pipe overlap within a wave. Wider tiles take fewer to stay within 256 VGPRs.
// Float32 inputs (split into fp16 hi + lo parts) hold twice the operands, so they take fewer.
constexpr int fwd_query_tiles(int D, int C, bool split) {
  return split ? ((D <= 64 && C <= 32) || D == 32 ? 4 : (D > 64 && C == 64 ? 1 : 2))
               : ((D == 32 && C <= 32) ? 8 : (D <= 64 ? 4 : 2));
}
// The fused form scores and uses one query tile at a time while rows are tracked and runs
// software-pipelined settled stages (fwd_kernel's stage_fused / stage_pipe); the other form
// scores every tile of a subtile first. The fused form is taken with C <= 32 (measured faster
// at every D with eight-wave, 128-key stages) and wherever the batched order would need more
// than 256 VGPRs (one wave per SIMD), as at D = C = 64.
constexpr bool fwd_fused(int D, int C, bool split) {
  return split ? (C == 64 && D >= 64) : (C <= 32 || (D == 64 && C == 64));
}
// Keys per LDS stage and waves per workgroup of the forward kernel. With C <= 32 (fp16 or bf16)
// eight waves (two per SIMD) share one stage of 128 keys: fewer stage barriers per key, and the
// barrier keeps the two waves of a SIMD in step (at D = 128 the stage takes 92 KB of LDS: one
// such workgroup per CU, still two waves per SIMD). Measured at B = 4, 16384^2: the D = C = 32
// sweep took 186 us with four waves and 64-key stages, 175 us like this; with the
// software-pipelined stages of fwd_fused the C = 1 forward went 0.167 -> 0.157 ms per call, and
// at B = 64, C = 1 the D = 64 / 128 sweeps 2.94 -> 2.71 / 5.54 -> 4.84 ms. Float32 inputs (two
// operand parts in LDS) take eight waves too, with 64-key stages at C <= 16 and at D = 32 (32
// elsewhere, where 64 would spill): the B = 4, 16384^2, D = C = 32 sweep 0.558 -> 0.490 ms and the B = 64,
// C = 1 D sweep 6.16 / 6.21 / 7.90 / 17.6 -> 5.44 / 5.48 / 7.47 / 14.7 ms at D = 16 / 32 / 64 /
// 128, against four waves and 32-key stages.
constexpr int fwd_stage(int D, int C, bool split) {
  return split ? ((C <= 16 || (D == 32 && C <= 32)) ? 64 : 32) : (C <= 32 ? 128 : kStageKeys);
}
constexpr int fwd_waves(int D, int C, bool split) { return (split || C <= 32) ? 8 : kWaves; }
// The gradient kernel holds three products per subtile, so it takes fewer.
// (Sizes chosen so every instantiation fits 256 VGPRs, i.e. two waves per SIMD.)
constexpr int grad_query_tiles(int D, int CK, int CB) { return D <= 32 ? (CK <= 32 && CB == 0 ? 4 : 2) : 1; }
// Waves per workgroup and keys per LDS stage of the gradient sweep.
constexpr int grad_waves(int D) { return D <= 32 ? 8 : kWaves; }
constexpr int grad_stage(int D) { return D <= 64 ? kStageKeys : 32; }
// The gradient sweep can also produce the weights' gradient (a second output of at most
// kFusedWeightChannels channels) from the same kernel values.
constexpr int kFusedWeightChannels = 16;
// Features run in steps of 32 (the K of one MFMA) and are read as zero past D; output and
// weight channels run in tiles of 16.
constexpr int padded_features(int D) { return (D + 31) / 32 * 32; }
constexpr int padded_channels(int C) { return C <= 16 ? 16 : (C <= 32 ? 32 : 64); }
// Channel count of the gradient's weight vectors (the K of the dP product): a multiple of 32.
constexpr int padded_k_channels(int C) { return C <= 32 ? 32 : 64; }

__device__ __forceinline__ float exp2_hw(float v) { return __builtin_amdgcn_exp2f(v); }

// Folded form of the fp16 forward sweeps. Once a wave's rows are settled, the per-value FMA
// cs S' + alpha can go: with the query operands replaced by qs = fp16(cs q) and the accumulator
// starting from cs beta (kept in LDS beside beta), the MFMA returns the unshifted exponent
// itself, and each row's own shift alpha_i moves into its output scale (O_i is multiplied by
// 2^-alpha_i once). That needs alpha_i in [-kFoldLow, kFoldHigh]: later terms, at most 2^kSlack
// under the row shift, stay below 2^(kSlack + kFoldLow) = 2^15 (fp16 holds up to 65504), and no
// row's terms move more than kFoldHigh binades towards the fp16 subnormals. The rounding of cs q
// moves each exponent by e_ij = sum_d (qs_d - cs q_d) k_jd, |e_ij| <= |qs_i - cs q_i| |k_j|; a
// wave takes the folded form only where that bound, with the largest |k_j| of its column split,
// is at most 2^-9.5: each term then changes by a factor within 2^(+-2^-9.5), i.e. by less than
// 9.6e-4, and with the fp16 rounding of P (2^-11) by less than 1.45e-3 in all, inside the fp16
// path's 2e-3. Otherwise it keeps the FMA.
constexpr float kFoldLow = 7.0f, kFoldHigh = 4.0f;
// Largest |qs - cs q|^2 |k|^2 of the folded form: (2^-9.5)^2, less 2^-8 of it for the float32
// rounding of the quantities it is computed from.
constexpr float kFoldErr2 = 1.9073486328125e-06f * (1.0f - 0.00390625f);

// Largest squared key norm over the keys [j0, j1) of a column split, from beta_j <= -|k_j|^2/2,
// left by every wave in red[wave] (read after the next barrier).
__device__ __forceinline__ void fold_key_norm(const float* bb, int64_t j0, int64_t j1, int tid, int nthreads,
                                              int lane, int wave, float* red) {
  float kn = 0.0f;
  for (int64_t j = j0 + tid; j < j1; j += nthreads) kn = fmaxf(kn, -2.0f * bb[j]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) kn = fmaxf(kn, __shfl_xor(kn, o));
  if (lane == 0) red[wave] = kn;
}

// Squared rounding error of fp16(cs x) over the 8 features of one operand, accumulated into d2;
// fits turns false where a product leaves the fp16 range.
__device__ __forceinline__ void fold_rounding(const half8& x, float cs, float& d2, bool& fits) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float cq = cs * (float)x[e];
    fits = fits && fabsf(cq) < 65504.0f;
    const float dd = fits ? (float)(_Float16)cq - cq : 0.0f;
    d2 = fmaf(dd, dd, d2);
  }
}

// The wave's decision: shifts in range, every product finite, and the rounding bound met
// (amin, amax over the lane's rows; d2 the largest full-row squared rounding error of its rows;
// kn2 the split's largest squared key norm).
__device__ __forceinline__ bool fold_decide(float amin, float amax, float d2, bool fits, float kn2) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    amin = fminf(amin, __shfl_xor(amin, o));
    amax = fmaxf(amax, __shfl_xor(amax, o));
    d2 = fmaxf(d2, __shfl_xor(d2, o));
  }
  return __all(fits) && (amin >= -kFoldLow) && (amax <= kFoldHigh) && (d2 * kn2 <= kFoldErr2);
}

// The folded query operand: each feature times cs, rounded to fp16 (the rounding fold_rounding
// measured).
__device__ __forceinline__ half8 fold_scale(const half8& x, float cs) {
  half8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (_Float16)(cs * (float)x[e]);
  return r;
}

__host__ __device__ inline int64_t hd_ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline int64_t padded_keys(int64_t N) { return hd_ceil_div(N, kKeyPad) * kKeyPad; }

// In the accumulator of a 16x16 MFMA tile S^T (rows = keys, columns = queries) a lane of
// 16-lane group g holds keys 4g..4g+3 of its column. Over the two 16-key halves of a 32-key
// subtile that is 8 values, which are exactly the lane's fp16 B operand of a K = 32 product
// when the subtile's keys are taken in the order slot_key(): slot 8g + s holds key
// 4g + (s & 3) + 16 (s >> 2). Matrices that multiply P^T are therefore stored with their
// key axis permuted by key_slot(), the inverse.
__host__ __device__ inline int slot_key(int slot) {
  const int g = slot >> 3, s = slot & 7;
  return 4 * g + (s & 3) + 16 * (s >> 2);
}
__host__ __device__ inline int key_slot(int o) {
  const int half = o >> 4, rem = o & 15;
  return 8 * (rem >> 2) + 4 * half + (rem & 3);
}
// The same for 32x32x16 MFMA tiles: a lane of 32-lane group g holds keys 8w + 4g + (v & 3)
// (w = v >> 2, v < 16) of its column of S^T, and the two K = 16 products of P^T take values
// v < 8 and v >= 8. So slot 16h + 8g + s holds key 16h + 8(s >> 2) + 4g + (s & 3).
__host__ __device__ inline int slot32_key(int slot) {
  const int h = slot >> 4, g = (slot >> 3) & 1, s = slot & 7;
  return 16 * h + 8 * (s >> 2) + 4 * g + (s & 3);
}

// The forward on 32x32x16 tiles (fwd32_kernel): fp16 or bf16 inputs with D <= 32 and
// 17 <= C <= 32 (padded to 32 features and 32 channels). Its column weights are stored in the
// slot32_key() order.
inline bool fwd_square(bool split, int Dp, int Cp) { return !split && Dp == 32 && Cp == 32; }

// Forward: out[split][t][i][c] = oscale[t] * rscale[t][i] * sum_j Phi_ij vp_j[c] over the
// split's keys, where the stored column weights vp and the key terms beta may carry a per-key
// factor (see the column preparation in highd.hip).
struct FwdArgs {
  const void* q;           // [B][M][D] of the input type
  const void* k;           // [B][N][D] of the input type
  const float* beta;       // [B][Npad]: -|k_j|^2/2 (+ log2 of the key weight / cs), -inf past N
  const _Float16* vp;      // [B][Npad/32][Cp][32] key-permuted column weights
  const _Float16* vpl;     // the same for the lo parts (float32 inputs), else null
  float* out;              // [S][B][M][C]
  const float* rscale;     // [B][M] or null
  const float* oscale;     // [B] or null
  int64_t M, N, Npad, kps;
  float cs;
  int D, C;
  dim3 grid;
  hipStream_t stream;
};

// Gradient sweep: out[split][t][i][d] = -tau * scale_i * sum_j W_ij (x_i - y_j)_d with
// W_ij = Phi_ij (a'_i . bv'_j); see highd_grad.h.
struct GradArgs {
  const _Float16* x;       // [B][M][D] rows
  const _Float16* y;       // [B][N][D] columns
  const _Float16* ap;      // [B][M][Ck] unit-norm row weights a'_i
  const float* rho;        // [B][M] their norms
  const float* beta;       // [B][Npad]
  const _Float16* bvp;     // [B][Npad][Ck] unit-norm column weights bv'_j
  const _Float16* yp;      // [B][Npad/32][Dp + 16][32] key-permuted columns plus a ones channel
  const float* oscale;     // [B] largest column weight norm
  float* out;              // [S][B][M][D]
  const _Float16* gp;      // [B][Npad/32][16][32] key-permuted unit column weights (second output), or null
  float* out2;             // [S][B][M][C2] second output sum_j Phi_ij bv_j, or null
  int64_t M, N, Npad, kps;
  float cs, tau;
  int D, Ck, C2;
  dim3 grid;
  hipStream_t stream;
};

template <typename TIn, int Dp>
hipError_t fwd_launch(const FwdArgs& a);
template <typename TIn>
hipError_t fwd32_launch(const FwdArgs& a);
template <int Dp>
hipError_t grad_launch(const GradArgs& a);

}  // namespace hd
}  // namespace keops
