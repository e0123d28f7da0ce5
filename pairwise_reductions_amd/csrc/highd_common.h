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
// Where scoring every query tile of a subtile before using them needs more than 256 VGPRs
// (one wave per SIMD), the forward kernel scores and uses one tile at a time instead, which
// keeps two waves per SIMD; elsewhere the tile-batched order runs faster (more independent
// products in flight). Measured on the register counts of the compiled kernels.
constexpr bool fwd_fused(int D, int C, bool split) {
  return split ? (C == 64 && D >= 64) : ((D == 32 && C == 32) || (D == 64 && C == 64));
}
// The gradient kernel holds three products per subtile, so it takes fewer.
// (Sizes chosen so every instantiation fits 256 VGPRs, i.e. two waves per SIMD.)
constexpr int grad_query_tiles(int D, int CK, int CB) { return D <= 32 ? (CK <= 32 && CB == 0 ? 4 : 2) : 1; }
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
template <int Dp>
hipError_t grad_launch(const GradArgs& a);

}  // namespace hd
}  // namespace keops
