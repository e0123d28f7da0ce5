// Shared pieces of the low-dimensional (D <= 8) float32 reductions. Internal to the library.
//
// Every low-D kernel streams the column set j through wave-uniform loads (the column record
// of j is the same for all 64 lanes, so it lands in scalar registers) while each lane keeps R
// rows i in vector registers for the whole sweep; the M-by-N table never exists. Columns are
// split into ranges reduced independently and combined in a fixed order afterwards.
#pragma once

#include "internal.h"

#include <math.h>

namespace keops {
namespace lowd {

__device__ __forceinline__ float exp2_hw(float v) { return __builtin_amdgcn_exp2f(v); }

constexpr int kChunk = 512;            // columns per first-level partial sum
constexpr float kLseSlack = 16.0f;     // lazy rescale: terms may grow to 2^16 before a rescale

// Rows per lane of each family (register budgets measured on gfx950).
constexpr int kRowsSum = 4;
constexpr int kRowsSumSmall = 1;       // small M: more, smaller row blocks to fill the chip
constexpr int kRowsLse = 4;
constexpr int kRowsGrad = 2;
constexpr int kLseTile = 8;            // columns per log-sum-exp tile
// Largest column range of one split. A split's matrix-core column pieces (84 bytes a column)
// then take at most 2.75 MB of an XCD's 4 MB L2 while that XCD's resident workgroups stream
// them; at 65536 columns (5.5 MB) they did not fit, and the 1M x 1M sum fetched 9.0 GB from
// HBM per launch instead of 3.3 GB, in the same time.
constexpr int64_t kSplitCols = 32768;
// Fewest workgroups per CU a sweep launch aims for, by operation (0 sum, 1 log-sum-exp,
// 2 / 6 argKmin, 3 gradient) and channel count. The sweeps run in rounds of one workgroup per
// resident slot; with only a round or two the launch ends with the slowest CU, so more and
// shorter workgroups let the dispatcher even the load out, at the price of more partial
// results (splits x M x C floats) and of each split's own start-up. Measured at 100k x 100k
// and N = 2^17: the sum gains 6-8 % from 8 to 32, the gradient 4 % at 16; the log-sum-exp on
// 32 x 32 tiles (D <= 3, no running shift) 8 % at 16 (1.05 -> 0.97 ms), while the one with a
// running shift (whose splits each re-establish it) and argKmin (K-entry partial lists) are
// fastest at 8. Wide outputs keep 8 so the partials stay small.
constexpr int64_t wg_per_cu(int op, int C, int D) {
  return C > 4 ? 8 : (op == 0 ? 32 : (op == 3 || (op == 1 && D <= 3) ? 16 : 8));
}

inline int argk_bucket(int K) {
  if (K <= 1) return 1;
  if (K <= 2) return 2;
  if (K <= 4) return 4;
  if (K <= 8) return 8;
  if (K <= 10) return 10;
  if (K <= 16) return 16;
  if (K <= 32) return 32;
  return 64;
}
inline int argk_rows(int Kb) { return Kb <= 16 ? 2 : 1; }

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The device-side decision of a prepared matrix-core sweep, mf = {gate, bad}: 1 when it admits
// the matrix-core form (gate set, every piece exact), else 0. Both words are read and combined
// as integers (a short-circuit form of this test, used to select a value rather than to
// branch, was compiled into code that ignored its outcome).
__device__ __forceinline__ int mf_admits(const int* mf) {
  const int gate = mf[0], bad = mf[1];
  return (gate != 0 ? 1 : 0) & (bad == 0 ? 1 : 0);
}

// Per-row partial of a log-sum-exp over one split: l = sum_j 2^{e_ij - m} with the float64
// shift m in log2 units.
struct LsePartial {
  double m;
  float l;
  float pad;
};

// A (key, column) entry of an argKmin list.
struct KeyIdx {
  double key;
  int32_t idx;
  int32_t pad;
};

// out[i] = rscale[i / C] * sum over s of partial[s][i] (rscale may be null), in increasing s.
hipError_t launch_combine_sum(const float* partial, float* out, int64_t n, int64_t S, const float* rscale, int C,
                              hipStream_t s);
// out[i] = ln(sum over s of l_s 2^{m_s}), merged in float64.
// (mf: a device-side matrix-core decision; the combine then runs only when admitted == run_if_mf)
hipError_t launch_combine_lse(const LsePartial* partial, float* out, int64_t M, int64_t S, hipStream_t s,
                              const int* mf = nullptr, int run_if_mf = 0);

#define KEOPS_SWITCH_D(D_, CALL)                   \
  switch (D_) {                                    \
    case 1: return CALL(1);                        \
    case 2: return CALL(2);                        \
    case 3: return CALL(3);                        \
    case 4: return CALL(4);                        \
    case 5: return CALL(5);                        \
    case 6: return CALL(6);                        \
    case 7: return CALL(7);                        \
    case 8: return CALL(8);                        \
  }                                                \
  return hipErrorInvalidValue;

#define KEOPS_SWITCH_C(C_, CALL)                   \
  switch (C_) {                                    \
    case 1: return CALL(1);                        \
    case 2: return CALL(2);                        \
    case 3: return CALL(3);                        \
    case 4: return CALL(4);                        \
    case 5: return CALL(5);                        \
    case 6: return CALL(6);                        \
    case 7: return CALL(7);                        \
    case 8: return CALL(8);                        \
  }                                                \
  return hipErrorInvalidValue;

}  // namespace lowd
}  // namespace keops
