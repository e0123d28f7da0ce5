// Issue rates on gfx950 of the instructions the library's sweeps are built from, and of the
// per-unit mix of the matrix-core Gauss sum. Measurement aid behind the kernel-design figures;
// not part of the library.
//
//   hipcc --offload-arch=gfx950 -O3 -Xclang -target-feature -Xclang -packed-fp32-ops \
//         -mllvm -amdgpu-mfma-vgpr-form microbench/issue_rates.hip -o issue_rates && ./issue_rates
//
// Every kernel runs ITERS iterations of a fixed block of independent instructions in registers
// (eight independent chains, so a single wave is not latency-bound on one chain), on
// (CUs x waves per SIMD) workgroups of 4 waves, i.e. the given number of waves on every SIMD.
// The printed figure is nanoseconds per iteration per wave: with W waves per SIMD the SIMD
// runs W iterations in W times that long, so the figure is the SIMD's issue time for one
// iteration's block. The only memory access is one float per thread written at the end (out
// holds grid x block floats), which keeps the results live.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <utility>

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kIters = 4096;

#define EACH8(X) X(0) X(1) X(2) X(3) X(4) X(5) X(6) X(7)

enum Kind {
  kExpF32, kExpF16, kFmaF32, kAddF32, kFmaF64, kCvtPkF16, kCvtPkBf16, kPkFmaF16, kMfma16, kMfma32x2,
  kExp8Fma8, kExp8Fma8Cvt4, kMfma4Fma8, kMfma4Exp8, kMfma4Exp8Cvt4, kMfma4Exp8Fma8Cvt4, kMfma32x2Exp8Fma8Cvt4,
  kKinds
};
static const char* kNames[kKinds] = {
    "8 v_exp_f32", "8 v_exp_f16", "8 v_fma_f32", "8 v_add_f32", "8 v_fma_f64", "8 v_cvt_pk_f16_f32",
    "8 v_cvt_pk_bf16_f32", "8 v_pk_fma_f16", "4 mfma 16x16x32 f16", "2 mfma 32x32x16 f16",
    "8 exp + 8 fma", "8 exp + 8 fma + 4 cvt", "4 mfma16 + 8 fma", "4 mfma16 + 8 exp", "4 mfma16 + 8 exp + 4 cvt",
    "4 mfma16 + 8 exp + 8 fma + 4 cvt", "2 mfma32 + 8 exp + 8 fma + 4 cvt"};

#define EXP_F32(i) asm volatile("v_exp_f32 %0, %0" : "+v"(a[i]));
#define FMA_F32(i) asm volatile("v_fma_f32 %0, %0, %0, 1.0" : "+v"(a[i]));
#define CVT4 CVT(0) CVT(1) CVT(2) CVT(3)
#define CVT(i) asm volatile("v_cvt_pk_f16_f32 %0, %1, %1" : "=v"(h[i]) : "v"(a[i]));

template <int K>
__global__ void __launch_bounds__(256) rates_kernel(float* out, float seed) {
  float a[8];
  unsigned int h[8];
  double dd[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = seed * (float)(threadIdx.x + i) * 1e-3f;
    h[i] = 0x3c003c00u + i;
    dd[i] = (double)a[i];
  }
  const _Float16 hs = (_Float16)seed;
  const half8 ha = {hs, hs, hs, hs, hs, hs, hs, hs};
  f32x4 acc[4] = {};
  f32x16 big[2] = {};
  for (int it = 0; it < kIters; ++it) {
    if constexpr (K == kExpF32) {
      EACH8(EXP_F32)
    } else if constexpr (K == kExpF16) {
#define X(i) asm volatile("v_exp_f16 %0, %0" : "+v"(h[i]));
      EACH8(X)
#undef X
    } else if constexpr (K == kFmaF32) {
      EACH8(FMA_F32)
    } else if constexpr (K == kAddF32) {
#define X(i) asm volatile("v_add_f32 %0, %0, 1.0" : "+v"(a[i]));
      EACH8(X)
#undef X
    } else if constexpr (K == kFmaF64) {
#define X(i) asm volatile("v_fma_f64 %0, %0, %0, 1.0" : "+v"(dd[i]));
      EACH8(X)
#undef X
    } else if constexpr (K == kCvtPkF16) {
      EACH8(CVT)
    } else if constexpr (K == kCvtPkBf16) {
#define X(i) asm volatile("v_cvt_pk_bf16_f32 %0, %1, %1" : "=v"(h[i]) : "v"(a[i]));
      EACH8(X)
#undef X
    } else if constexpr (K == kPkFmaF16) {
#define X(i) asm volatile("v_pk_fma_f16 %0, %0, %0, %0" : "+v"(h[i]));
      EACH8(X)
#undef X
    } else if constexpr (K == kMfma16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ha, ha, acc[i], 0, 0, 0);
    } else if constexpr (K == kMfma32x2) {
#pragma unroll
      for (int i = 0; i < 2; ++i) big[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha, ha, big[i], 0, 0, 0);
    } else if constexpr (K == kExp8Fma8) {
      EACH8(FMA_F32) EACH8(EXP_F32)
    } else if constexpr (K == kExp8Fma8Cvt4) {
      EACH8(FMA_F32) EACH8(EXP_F32) CVT4
    } else if constexpr (K == kMfma4Fma8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ha, ha, acc[i], 0, 0, 0);
      EACH8(FMA_F32)
    } else if constexpr (K == kMfma4Exp8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ha, ha, acc[i], 0, 0, 0);
      EACH8(EXP_F32)
    } else if constexpr (K == kMfma4Exp8Cvt4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ha, ha, acc[i], 0, 0, 0);
      EACH8(EXP_F32) CVT4
    } else if constexpr (K == kMfma4Exp8Fma8Cvt4) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ha, ha, acc[i], 0, 0, 0);
      EACH8(FMA_F32) EACH8(EXP_F32) CVT4
    } else if constexpr (K == kMfma32x2Exp8Fma8Cvt4) {
#pragma unroll
      for (int i = 0; i < 2; ++i) big[i] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ha, ha, big[i], 0, 0, 0);
      EACH8(FMA_F32) EACH8(EXP_F32) CVT4
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += a[i] + (float)__builtin_bit_cast(half2v, h[i])[0] + (float)dd[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) s += acc[i][0];
  s += big[0][0] + big[1][0];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// The fp16 forward's unit structure without memory: per iteration a 32-key subtile against
// 8 query tiles; for each tile the scores of the next one are issued (2 MFMAs), then
// P = fp16(2^(cs S + alpha)) of the current one (with kFma; 2^S without), then O += V P
// (2 MFMAs). One iteration is 8 units of 512 pairs.
template <bool kFma>
__global__ void __launch_bounds__(256) unit_kernel(float* out, float seed) {
  half8 k0, k1, v0, v1, q[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    k0[s] = (_Float16)(seed * 0.01f * s);
    k1[s] = (_Float16)(seed * 0.02f * s);
    v0[s] = (_Float16)(seed * 0.03f);
    v1[s] = (_Float16)(seed * 0.04f);
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) q[t] = k0 * (_Float16)(0.1f * t);
  f32x4 b0 = {-1.f, -2.f, -3.f, -4.f}, b1 = b0;
  float alpha[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) alpha[t] = -0.5f - 0.01f * t;
  f32x4 O[8][2] = {};
  const float cs = 1.4427f;
  for (int it = 0; it < kIters / 8; ++it) {
    asm volatile("" : "+v"(k0), "+v"(k1), "+v"(v0), "+v"(v1), "+v"(b0), "+v"(b1));
    f32x4 S[2][2];
    S[0][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, q[0], b0, 0, 0, 0);
    S[0][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, q[0], b1, 0, 0, 0);
#pragma unroll
    for (int qt = 0; qt < 8; ++qt) {
      if (qt + 1 < 8) {
        S[(qt + 1) & 1][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k0, q[qt + 1], b0, 0, 0, 0);
        S[(qt + 1) & 1][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k1, q[qt + 1], b1, 0, 0, 0);
      }
      half8 p;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        float e = S[qt & 1][s >> 2][s & 3];
        if constexpr (kFma) e = fmaf(e, cs, alpha[qt]);
        p[s] = (_Float16)__builtin_amdgcn_exp2f(e);
      }
      O[qt][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v0, p, O[qt][0], 0, 0, 0);
      O[qt][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(v1, p, O[qt][1], 0, 0, 0);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int t = 0; t < 8; ++t) s += O[t][0][0] + O[t][1][1];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// The fp16 forward's unit structure on 32x32x16 MFMAs: per iteration a 32-key subtile against
// 4 query tiles of 32; for each tile the scores of the next one are issued (2 MFMAs, K = 16 each
// for 32 features), then P = fp16(2^(cs S + alpha)) of the current one (16 values per lane),
// then O += V P (2 MFMAs for 32 channels, K = 16 keys each). One iteration is 8 units of 512
// pairs, as in unit_kernel. kMode 0: as described. kMode 1: the scale is in the query operand
// and one shift serves the wave, so the accumulator starts from beta + u (16 adds per subtile,
// shared by the 4 tiles) and P = fp16(2^S) needs no FMA. kMode 2: as 1 with the scaled query
// in two fp16 parts (hi + lo), i.e. 4 MFMAs for the scores.
template <int kMode>
__global__ void __launch_bounds__(256) unit32_kernel(float* out, float seed) {
  half8 k0, k1, v0, v1, q0[4], q1[4];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    k0[s] = (_Float16)(seed * 0.01f * s);
    k1[s] = (_Float16)(seed * 0.02f * s);
    v0[s] = (_Float16)(seed * 0.03f);
    v1[s] = (_Float16)(seed * 0.04f);
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    q0[t] = k0 * (_Float16)(0.1f * t);
    q1[t] = k1 * (_Float16)(0.1f * t);
  }
  f32x16 beta;
#pragma unroll
  for (int i = 0; i < 16; ++i) beta[i] = -1.0f - 0.1f * i;
  float alpha[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) alpha[t] = -0.5f - 0.01f * t;
  f32x16 O[4] = {};
  const float cs = 1.4427f;
  float u = -0.75f;
  for (int it = 0; it < kIters / 8; ++it) {
    asm volatile("" : "+v"(k0), "+v"(k1), "+v"(v0), "+v"(v1), "+v"(beta), "+s"(u));
    f32x16 bu = beta;
    if constexpr (kMode > 0) {
#pragma unroll
      for (int s = 0; s < 16; ++s) bu[s] = beta[s] + u;
    }
    auto score = [&](int qt) {
      f32x16 S = __builtin_amdgcn_mfma_f32_32x32x16_f16(k0, q0[qt], bu, 0, 0, 0);
      S = __builtin_amdgcn_mfma_f32_32x32x16_f16(k1, q1[qt], S, 0, 0, 0);
      if constexpr (kMode == 2) {
        S = __builtin_amdgcn_mfma_f32_32x32x16_f16(k0, q1[qt], S, 0, 0, 0);
        S = __builtin_amdgcn_mfma_f32_32x32x16_f16(k1, q0[qt], S, 0, 0, 0);
      }
      return S;
    };
    f32x16 S[2];
    S[0] = score(0);
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      if (qt + 1 < 4) S[(qt + 1) & 1] = score(qt + 1);
      half8 pa, pb;
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        float e = S[qt & 1][s];
        if constexpr (kMode == 0) e = fmaf(e, cs, alpha[qt]);
        const _Float16 h = (_Float16)__builtin_amdgcn_exp2f(e);
        if (s < 8) pa[s] = h;
        else pb[s - 8] = h;
      }
      O[qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(v0, pa, O[qt], 0, 0, 0);
      O[qt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(v1, pb, O[qt], 0, 0, 0);
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int t = 0; t < 4; ++t) s += O[t][0] + O[t][5];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// The float32 Gauss sum's tile structure without memory, per 1024 pairs: a high-part MFMA whose
// result feeds the low-part MFMA as its accumulator, then per output one exp2 and one FMA into
// a per-row partial sum. kWide = false: 16x16x32 MFMAs, 4 row tiles of 16 (8 MFMAs per 1024
// pairs); kWide = true: 32x32x16 MFMAs, 2 row tiles of 32 (2 MFMAs per 1024 pairs). One
// iteration is 1024 pairs (16x16) or 2048 pairs (32x32).
template <bool kWide>
__global__ void __launch_bounds__(256) sum_tile_kernel(float* out, float seed) {
  const _Float16 hs = (_Float16)(seed * 0.001f);
  half8 hi = {hs, hs, hs, hs, hs, hs, hs, hs}, lo = hi;
  float w = seed;
  constexpr int RT = kWide ? 2 : 4, Q = kWide ? 16 : 4;
  half8 ahi[RT], alo[RT];
  f32x4 cinit[RT];
  float part[RT][Q];
#pragma unroll
  for (int r = 0; r < RT; ++r) {
    ahi[r] = hi * (_Float16)(0.5f + 0.1f * r);
    alo[r] = lo * (_Float16)(0.25f + 0.1f * r);
    cinit[r] = f32x4{-1.f, -2.f, -3.f, -4.f};
#pragma unroll
    for (int q = 0; q < Q; ++q) part[r][q] = 0.0f;
  }
  for (int it = 0; it < kIters / 8; ++it) {
    asm volatile("" : "+v"(hi), "+v"(lo), "+v"(w));
#pragma unroll
    for (int r = 0; r < RT; ++r) {
      if constexpr (kWide) {
        f32x16 e = __builtin_amdgcn_mfma_f32_32x32x16_f16(ahi[r], hi, f32x16{}, 0, 0, 0);
        e = __builtin_amdgcn_mfma_f32_32x32x16_f16(alo[r], lo, e, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < Q; ++q) part[r][q] = fmaf(__builtin_amdgcn_exp2f(e[q]), w, part[r][q]);
      } else {
        f32x4 e = __builtin_amdgcn_mfma_f32_16x16x32_f16(ahi[r], hi, cinit[r], 0, 0, 0);
        e = __builtin_amdgcn_mfma_f32_16x16x32_f16(alo[r], lo, e, 0, 0, 0);
#pragma unroll
        for (int q = 0; q < Q; ++q) part[r][q] = fmaf(__builtin_amdgcn_exp2f(e[q]), w, part[r][q]);
      }
    }
  }
  float s = 0.0f;
#pragma unroll
  for (int r = 0; r < RT; ++r)
#pragma unroll
    for (int q = 0; q < Q; ++q) s += part[r][q];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

static void check(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    std::fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    std::exit(1);
  }
}

template <typename Launch>
static double time_ms(Launch launch, int reps) {
  hipEvent_t e0, e1;
  check(hipEventCreate(&e0), "hipEventCreate");
  check(hipEventCreate(&e1), "hipEventCreate");
  launch();
  check(hipDeviceSynchronize(), "warm-up");
  check(hipEventRecord(e0), "hipEventRecord");
  for (int r = 0; r < reps; ++r) launch();
  check(hipEventRecord(e1), "hipEventRecord");
  check(hipEventSynchronize(e1), "hipEventSynchronize");
  float ms = 0.0f;
  check(hipEventElapsedTime(&ms, e0, e1), "hipEventElapsedTime");
  check(hipEventDestroy(e0), "hipEventDestroy");
  check(hipEventDestroy(e1), "hipEventDestroy");
  return ms / reps;
}

template <int K>
static double run_kind(float* out, int blocks) {
  return time_ms([&] { rates_kernel<K><<<blocks, 256>>>(out, 1.0f); }, 5);
}

template <int... Ks>
static void run_all(float* out, int blocks, double* t, std::integer_sequence<int, Ks...>) {
  ((t[Ks] = run_kind<Ks>(out, blocks)), ...);
}

int main() {
  int cus = 0;
  check(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0), "hipDeviceGetAttribute");
  std::printf("%-40s %12s %12s %12s\n", "ns per iteration per wave", "1 wave/SIMD", "2 waves/SIMD", "4 waves/SIMD");
  double t[3][kKinds + 7];
  for (int w = 0; w < 3; ++w) {
    const int wps = 1 << w;
    const int blocks = cus * wps;  // 4 waves per workgroup: wps waves on every SIMD
    float* out = nullptr;
    check(hipMalloc(&out, sizeof(float) * blocks * 256), "hipMalloc");
    run_all(out, blocks, t[w], std::make_integer_sequence<int, kKinds>{});
    t[w][kKinds] = time_ms([&] { unit_kernel<true><<<blocks, 256>>>(out, 1.0f); }, 5);
    t[w][kKinds + 1] = time_ms([&] { unit_kernel<false><<<blocks, 256>>>(out, 1.0f); }, 5);
    t[w][kKinds + 2] = time_ms([&] { sum_tile_kernel<false><<<blocks, 256>>>(out, 1.0f); }, 5);
    t[w][kKinds + 3] = time_ms([&] { sum_tile_kernel<true><<<blocks, 256>>>(out, 1.0f); }, 5) / 2.0;
    t[w][kKinds + 4] = time_ms([&] { unit32_kernel<0><<<blocks, 256>>>(out, 1.0f); }, 5);
    t[w][kKinds + 5] = time_ms([&] { unit32_kernel<1><<<blocks, 256>>>(out, 1.0f); }, 5);
    t[w][kKinds + 6] = time_ms([&] { unit32_kernel<2><<<blocks, 256>>>(out, 1.0f); }, 5);
    check(hipGetLastError(), "launch");
    check(hipFree(out), "hipFree");
    for (int k = 0; k < kKinds + 7; ++k) t[w][k] = t[w][k] * 1e6 / kIters / wps;
  }
  for (int k = 0; k < kKinds; ++k)
    std::printf("%-40s %12.2f %12.2f %12.2f\n", kNames[k], t[0][k], t[1][k], t[2][k]);
  std::printf("%-40s %12.2f %12.2f %12.2f   (per 512-pair unit)\n", "fp16 forward unit, cs S + alpha", t[0][kKinds],
              t[1][kKinds], t[2][kKinds]);
  std::printf("%-40s %12.2f %12.2f %12.2f   (per 512-pair unit)\n", "fp16 forward unit, no FMA", t[0][kKinds + 1],
              t[1][kKinds + 1], t[2][kKinds + 1]);
  std::printf("%-40s %12.2f %12.2f %12.2f   (per 512-pair unit)\n", "fp16 forward unit on 32x32x16 tiles",
              t[0][kKinds + 4], t[1][kKinds + 4], t[2][kKinds + 4]);
  std::printf("%-40s %12.2f %12.2f %12.2f   (per 512-pair unit)\n", "fp16 unit, 32x32, wave shift, no FMA",
              t[0][kKinds + 5], t[1][kKinds + 5], t[2][kKinds + 5]);
  std::printf("%-40s %12.2f %12.2f %12.2f   (per 512-pair unit)\n", "fp16 unit, 32x32, wave shift, hi+lo q",
              t[0][kKinds + 6], t[1][kKinds + 6], t[2][kKinds + 6]);
  std::printf("%-40s %12.2f %12.2f %12.2f   (per 1024 pairs)\n", "Gauss-sum tile, 16x16x32, 4 row tiles",
              t[0][kKinds + 2] * 8, t[1][kKinds + 2] * 8, t[2][kKinds + 2] * 8);
  std::printf("%-40s %12.2f %12.2f %12.2f   (per 1024 pairs)\n", "Gauss-sum tile, 32x32x16, 2 row tiles",
              t[0][kKinds + 3] * 8, t[1][kKinds + 3] * 8, t[2][kKinds + 3] * 8);
  return 0;
}
