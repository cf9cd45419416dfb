// Device-side building blocks shared by the gfx950 kernels: element types,
// 16-byte vector loads/stores, the 8-element MFMA step and wavefront reductions.
//
// Compute types: fp32 (everything fp32) and fp16 (activations and MFMA
// operands fp16, accumulation and all statistics fp32). bf16 appears only as a
// weight storage type that is converted once at set-up.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kmd {

typedef __bf16 bf16;
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int WAVE = 64;

template <typename T> struct Vec8;
template <> struct Vec8<f16> { typedef f16x8 type; };
template <> struct Vec8<float> { typedef f32x8 type; };

// 8 consecutive elements (16 B for fp16, 32 B for fp32) from a 16-byte aligned address.
__device__ __forceinline__ f16x8 load8(const f16 *p) { return *reinterpret_cast<const f16x8 *>(p); }
__device__ __forceinline__ f32x8 load8(const float *p) {
  f32x4 a = *reinterpret_cast<const f32x4 *>(p);
  f32x4 b = *reinterpret_cast<const f32x4 *>(p + 4);
  return f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}
__device__ __forceinline__ void store8(f16 *p, f16x8 v) { *reinterpret_cast<f16x8 *>(p) = v; }
__device__ __forceinline__ void store8(float *p, f32x8 v) {
  *reinterpret_cast<f32x4 *>(p) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4 *>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

__device__ __forceinline__ float to_f32(f16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ f16 from_f32<f16>(float x) { return (f16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

template <typename T> __device__ __forceinline__ typename Vec8<T>::type zero8() {
  typename Vec8<T>::type z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = from_f32<T>(0.f);
  return z;
}

// acc(16x16, fp32) += A(16x32) * B(32x16) for one wavefront.
// Lane l supplies row (l % 16) of A and column (l % 16) of B, at the 8 k-slots
// owned by lane group g = l / 16. Any assignment of the 32 k values to
// (group, slot) pairs is valid as long as A and B use the same one.
// Result: lane l holds acc rows 4g .. 4g+3 of column l % 16.
__device__ __forceinline__ f32x4 mfma8(f16x8 a, f16x8 b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// acc(32x32) += A(32x16) B(16x32): lane l supplies row (l % 32) of A and column
// (l % 32) of B at the 8 k-slots of group l / 32. Result: lane l holds column
// l % 32, rows 8q + 4 (l / 32) + r (q, r = 0..3) in acc[4q + r].
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 acc) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
}
// fp32 operands: eight 32x32x2 steps; step j sums slot j of the two groups.
__device__ __forceinline__ f32x16 mfma32(f32x8 a, f32x8 b, f32x16 acc) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], acc, 0, 0, 0);
  return acc;
}

// XOR swizzle of the eight 16-byte chunks of a 128-byte LDS row: gives 8
// distinct chunks for rows 0..7 and for each parity class of rows 0..15, so
// reads of one chunk from 8 or 16 consecutive rows hit disjoint banks.
__device__ __forceinline__ int swz8(int r) { return ((r >> 1) ^ ((r & 1) << 2)) & 7; }

// s_waitcnt immediate (gfx9 encoding): vmcnt <= vm, lgkmcnt <= lgkm, expcnt not waited.
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }
// fp32 operands: eight 16x16x4 steps; step j sums slot j of each of the 4 groups.
__device__ __forceinline__ f32x4 mfma8(f32x8 a, f32x8 b, f32x4 acc) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], acc, 0, 0, 0);
  return acc;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// Exact (erf) GELU, x * Phi(x), with erf from Abramowitz & Stegun, Handbook of
// Mathematical Functions, formula 7.1.26: for z >= 0,
//   erf(z) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2),
//   t = 1 / (1 + p z),  |error| <= 1.5e-7.
// With z = |x| / sqrt(2) and q = t (...) exp(-z^2) / 2, Phi(x) = 1 - q for
// x >= 0 and q for x < 0, so the negative tail has no cancellation. About 15
// VALU operations, a fifth of the library erff; the error is far below the
// fp16 rounding of the stored activation.
__device__ __forceinline__ float gelu_erf(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.3275911f * z);
  const float poly = t * (0.254829592f + t * (-0.284496736f + t * (1.421413741f + t * (-1.453152027f + t * 1.061405429f))));
  const float q = 0.5f * poly * __builtin_amdgcn_exp2f(-z * z * 1.44269504088896341f);
  return x * (x >= 0.f ? 1.0f - q : q);
}
__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

}  // namespace kmd
