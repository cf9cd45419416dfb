// Fused residual add + post-norm LayerNorm (Kimodo WebGPU README, "WGSL compute shaders"
// table, layernorm_vit.wgsl and elementwise.wgsl rows; "Model details" table:
// post-norm): out = (v - mean(v)) / sqrt(var(v) + 1e-5) * gamma + beta with
// v = x + y, biased variance, statistics in fp32.
//
// One wavefront per 1024-wide row: each lane keeps 16 values in registers
// (two 16-byte loads per operand for fp16), so a row is read once and written
// once. All loads, gamma and beta included, are issued before any arithmetic.
// Statistics in one pass: each lane takes the mean and centred sum of squares
// of its 16 values, and a butterfly merges them pairwise with the update of
// Chan, Golub & LeVeque (1979) for equal counts n: mean = (m_a + m_b) / 2,
// M2 = M2_a + M2_b + (m_b - m_a)^2 n / 2 (both partners compute the same
// value, so every lane ends with the row's statistics). The kernel is
// HBM/L2-bound: 3 x 1024 x sizeof(T) bytes per row.
#include "common.h"
#include "kernels.h"

namespace kmd {
namespace {

constexpr int D = 1024;

template <typename T>
__global__ __launch_bounds__(256) void add_ln_kernel(const T *__restrict__ x, const T *__restrict__ y,
                                                     const float *__restrict__ gamma, const float *__restrict__ beta,
                                                     T *__restrict__ out, int M) {
  typedef typename Vec8<T>::type V8;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const size_t base = (size_t)row * D;
  V8 a[2], b[2];
  f32x8 gm[2], bt[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int c = hf * (D / 2) + 8 * lane;
    a[hf] = load8(x + base + c);
    b[hf] = load8(y + base + c);
  }
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int c = hf * (D / 2) + 8 * lane;
    gm[hf] = load8(gamma + c);
    bt[hf] = load8(beta + c);
  }
  float v[16];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int e = 0; e < 8; ++e) v[8 * hf + e] = to_f32(a[hf][e]) + to_f32(b[hf][e]);
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) m += v[e];
  m *= 1.0f / 16;
  float q = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float dlt = v[e] - m;
    q += dlt * dlt;
  }
  float n = 16.f;
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) {
    const float mb = __shfl_xor(m, o, WAVE), qb = __shfl_xor(q, o, WAVE);
    const float dlt = mb - m;
    q = q + qb + dlt * dlt * (0.5f * n);
    m = 0.5f * (m + mb);
    n *= 2.f;
  }
  const float rstd = 1.0f / sqrtf(q * (1.0f / D) + 1e-5f);
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int c = hf * (D / 2) + 8 * lane;
    V8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = from_f32<T>((v[8 * hf + e] - m) * rstd * gm[hf][e] + bt[hf][e]);
    store8(out + base + c, r);
  }
}

// The same row normalisation with the residual branch given as split-K
// partial sums of its projection: y = sum_s P[s][row] + bias in fp32 (the
// splits added in index order), v = x + y. Replaces the split-K reduction
// kernel and the add + LayerNorm kernel.
template <typename T>
__global__ __launch_bounds__(256) void add_ln_splitk_kernel(const T *__restrict__ x, const float *__restrict__ P,
                                                            int splits, const float *__restrict__ bias,
                                                            const float *__restrict__ gamma,
                                                            const float *__restrict__ beta, T *__restrict__ out,
                                                            int M) {
  typedef typename Vec8<T>::type V8;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= M) return;
  const size_t base = (size_t)row * D;
  float v[16];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int c = hf * (D / 2) + 8 * lane;
    const V8 a = load8(x + base + c);
    const f32x8 b = load8(bias + c);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[8 * hf + e] = b[e];
    // up to 8 splits' loads in flight at once; the sums stay in split order
    const float *pp = P + base + c;
    const size_t stride = (size_t)M * D;
    for (int s0 = 0; s0 < splits; s0 += 8) {
      f32x8 pv[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (s0 + k < splits) pv[k] = load8(pp + (size_t)(s0 + k) * stride);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (s0 + k < splits)
#pragma unroll
          for (int e = 0; e < 8; ++e) v[8 * hf + e] += pv[k][e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[8 * hf + e] += to_f32(a[e]);
  }
  f32x8 gm[2], bt[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int c = hf * (D / 2) + 8 * lane;
    gm[hf] = load8(gamma + c);
    bt[hf] = load8(beta + c);
  }
  float m = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) m += v[e];
  m *= 1.0f / 16;
  float q = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float dlt = v[e] - m;
    q += dlt * dlt;
  }
  float n = 16.f;
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) {
    const float mb = __shfl_xor(m, o, WAVE), qb = __shfl_xor(q, o, WAVE);
    const float dlt = mb - m;
    q = q + qb + dlt * dlt * (0.5f * n);
    m = 0.5f * (m + mb);
    n *= 2.f;
  }
  const float rstd = 1.0f / sqrtf(q * (1.0f / D) + 1e-5f);
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int c = hf * (D / 2) + 8 * lane;
    V8 r;
#pragma unroll
    for (int e = 0; e < 8; ++e) r[e] = from_f32<T>((v[8 * hf + e] - m) * rstd * gm[hf][e] + bt[hf][e]);
    store8(out + base + c, r);
  }
}

}  // namespace

template <typename T>
hipError_t add_layernorm_splitk(const T *x, const float *P, int splits, const float *bias, const float *gamma,
                                const float *beta, T *out, int M, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  launch("add_layernorm_splitk", add_ln_splitk_kernel<T>, dim3((M + 3) / 4), dim3(256), stream, x, P, splits, bias,
         gamma, beta, out, M);
  return hipGetLastError();
}

template hipError_t add_layernorm_splitk<f16>(const f16 *, const float *, int, const float *, const float *,
                                              const float *, f16 *, int, hipStream_t);
template hipError_t add_layernorm_splitk<float>(const float *, const float *, int, const float *, const float *,
                                                const float *, float *, int, hipStream_t);

template <typename T>
hipError_t add_layernorm(const T *x, const T *y, const float *gamma, const float *beta, T *out, int M,
                         hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  launch("add_layernorm", add_ln_kernel<T>, dim3((M + 3) / 4), dim3(256), stream, x, y, gamma, beta, out, M);
  return hipGetLastError();
}

template hipError_t add_layernorm<f16>(const f16 *, const f16 *, const float *, const float *, f16 *, int,
                                       hipStream_t);
template hipError_t add_layernorm<float>(const float *, const float *, const float *, const float *, float *, int,
                                         hipStream_t);

}  // namespace kmd
