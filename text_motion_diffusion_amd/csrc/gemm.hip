// Dense projection GEMMs of the denoiser (QKV, attention output, FFN, input and
// output heads, text and timestep MLPs): C = epi(A W^T + b) with W in the torch
// Linear layout [out, in] (Kimodo WebGPU README, shader table, "Matrix multiply
// + bias"; the GELU and SiLU shaders are folded into the epilogue).
//
// gfx950 design: one 256-thread workgroup computes a 128x128 tile of C; each of
// its 4 wavefronts owns a 64x64 sub-tile as 4x4 blocks of 16x16 MFMA
// accumulators (fp32). Each k-tile is 128 bytes of K per row (64 fp16 or 32
// fp32), staged through LDS in two buffers so the global loads of tile k+1 are
// in flight while tile k is multiplied. Rows of the LDS tiles are padded by 16
// bytes, so the 16-byte fragment reads of 8 consecutive rows fall on disjoint
// banks. The MFMA is issued as D = W_tile * A_tile^T, which leaves every lane
// with 4 consecutive output columns of one row: the epilogue stores 8 bytes
// (fp16) or 16 bytes (fp32) per lane.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace kmd {
namespace {

enum { EPI_BIAS = 0, EPI_BIAS_GELU = 1, EPI_BIAS_SILU = 2 };
constexpr int BM = 128, BN = 128;
constexpr int ROW_BYTES = 128;
constexpr int PITCH = ROW_BYTES + 16;
constexpr int STAGE = (BM + BN) * PITCH;

template <typename T, int EPI, typename TO>
__device__ __forceinline__ void gemm_tile(const T *__restrict__ A, int lda, const T *__restrict__ W, int ldw,
                                          const float *__restrict__ bias, TO *__restrict__ C, int ldc, int M, int N,
                                          int K, int vec_store) {
  typedef typename Vec8<T>::type V8;
  constexpr int BK = ROW_BYTES / (int)sizeof(T);
  constexpr int CH = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  constexpr int FRAG = 8 * (int)sizeof(T);  // bytes of one 8-element fragment
  constexpr int KSTEPS = ROW_BYTES / (4 * FRAG);
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;

  // Global -> register staging: 256 rows (A then W) x 8 chunks = 2048 chunks,
  // 8 per thread; chunk j of thread t is row 32 j + t / 8, chunk t % 8.
  uint4 stage[8];
  const int ld_row = tid >> 3, ld_ch = tid & 7;
  auto gload = [&](int kt) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int m = m0 + 32 * j + ld_row;
      stage[j] = m < M ? *reinterpret_cast<const uint4 *>(A + (size_t)m * lda + kt * BK + ld_ch * CH)
                       : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int n = n0 + 32 * j + ld_row;
      stage[4 + j] = n < N ? *reinterpret_cast<const uint4 *>(W + (size_t)n * ldw + kt * BK + ld_ch * CH)
                           : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
    char *base = smem + buf * STAGE;
#pragma unroll
    for (int j = 0; j < 8; ++j) *reinterpret_cast<uint4 *>(base + (32 * j + ld_row) * PITCH + ld_ch * 16) = stage[j];
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) {
    const char *a_base = smem + buf * STAGE + (wm * 64 + l16) * PITCH;
    const char *w_base = smem + buf * STAGE + (BM + wn * 64 + l16) * PITCH;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const int kb = ks * 4 * FRAG + g * FRAG;
      V8 af[4], wf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = load8(reinterpret_cast<const T *>(a_base + i * 16 * PITCH + kb));
#pragma unroll
      for (int j = 0; j < 4; ++j) wf[j] = load8(reinterpret_cast<const T *>(w_base + j * 16 * PITCH + kb));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma8(wf[j], af[i], acc[i][j]);
    }
  };

  const int nk = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload(kt + 1);
    compute(kt & 1);
    if (kt + 1 < nk) sstore((kt + 1) & 1);
    __syncthreads();
  }

  // Epilogue: acc[i][j][r] = C[m0 + wm*64 + 16i + l16][n0 + wn*64 + 16j + 4g + r].
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + wm * 64 + 16 * i + l16;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + wn * 64 + 16 * j + 4 * g;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = acc[i][j][r];
        if (n + r < N) x += bias[n + r];
        if (EPI == EPI_BIAS_GELU) x = gelu_erf(x);
        if (EPI == EPI_BIAS_SILU) x = silu(x);
        v[r] = x;
      }
      TO *dst = C + (size_t)m * ldc + n;
      if (vec_store && n + 3 < N) {
        if constexpr (sizeof(TO) == 4) {
          *reinterpret_cast<f32x4 *>(dst) = f32x4{v[0], v[1], v[2], v[3]};
        } else {
          *reinterpret_cast<f16x4 *>(dst) = f16x4{from_f32<TO>(v[0]), from_f32<TO>(v[1]), from_f32<TO>(v[2]),
                                                  from_f32<TO>(v[3])};
        }
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (n + r < N) dst[r] = from_f32<TO>(v[r]);
      }
    }
  }
}

#define KMD_GEMM_ROLE(NAME, EPI, OUT_F32)                                                                      \
  template <typename T>                                                                                        \
  __global__ __launch_bounds__(256, 2) void NAME(const T *__restrict__ A, int lda, const T *__restrict__ W,    \
                                                 int ldw, const float *__restrict__ bias, void *__restrict__ C, \
                                                 int ldc, int M, int N, int K, int vec_store) {                  \
    typedef typename std::conditional<OUT_F32, float, T>::type TO;                                            \
    gemm_tile<T, EPI, TO>(A, lda, W, ldw, bias, static_cast<TO *>(C), ldc, M, N, K, vec_store);               \
  }
KMD_GEMM_ROLE(gemm_qkv, EPI_BIAS, false)
KMD_GEMM_ROLE(gemm_out, EPI_BIAS, false)
KMD_GEMM_ROLE(gemm_ffn1_gelu, EPI_BIAS_GELU, false)
KMD_GEMM_ROLE(gemm_ffn2, EPI_BIAS, false)
KMD_GEMM_ROLE(gemm_in_proj, EPI_BIAS, true)
KMD_GEMM_ROLE(gemm_head, EPI_BIAS, true)
KMD_GEMM_ROLE(gemm_text, EPI_BIAS, false)
KMD_GEMM_ROLE(gemm_tmlp1_silu, EPI_BIAS_SILU, false)
KMD_GEMM_ROLE(gemm_tmlp2, EPI_BIAS, false)
#undef KMD_GEMM_ROLE

}  // namespace

template <typename T>
hipError_t gemm(GemmRole role, const T *A, int lda, const T *W, int ldw, const float *bias, void *C, int ldc, int M,
                int N, int K, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K % gemm_k_tile<T>() != 0 || lda % (16 / (int)sizeof(T)) || ldw % (16 / (int)sizeof(T)))
    return hipErrorInvalidValue;
  const bool out_f32 = role == ROLE_IN || role == ROLE_HEAD;
  const size_t osize = out_f32 ? 4 : sizeof(T);
  const int vec = (ldc % 4 == 0) && (reinterpret_cast<uintptr_t>(C) % (4 * osize) == 0);
  const dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM), block(256);
  switch (role) {
#define KMD_CASE(R, NAME) \
  case R: launch(#NAME, NAME<T>, grid, block, s, A, lda, W, ldw, bias, C, ldc, M, N, K, vec); break;
    KMD_CASE(ROLE_QKV, gemm_qkv)
    KMD_CASE(ROLE_OUT, gemm_out)
    KMD_CASE(ROLE_FFN1, gemm_ffn1_gelu)
    KMD_CASE(ROLE_FFN2, gemm_ffn2)
    KMD_CASE(ROLE_IN, gemm_in_proj)
    KMD_CASE(ROLE_HEAD, gemm_head)
    KMD_CASE(ROLE_TXT, gemm_text)
    KMD_CASE(ROLE_TMLP1, gemm_tmlp1_silu)
    KMD_CASE(ROLE_TMLP2, gemm_tmlp2)
#undef KMD_CASE
  }
  return hipGetLastError();
}

template hipError_t gemm<f16>(GemmRole, const f16 *, int, const f16 *, int, const float *, void *, int, int, int, int,
                              hipStream_t);
template hipError_t gemm<float>(GemmRole, const float *, int, const float *, int, const float *, void *, int, int, int,
                                int, hipStream_t);

}  // namespace kmd
