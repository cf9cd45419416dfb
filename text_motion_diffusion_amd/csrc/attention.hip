// Multi-head self-attention with key masking (Kimodo WebGPU README, shader
// table: "Multi-head self-attention with optional key masking"; the QKV
// deinterleave shader is not needed: Q, K and V are read in place from the
// fused projection rows [q | k | v], head j at columns 128j .. 128j+127 of each).
//
// Per (sequence p, head h, 64-query tile) one 256-thread workgroup; each of
// its 4 wavefronts owns 16 query rows, whose Q fragments stay in registers.
// Keys are processed in blocks of 64: the K block is staged in LDS row-major and
// the V block as Vt[d][key], copied from the transposed V that the QKV
// projection's epilogue writes (vt[p][head][d][key], keys contiguous), so both
// staging copies are 16-byte loads and stores and both MFMA operands of the
// P V product are contiguous 8- or 16-byte LDS reads. Scores are computed as
// S^T = K Q^T, which leaves each lane holding 16 scores of ONE query row, so the
// online-softmax max and the rescale of the output accumulators are per-lane
// plus two cross-lane steps (lanes l, l^16, l^32, l^48 share a row). Masked keys
// (position >= length + 2) are never read: they are zero-filled in LDS and get
// probability exactly 0 (score -inf). Softmax runs in fp32 with exp2 on
// log2(e)-prescaled scores; P is rounded to the operand type for the MFMA.
#include "common.h"
#include "kernels.h"

namespace kmd {
namespace {

constexpr int D_MODEL = 1024, D_HEAD = 128, QKV_LD = 3 * D_MODEL;
constexpr int QT = 64, KB = 64;

template <typename T>
__global__ __launch_bounds__(256) void attention_kernel(const T *__restrict__ qkv, const T *__restrict__ vt,
                                                        T *__restrict__ out, const int32_t *__restrict__ lengths,
                                                        int B, int S, int S_pad, float scale_log2) {
  typedef typename Vec8<T>::type V8;
  constexpr int ES = (int)sizeof(T);
  constexpr int K_PITCH = D_HEAD * ES + 16;  // bytes per key row of K
  constexpr int V_PITCH = KB * ES + 16;      // bytes per d row of Vt
  constexpr int CH = 16 / ES;                // elements per 16-byte chunk
  __shared__ __attribute__((aligned(16))) char k_lds[KB * K_PITCH];
  __shared__ __attribute__((aligned(16))) char v_lds[D_HEAD * V_PITCH];

  const int p = blockIdx.z, head = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g = lane >> 4;
  const int n_valid = min(lengths[p % B] + 2, S);
  const int q_tile0 = blockIdx.x * QT;
  const T *seq = qkv + (size_t)p * S * QKV_LD;
  const T *vhead = vt + ((size_t)p * (D_MODEL / D_HEAD) + head) * D_HEAD * S_pad;  // [d][S_pad]
  T *oseq = out + (size_t)p * S * D_MODEL + head * D_HEAD;

  if (q_tile0 >= n_valid) {
    // every query of this tile is a padded token: its output is never used by a
    // valid position; write zeros so the buffer stays finite.
    for (int idx = tid; idx < QT * D_HEAD / CH; idx += 256) {
      int r = q_tile0 + idx / (D_HEAD / CH), c = (idx % (D_HEAD / CH)) * CH;
      if (r < S) *reinterpret_cast<uint4 *>(oseq + (size_t)r * D_MODEL + c) = make_uint4(0, 0, 0, 0);
    }
    return;
  }

  const int q = q_tile0 + wave * 16 + l16;
  const bool q_ok = q < S;
  V8 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    qf[kk] = q_ok ? load8(seq + (size_t)q * QKV_LD + head * D_HEAD + 32 * kk + 8 * g) : zero8<T>();

  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (int j0 = 0; j0 < n_valid; j0 += KB) {
    __syncthreads();  // previous block's LDS reads are done
    // K block: KB key rows x (D_HEAD / CH) chunks; Vt block: D_HEAD rows x (KB / CH) chunks.
    for (int idx = tid; idx < KB * (D_HEAD / CH); idx += 256) {
      const int r = idx / (D_HEAD / CH), c = (idx % (D_HEAD / CH)) * CH;
      const int key = j0 + r;
      uint4 kv = make_uint4(0, 0, 0, 0);
      if (key < n_valid) kv = *reinterpret_cast<const uint4 *>(seq + (size_t)key * QKV_LD + D_MODEL + head * D_HEAD + c);
      *reinterpret_cast<uint4 *>(k_lds + r * K_PITCH + c * ES) = kv;
    }
    for (int idx = tid; idx < D_HEAD * (KB / CH); idx += 256) {
      const int d = idx / (KB / CH), c = (idx % (KB / CH)) * CH;
      *reinterpret_cast<uint4 *>(v_lds + d * V_PITCH + c * ES) =
          *reinterpret_cast<const uint4 *>(vhead + (size_t)d * S_pad + j0 + c);
    }
    __syncthreads();

    // S^T block: s[sb][r] = score(key j0 + 16 sb + 4g + r, query q), log2-scaled.
    float s[4][4];
    float mx = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      const char *krow = k_lds + (16 * sb + l16) * K_PITCH + g * 8 * ES;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc = mfma8(load8(reinterpret_cast<const T *>(krow + kk * 32 * ES)), qf[kk], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = j0 + 16 * sb + 4 * g + r;
        s[sb][r] = key < n_valid ? acc[r] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[sb][r]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, WAVE));
    mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
    const float m_new = fmaxf(m_run, mx);
    const float corr = exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[sb][r] = exp2f(s[sb][r] - m_new);
        psum += s[sb][r];
      }
    l_run = l_run * corr + psum;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= corr;

    // O^T[d][q] += Vt[d][keys] P^T[keys][q]; group g's 8 k-slots of half hf are
    // keys 32 hf + {4g..4g+3, 16+4g..16+4g+3}.
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      V8 pf;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pf[r] = from_f32<T>(s[2 * hf][r]);
        pf[4 + r] = from_f32<T>(s[2 * hf + 1][r]);
      }
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const char *vrow = v_lds + (16 * db + l16) * V_PITCH + (32 * hf + 4 * g) * ES;
        V8 vf;
        const T *lo = reinterpret_cast<const T *>(vrow);
        const T *hi = reinterpret_cast<const T *>(vrow + 16 * ES);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vf[e] = lo[e];
          vf[4 + e] = hi[e];
        }
        o[db] = mfma8(vf, pf, o[db]);
      }
    }
  }

  float l_tot = l_run + __shfl_xor(l_run, 16, WAVE);
  l_tot += __shfl_xor(l_tot, 32, WAVE);
  const float inv = 1.f / l_tot;
  if (q_ok) {
    T *dst = oseq + (size_t)q * D_MODEL + 4 * g;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      if constexpr (sizeof(T) == 4) {
        *reinterpret_cast<f32x4 *>(dst + 16 * db) = o[db] * inv;
      } else {
        *reinterpret_cast<f16x4 *>(dst + 16 * db) = f16x4{from_f32<T>(o[db][0] * inv), from_f32<T>(o[db][1] * inv),
                                                            from_f32<T>(o[db][2] * inv), from_f32<T>(o[db][3] * inv)};
      }
    }
  }
}

}  // namespace

template <typename T>
hipError_t attention(const T *qkv, const T *vt, T *out, const int32_t *lengths, int B, int P, int S, int S_pad,
                     hipStream_t stream) {
  if (P <= 0 || S <= 0) return hipSuccess;
  if (S_pad % KB != 0 || S_pad < S) return hipErrorInvalidValue;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D_HEAD);
  dim3 grid((S + QT - 1) / QT, D_MODEL / D_HEAD, P);
  launch("attention", attention_kernel<T>, grid, dim3(256), stream, qkv, vt, out, lengths, B, S, S_pad, scale_log2);
  return hipGetLastError();
}

template hipError_t attention<f16>(const f16 *, const f16 *, f16 *, const int32_t *, int, int, int, int, hipStream_t);
template hipError_t attention<float>(const float *, const float *, float *, const int32_t *, int, int, int, int,
                                     hipStream_t);

}  // namespace kmd
