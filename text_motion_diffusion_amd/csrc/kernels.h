// Host-side launchers of the gfx950 kernels. Every launcher enqueues on
// `stream` and returns hipGetLastError() of the launch; shapes are checked by
// the caller (kimodo.hip) before anything is enqueued.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kmd {

typedef __bf16 bf16;
typedef _Float16 f16;

// Optional per-launch timing. While a KernelTimer is installed on the calling
// host thread, every launch goes through hipExtLaunchKernelGGL with a start and
// a stop event that the dispatch itself records around the kernel.
struct KernelTimer {
  virtual bool slot(const char *name, hipEvent_t *start, hipEvent_t *stop) = 0;
};
KernelTimer *&kernel_timer();

template <typename K, typename... Args>
inline void launch(const char *name, K kernel, dim3 grid, dim3 block, hipStream_t s, Args... args) {
  KernelTimer *t = kernel_timer();
  hipEvent_t a, b;
  if (t && t->slot(name, &a, &b))
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, a, b, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
}

// The projections of the denoiser. The role fixes the epilogue and the output
// type (each role is its own kernel symbol, so profiles separate them):
//   QKV, OUT, FFN2, TXT, TMLP2: bias, output T;  FFN1: bias + GELU, output T;
//   TMLP1: bias + SiLU, output T;  IN, HEAD: bias, output fp32.
enum GemmRole { ROLE_QKV, ROLE_OUT, ROLE_FFN1, ROLE_FFN2, ROLE_IN, ROLE_HEAD, ROLE_TXT, ROLE_TMLP1, ROLE_TMLP2 };

// Token rows of a kernel chain of P sequences, packed: sequence p has
// n_p = mot[p + 1] - mot[p] + 2 tokens (its length + 2) at rows tok[p] ..
// tok[p] + n_p - 1, and its frames at motion rows mot[p] + f. Each sequence
// starts on a multiple of 8 rows (tok[p + 1] - tok[p] = n_p rounded up to 8):
// the up to 7 rows after its tokens are dead rows, computed by the row-wise
// kernels like any other and never read into a live row, and every 8-row run
// lies in one sequence. Padded frames have no rows. row_ps[r] = (p << 16) | s
// for every row r < tok[P], dead rows included (s >= n_p). All device arrays,
// built per call from the lengths.
struct Packing {
  const int32_t *tok = nullptr;     // [P + 1]
  const int32_t *mot = nullptr;     // [P + 1]
  const int32_t *row_ps = nullptr;  // [tok[P]]
};

// Extra epilogue target of the QKV projection: the V columns are written
// transposed to vt[p][head][d][seq_pad] for the token (p, s) of row m, given
// by pk (the attention kernel reads keys contiguously). Dead rows write
// positions n_p .. of their sequence; the rows past that are never written.
// Either way positions past a sequence's tokens must hold finite values.
struct GemmAux {
  void *vt = nullptr;
  int seq_pad = 1;
  Packing pk;
  // fp16 GEMMs with few output tiles split K across workgroups when given a
  // buffer for the fp32 partial sums (up to partial_cap floats).
  float *partial = nullptr;
  size_t partial_cap = 0;
};

// K extent of one GEMM k-tile: 128 bytes of operand per row.
template <typename T> constexpr int gemm_k_tile() { return 128 / (int)sizeof(T); }

// C[m, n] = epi(sum_k A[m, k] W[n, k] + bias[n]) for m < M, n < N.
// A [M, lda] and W [N, ldw] in T, both K-contiguous, 16-byte aligned rows;
// K % gemm_k_tile<T>() == 0; bias fp32 [N]. C has row stride ldc.
template <typename T>
hipError_t gemm(GemmRole role, const T *A, int lda, const T *W, int ldw, const float *bias, void *C, int ldc, int M,
                int N, int K, hipStream_t stream, const GemmAux &aux = GemmAux());

// Split-K partial sums only: if the GEMM A W^T (as in gemm) qualifies for
// split-K, writes its fp32 partials aux.partial[split][M][N] and sets *splits;
// otherwise launches nothing and sets *splits = 1. The caller reduces.
// name labels the launch for per-kernel timing.
template <typename T>
hipError_t gemm_partials(const char *name, const T *A, int lda, const T *W, int ldw, int M, int N, int K,
                         const GemmAux &aux, int *splits, hipStream_t stream);

// Masked multi-head self-attention over the fused QKV rows of P sequences of
// at most S tokens, packed by tok and mot (see Packing): Q and K from qkv
// [rows][3*1024] (columns 0..2047), V from its transposed copy vt
// [P][8][128][S_pad] (S_pad a multiple of 64, positions past a sequence's
// tokens finite), out [rows][1024], written on live rows only. Sequence p
// attends to its n_p tokens.
template <typename T>
hipError_t attention(const T *qkv, const T *vt, T *out, const int32_t *tok, const int32_t *mot, int P, int S,
                     int S_pad, hipStream_t stream);
// fp16, S <= 160 (the longest sequence's tokens; it sizes the kernel): QKV
// projection of the packed token rows h [rows][1024] with W
// [3072][1024] and bias [3072], then masked attention, straight into out
// [rows][1024] on live rows (Q, K, V stay on chip).
hipError_t qkv_attention(const f16 *h, const f16 *wqkv, const float *bqkv, f16 *out, const int32_t *tok,
                         const int32_t *mot, int P, int S, hipStream_t stream);
// dst[0:n] = 0
template <typename T> hipError_t fill_zero(T *dst, size_t n, hipStream_t stream);

// out = LayerNorm(x + y) * gamma + beta over rows of 1024, eps 1e-5.
// out = LN(x + sum_{s < splits} P[s] + bias) * gamma + beta, P fp32
// [splits][M][1024] split-K partials of the projection feeding the residual.
template <typename T>
hipError_t add_layernorm_splitk(const T *x, const float *P, int splits, const float *bias, const float *gamma,
                                const float *beta, T *out, int M, hipStream_t stream);
template <typename T>
hipError_t add_layernorm(const T *x, const T *y, const float *gamma, const float *beta, T *out, int M,
                         hipStream_t stream);

// --- elementwise / data movement -----------------------------------------
// Sinusoid rows: out[r][2i] = sin(pos[r] w_i), out[r][2i+1] = cos(pos[r] w_i),
// w_i = 10000^(-2i/1024). pos == NULL means pos[r] = r.
template <typename T> hipError_t sinusoid(const int32_t *pos, int rows, T *out, hipStream_t stream);
// dst[r][0:kpad] = [src[r][0:k], 0...]
template <typename T> hipError_t pad_cols(const T *src, int rows, int k, T *dst, int kpad, hipStream_t stream);
// text rows: dst[b] = text[b], dst[B + b] = 0 (the unconditional rows).
template <typename T> hipError_t text_rows(const float *text, int B, T *dst, hipStream_t stream);
// Root-net input rows (motion row mot[p] + f of frame f < n_p - 2 of
// sequence p < P): [x_t[p % B][f][0:5], 0 ...] (width kpad).
template <typename T>
hipError_t gather_root(const float *x_t, int B, int P, int T_, const int32_t *mot, T *a_in, int kpad,
                       hipStream_t stream);
// h[tok[p] + s] = (s == 0 ? ttok[*step] : s == 1 ? txtok[p] : proj[mot[p] + s - 2]) + pe[s], s < n_p
template <typename T>
hipError_t assemble_tokens(const float *proj, const T *ttok, const int32_t *step, const T *txtok, const float *pe,
                           T *h, int P, int T_, const int32_t *tok, const int32_t *mot, hipStream_t stream);
// Global -> local root conversion of the root head rows (token rows tok[p] + 2
// + f) of sequences p < P and the body-net input rows [l || x_t[p % B][f][5:279]
// || 0...] (width kpad, motion rows). known / kmask (fp32 and u8 [B][T][279],
// both NULL when there are no constraints): root entries with kmask set take
// the known value before the conversion. local_out (fp32 [P][T][5], padded
// frames 0) may be NULL.
template <typename T>
hipError_t g2l_gather(const float *head_root, const float *x_t, const float *known, const uint8_t *kmask, int B,
                      int P, int T_, const int32_t *tok, const int32_t *mot, T *a_in, int kpad, float *local_out,
                      hipStream_t stream);
// CFG combine + DDIM update + zeroing of padded frames, scalars read at
// coef[*step] = (c_x0, c_xt); x0 = known where kmask is set (both may be
// NULL). The head rows of sequence p start at token row tok_g[p] (p < 2B).
// x0_out (fp32 [B][T][279], padded frames 0) may be NULL.
hipError_t cfg_ddim(const float *head_root, const float *head_body, const float *x_t, float *x_prev,
                    const float *coef, const int32_t *step, const int32_t *lengths, const int32_t *tok_g,
                    const float *known, const uint8_t *kmask, int B, int T_, float w, float *x0_out,
                    hipStream_t stream);
// row_ps of P sequences of at most S8 rows each (a multiple of 8), from tok
// (see Packing).
hipError_t packing_maps(const int32_t *tok, int P, int S8, int32_t *row_ps, hipStream_t stream);
// dst[p][s][0:width] = src[tok[p] + s + first][0:width] for s < n_p - first,
// 0 for the rest of s < S_dst (dense trace copies of packed rows; width a
// multiple of 4 bytes).
hipError_t unpack_rows(const void *src, int width_bytes, const int32_t *tok, const int32_t *mot, int P, int first,
                       int S_dst, void *dst, hipStream_t stream);
// Timeline segment constraints: known / kmask [V][T][279] = frames f0 .. f0 +
// n_tr - 1 of src [V][total][279] on the first n_tr frames, free elsewhere.
hipError_t tail_known(const float *src, int total, int f0, int V, int T_, int n_tr, float *known, uint8_t *kmask,
                      hipStream_t stream);
// dst[0 .. n-1] = v
hipError_t fill_int(int32_t *dst, int n, int32_t v, hipStream_t stream);

// Skeleton of the FK decode, passed by value: joints in topological order,
// parent[0] = -1, 0 <= parent[j] < j; offset[j] in the parent's frame;
// rounds = ceil(log2(max depth + 1)), the pointer-jumping rounds.
constexpr int FK_MAX_ROUNDS = 5;  // ceil(log2(30)): the deepest 30-joint chain
struct FkSkeleton {
  int32_t parent[32];
  float offset[32][3];
  int32_t rounds;
  // anc[r][j]: the joint whose transform lane j composes with in pointer-
  // jumping round r (its 2^r-th ancestor), -1 once the path reaches the root
  int32_t anc[FK_MAX_ROUNDS][32];
};
// Joint positions pos [n][30][3] and, if rot is not NULL, global rotation
// matrices rot [n][30][3][3] (row-major) of n motion frames x [n][279].
hipError_t fk_decode(const float *x, int n, const FkSkeleton &sk, float *pos, float *rot, hipStream_t stream);
// *step -= 1
hipError_t step_advance(int32_t *step, hipStream_t stream);
// Weight set-up: src (0 fp32, 1 bf16, 2 fp16) converted into dst, or only
// checked when dst is null; *bad is set to 1 if a converted value is not finite.
hipError_t convert_f16(const void *src, int src_type, f16 *dst, size_t n, int32_t *bad, hipStream_t stream);
hipError_t convert_f32(const void *src, int src_type, float *dst, size_t n, int32_t *bad, hipStream_t stream);
// step[0] = value (graph-safe replacement for a memset)
hipError_t set_int(int32_t *dst, int32_t value, hipStream_t stream);

}  // namespace kmd
