// Data movement and elementwise stages of one DDIM step: sinusoid tables,
// token assembly, the root-stream gather, the global -> local root conversion
// fused with the body-input gather, and the CFG combine fused with the DDIM
// update (Kimodo WebGPU README, "Architecture" diagram: globalRootToLocalRoot,
// CFG guidance and DDIM update run between and after the two transformers; the
// WebGPU port does them in JS after a GPU->CPU readback, here they stay on the
// device). All of these are bandwidth-bound, and consecutive lanes touch
// consecutive addresses. The frame-row kernels (root gather, root conversion,
// CFG + DDIM) give each row one wavefront, so per-row values are found once;
// the row index is made wavefront-uniform, so the index arithmetic, the
// packing-table lookups and the root rows that every lane of the row reads are
// scalar work and scalar loads.
#include "common.h"
#include "kernels.h"

namespace kmd {
namespace {

constexpr int D = 1024;
constexpr int ROOT = 5, BODY = 274, FEATS = ROOT + BODY;

template <typename T>
__global__ void sinusoid_kernel(const int32_t *__restrict__ pos, int rows, T *__restrict__ out) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;  // (row, pair)
  if (idx >= rows * (D / 2)) return;
  const int r = idx / (D / 2), i = idx % (D / 2);
  const double t = pos ? (double)pos[r] : (double)r;
  const double ang = t * pow(10000.0, -2.0 * i / D);
  out[(size_t)r * D + 2 * i] = from_f32<T>((float)sin(ang));
  out[(size_t)r * D + 2 * i + 1] = from_f32<T>((float)cos(ang));
}

template <typename T>
__global__ void pad_cols_kernel(const T *__restrict__ src, int rows, int k, T *__restrict__ dst, int kpad) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * kpad) return;
  const int r = idx / kpad, c = idx % kpad;
  dst[idx] = c < k ? src[(size_t)r * k + c] : from_f32<T>(0.f);
}

template <typename T>
__global__ void text_rows_kernel(const float *__restrict__ text, int B, int dim, T *__restrict__ dst) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= 2 * B * dim) return;
  const int p = idx / dim;
  dst[idx] = from_f32<T>(p < B ? text[idx] : 0.f);
}

// Input rows of the two projections: one wavefront per row (p, f), four rows
// per workgroup. Lane l owns columns l, l + 64, ... (kpad <= 320), so every
// load and store instruction of a wavefront touches consecutive addresses.
constexpr int ROW_COLS = 5;  // column slots per lane: 5 * 64 = 320 >= 279

// Root-net input rows of the frames f < n_p - 2 of sequences p < P (motion
// row mot[p] + f): [x_t[p % B][f][0:5], 0 ...] (width kpad). The grid covers
// every (p, f); padded frames have no row.
template <typename T>
__global__ __launch_bounds__(256) void gather_root_kernel(const float *__restrict__ x_t, int B, int P, int T_,
                                                          const int32_t *__restrict__ mot, T *__restrict__ a_in,
                                                          int kpad) {
  const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= P * T_) return;
  const int p = row / T_, f = row - p * T_, b = p % B;
  const int f0 = mot[p];
  if (f >= mot[p + 1] - f0) return;
  const float *xb = x_t + ((size_t)b * T_ + f) * FEATS;
  T *dst = a_in + (size_t)(f0 + f) * kpad;
#pragma unroll
  for (int j = 0; j < ROW_COLS; ++j) {
    const int c = lane + 64 * j;
    if (c < kpad) dst[c] = from_f32<T>(c < ROOT ? xb[c] : 0.f);
  }
}

// 4 consecutive columns per thread. The grid covers every (p, s < T + 2);
// tokens past a sequence's n_p have no row.
template <typename T>
__global__ void assemble_kernel(const float *__restrict__ proj, const T *__restrict__ ttok,
                                const int32_t *__restrict__ step, const T *__restrict__ txtok,
                                const float *__restrict__ pe, T *__restrict__ h, int P, int T_,
                                const int32_t *__restrict__ tok, const int32_t *__restrict__ mot) {
  const int S = T_ + 2;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)P * S * (D / 4)) return;
  const int pos = (int)(idx / (D / 4)), c = (int)(idx % (D / 4)) * 4;
  const int p = pos / S, s = pos % S;
  const int f0 = mot[p];
  if (s >= mot[p + 1] - f0 + 2) return;
  const int row = tok[p] + s;
  const f32x4 pv = *reinterpret_cast<const f32x4 *>(pe + (size_t)s * D + c);
  float v[4];
  if (s >= 2) {
    const f32x4 x = *reinterpret_cast<const f32x4 *>(proj + ((size_t)f0 + s - 2) * D + c);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = x[e];
  } else {
    const T *src = s == 0 ? ttok + (size_t)(*step) * D + c : txtok + (size_t)p * D + c;
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = to_f32(src[e]);
  }
  T *dst = h + (size_t)row * D + c;
#pragma unroll
  for (int e = 0; e < 4; ++e) dst[e] = from_f32<T>(v[e] + pv[e]);
}

// Root prediction of frame f of row p: the root head's output, replaced at the
// caller's known entries (KNOWN: known / kmask [B, T, 279] of the row's clip).
// A known entry takes the caller's value in both guidance rows, before the
// conversion below, so the body network reads the constrained root. Both
// values are loaded and then selected: no per-lane branch around the loads.
template <bool KNOWN>
__device__ __forceinline__ void root_pred(const float *__restrict__ head_root, const float *__restrict__ known,
                                          const uint8_t *__restrict__ kmask, int row, int b, int f, int T_,
                                          float g[ROOT]) {
  const float *src = head_root + (size_t)row * ROOT;  // token row of frame f
#pragma unroll
  for (int c = 0; c < ROOT; ++c) g[c] = src[c];
  if (KNOWN) {
    const size_t k = ((size_t)b * T_ + f) * FEATS;
    float kv[ROOT];
    uint8_t km[ROOT];
#pragma unroll
    for (int c = 0; c < ROOT; ++c) {
      kv[c] = known[k + c];
      km[c] = kmask[k + c];
    }
#pragma unroll
    for (int c = 0; c < ROOT; ++c) g[c] = km[c] ? kv[c] : g[c];
  }
}

// Body-input rows: one wavefront per row (p, f), four rows per workgroup.
// Global root g = (x, y, z, c, s); p = x + iz, heading h = (c + is)/max(|c + is|, 1e-8).
// v = conj(h_f)(p_f - p_{f-1}) (0 at f = 0), r = conj(h_{f-1}) h_f (1 at f = 0);
// local = (Re v, y_f, Im v, Re r, Im r). The row's x_t columns are loaded
// first (lane l: columns l + 64 j); every lane then computes the row's local
// root from the same few addresses, and the row [l || x_t[b][f][5:279] || 0]
// is stored with consecutive lanes on consecutive columns. The grid covers
// every (p, f); padded frames have no head row and no input row (their
// local_out entries are 0).
template <typename T, bool KNOWN>
__global__ __launch_bounds__(256) void g2l_gather_kernel(const float *__restrict__ head_root,
                                                         const float *__restrict__ x_t,
                                                         const float *__restrict__ known,
                                                         const uint8_t *__restrict__ kmask, int B, int P, int T_,
                                                         const int32_t *__restrict__ tok,
                                                         const int32_t *__restrict__ mot, T *__restrict__ a_in,
                                                         int kpad, float *__restrict__ local_out) {
  const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= P * T_) return;
  const int p = row / T_, f = row - p * T_, b = p % B;
  const int t0 = tok[p], f0 = mot[p];
  if (f >= mot[p + 1] - f0) {
    if (local_out && lane < ROOT) local_out[(size_t)row * ROOT + lane] = 0.f;
    return;
  }
  const float *xb = x_t + ((size_t)b * T_ + f) * FEATS;
  float v[ROW_COLS];
#pragma unroll
  for (int j = 0; j < ROW_COLS; ++j) {
    const int c = lane + 64 * j;
    v[j] = c >= ROOT && c < FEATS ? xb[c] : 0.f;
  }
  float g[ROOT];
  root_pred<KNOWN>(head_root, known, kmask, t0 + 2 + f, b, f, T_, g);
  const float hn = fmaxf(sqrtf(g[3] * g[3] + g[4] * g[4]), 1e-8f);
  const float hc = g[3] / hn, hs = g[4] / hn;
  float l[ROOT];
  if (f == 0) {
    l[0] = 0.f; l[2] = 0.f; l[3] = 1.f; l[4] = 0.f;
  } else {
    float q[ROOT];
    root_pred<KNOWN>(head_root, known, kmask, t0 + 1 + f, b, f - 1, T_, q);
    const float qn = fmaxf(sqrtf(q[3] * q[3] + q[4] * q[4]), 1e-8f);
    const float qc = q[3] / qn, qs = q[4] / qn;
    const float dx = g[0] - q[0], dz = g[2] - q[2];
    l[0] = hc * dx + hs * dz;
    l[2] = hc * dz - hs * dx;
    l[3] = qc * hc + qs * hs;
    l[4] = qc * hs - qs * hc;
  }
  l[1] = g[1];
  // columns 0 .. 4 (the local root) belong to lanes 0 .. 4 of slot 0
#pragma unroll
  for (int e = 0; e < ROOT; ++e)
    if (lane == e) v[0] = l[e];
  if (local_out && lane < ROOT) local_out[(size_t)row * ROOT + lane] = v[0];
  T *dst = a_in + (size_t)(f0 + f) * kpad;
#pragma unroll
  for (int j = 0; j < ROW_COLS; ++j) {
    const int c = lane + 64 * j;
    if (c < kpad) dst[c] = from_f32<T>(v[j]);
  }
}

// CFG + DDIM of x [B, T, 279]: one wavefront per frame row (b, f), four rows
// per workgroup; lane l owns features l + 64 j. All of a lane's loads (the
// state, both guidance rows of the two heads, the known entries) are issued
// before any result is formed. A padded frame has no head rows: its x_prev
// (and traced x0) is 0. The head rows of clip b's frame f are token rows
// tok_g[b] + 2 + f (conditional) and tok_g[B + b] + 2 + f (unconditional).
// A known entry (kmask set) has the caller's value in both guidance rows, so
// its x0 is that value.
template <bool KNOWN>
__global__ __launch_bounds__(256) void cfg_ddim_kernel(const float *__restrict__ head_root,
                                                       const float *__restrict__ head_body, const float *x_t,
                                                       float *x_prev, const float *__restrict__ coef,
                                                       const int32_t *__restrict__ step,
                                                       const int32_t *__restrict__ lengths,
                                                       const int32_t *__restrict__ tok_g,
                                                       const float *__restrict__ known,
                                                       const uint8_t *__restrict__ kmask, int B, int T_, float w,
                                                       float *__restrict__ x0_out) {
  const int row = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;  // row = b * T + f
  if (row >= B * T_) return;
  const int b = row / T_, f = row - b * T_;
  const size_t base = (size_t)row * FEATS;
  if (f >= lengths[b]) {
#pragma unroll
    for (int j = 0; j < ROW_COLS; ++j) {
      const int c = lane + 64 * j;
      if (c < FEATS) {
        x_prev[base + c] = 0.f;
        if (x0_out) x0_out[base + c] = 0.f;
      }
    }
    return;
  }
  const size_t rc = (size_t)tok_g[b] + 2 + f, ru = (size_t)tok_g[B + b] + 2 + f;
  float cv[ROW_COLS], uv[ROW_COLS], xv[ROW_COLS], kv[ROW_COLS];
  uint8_t km[ROW_COLS];
#pragma unroll
  for (int j = 0; j < ROW_COLS; ++j) {
    const int c = lane + 64 * j;
    cv[j] = uv[j] = xv[j] = kv[j] = 0.f;
    km[j] = 0;
    if (c < FEATS) {
      if (c < ROOT) {
        cv[j] = head_root[rc * ROOT + c];
        uv[j] = head_root[ru * ROOT + c];
      } else {
        cv[j] = head_body[rc * BODY + c - ROOT];
        uv[j] = head_body[ru * BODY + c - ROOT];
      }
      xv[j] = x_t[base + c];
      if (KNOWN) {
        kv[j] = known[base + c];
        km[j] = kmask[base + c];
      }
    }
  }
  const int k = *step;
  const float cx0 = coef[2 * k], cxt = coef[2 * k + 1];
#pragma unroll
  for (int j = 0; j < ROW_COLS; ++j) {
    const int c = lane + 64 * j;
    if (c >= FEATS) continue;
    float x0 = uv[j] + w * (cv[j] - uv[j]);
    if (KNOWN) x0 = km[j] ? kv[j] : x0;
    if (x0_out) x0_out[base + c] = x0;
    x_prev[base + c] = cx0 * x0 + cxt * xv[j];
  }
}

// row_ps: one thread per (p, s < S8); rows tok[p] + s of sequence p, its
// dead rows included, up to tok[p + 1].
__global__ void packing_maps_kernel(const int32_t *__restrict__ tok, int P, int S8, int32_t *__restrict__ row_ps) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= P * S8) return;
  const int p = idx / S8, s = idx - p * S8;
  const int t0 = tok[p];
  if (s < tok[p + 1] - t0) row_ps[t0 + s] = (p << 16) | s;
}

// Dense copies of packed rows (traces): one thread per 4 bytes of (p, s) with
// s < S_dst; rows s < n_p - first come from src row tok[p] + first + s, the
// rest are 0.
__global__ void unpack_rows_kernel(const uint32_t *__restrict__ src, int width_words, const int32_t *__restrict__ tok,
                                   const int32_t *__restrict__ mot, int P, int first, int S_dst,
                                   uint32_t *__restrict__ dst) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)P * S_dst * width_words) return;
  const int c = (int)(idx % width_words);
  const int pos = (int)(idx / width_words), p = pos / S_dst, s = pos - p * S_dst;
  const int n = mot[p + 1] - mot[p] + 2 - first;
  dst[idx] = s < n ? src[(size_t)(tok[p] + first + s) * width_words + c] : 0u;
}

// Known entries of a timeline segment: its first n_tr frames (all features)
// are frames f0 .. f0 + n_tr - 1 of the timeline written so far (src: [V, total,
// 279]); the rest of the segment is free.
__global__ void tail_known_kernel(const float *__restrict__ src, int total, int f0, int V, int T_, int n_tr,
                                  float *__restrict__ known, uint8_t *__restrict__ kmask) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)V * T_ * FEATS) return;
  const int c = (int)(idx % FEATS);
  const int f = (int)((idx / FEATS) % T_);
  const int v = (int)(idx / ((size_t)FEATS * T_));
  const bool k = f < n_tr;
  known[idx] = k ? src[((size_t)v * total + f0 + f) * FEATS + c] : 0.f;
  kmask[idx] = k ? 1 : 0;
}

__global__ void fill_int_kernel(int32_t *__restrict__ dst, int n, int32_t v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = v;
}

// Weight set-up: converts src (fp32, bf16 or fp16) to TD, or with dst null
// only reads it; any value that is not finite after conversion (a bf16 weight
// beyond the fp16 range becomes inf) sets *bad to 1.
template <typename TD>
__global__ void convert_kernel(const void *__restrict__ src, int src_type, TD *__restrict__ dst, size_t n,
                               int32_t *__restrict__ bad) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float v;
  if (src_type == 0) v = static_cast<const float *>(src)[i];
  else if (src_type == 1) v = (float)static_cast<const bf16 *>(src)[i];
  else v = (float)static_cast<const f16 *>(src)[i];
  const TD out = from_f32<TD>(v);
  if (dst) dst[i] = out;
  if (!__builtin_isfinite((float)out)) bad[0] = 1;
}

template <typename T>
__global__ void fill_zero_kernel(T *__restrict__ dst, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = from_f32<T>(0.f);
}

__global__ void step_advance_kernel(int32_t *step) { step[0] -= 1; }
__global__ void set_int_kernel(int32_t *dst, int32_t v) { dst[0] = v; }

inline dim3 blocks(size_t n, int bs = 256) { return dim3((unsigned)((n + bs - 1) / bs)); }

}  // namespace

template <typename T> hipError_t sinusoid(const int32_t *pos, int rows, T *out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  launch("sinusoid", sinusoid_kernel<T>, blocks((size_t)rows * (D / 2)), dim3(256), s, pos, rows, out);
  return hipGetLastError();
}

template <typename T> hipError_t pad_cols(const T *src, int rows, int k, T *dst, int kpad, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  launch("pad_cols", pad_cols_kernel<T>, blocks((size_t)rows * kpad), dim3(256), s, src, rows, k, dst, kpad);
  return hipGetLastError();
}

template <typename T> hipError_t text_rows(const float *text, int B, T *dst, hipStream_t s) {
  launch("text_rows", text_rows_kernel<T>, blocks((size_t)2 * B * 4096), dim3(256), s, text, B, 4096, dst);
  return hipGetLastError();
}

template <typename T>
hipError_t gather_root(const float *x_t, int B, int P, int T_, const int32_t *mot, T *a_in, int kpad,
                       hipStream_t s) {
  if (P <= 0 || T_ <= 0) return hipSuccess;
  if (kpad < ROOT || kpad > 64 * ROW_COLS) return hipErrorInvalidValue;
  launch("gather_root", gather_root_kernel<T>, dim3((unsigned)((P * T_ + 3) / 4)), dim3(256), s, x_t, B, P, T_, mot,
         a_in, kpad);
  return hipGetLastError();
}

template <typename T>
hipError_t assemble_tokens(const float *proj, const T *ttok, const int32_t *step, const T *txtok, const float *pe,
                           T *h, int P, int T_, const int32_t *tok, const int32_t *mot, hipStream_t s) {
  launch("assemble", assemble_kernel<T>, blocks((size_t)P * (T_ + 2) * (D / 4)), dim3(256), s, proj, ttok, step,
                     txtok, pe, h, P, T_, tok, mot);
  return hipGetLastError();
}

template <typename T>
hipError_t g2l_gather(const float *head_root, const float *x_t, const float *known, const uint8_t *kmask, int B,
                      int P, int T_, const int32_t *tok, const int32_t *mot, T *a_in, int kpad, float *local_out,
                      hipStream_t s) {
  if (P <= 0 || T_ <= 0) return hipSuccess;
  if (kpad < FEATS || kpad > 64 * ROW_COLS) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((P * T_ + 3) / 4));
  if (kmask)
    launch("g2l_gather", g2l_gather_kernel<T, true>, grid, dim3(256), s, head_root, x_t, known, kmask, B, P, T_, tok,
           mot, a_in, kpad, local_out);
  else
    launch("g2l_gather", g2l_gather_kernel<T, false>, grid, dim3(256), s, head_root, x_t, known, kmask, B, P, T_,
           tok, mot, a_in, kpad, local_out);
  return hipGetLastError();
}

hipError_t cfg_ddim(const float *head_root, const float *head_body, const float *x_t, float *x_prev,
                    const float *coef, const int32_t *step, const int32_t *lengths, const int32_t *tok_g,
                    const float *known, const uint8_t *kmask, int B, int T_, float w, float *x0_out, hipStream_t s) {
  if (B <= 0 || T_ <= 0) return hipSuccess;
  const dim3 grid((unsigned)((B * T_ + 3) / 4));
  if (kmask)
    launch("cfg_ddim", cfg_ddim_kernel<true>, grid, dim3(256), s, head_root, head_body, x_t, x_prev, coef, step,
           lengths, tok_g, known, kmask, B, T_, w, x0_out);
  else
    launch("cfg_ddim", cfg_ddim_kernel<false>, grid, dim3(256), s, head_root, head_body, x_t, x_prev, coef, step,
           lengths, tok_g, known, kmask, B, T_, w, x0_out);
  return hipGetLastError();
}

hipError_t tail_known(const float *src, int total, int f0, int V, int T_, int n_tr, float *known, uint8_t *kmask,
                      hipStream_t s) {
  launch("tail_known", tail_known_kernel, blocks((size_t)V * T_ * FEATS), dim3(256), s, src, total, f0, V, T_, n_tr,
                     known, kmask);
  return hipGetLastError();
}

hipError_t fill_int(int32_t *dst, int n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  launch("fill_int", fill_int_kernel, blocks((size_t)n), dim3(256), s, dst, n, v);
  return hipGetLastError();
}

hipError_t packing_maps(const int32_t *tok, int P, int S8, int32_t *row_ps, hipStream_t s) {
  if (P <= 0 || S8 <= 0) return hipSuccess;
  if (S8 % 8) return hipErrorInvalidValue;
  launch("packing_maps", packing_maps_kernel, blocks((size_t)P * S8), dim3(256), s, tok, P, S8, row_ps);
  return hipGetLastError();
}

hipError_t unpack_rows(const void *src, int width_bytes, const int32_t *tok, const int32_t *mot, int P, int first,
                       int S_dst, void *dst, hipStream_t s) {
  if (P <= 0 || S_dst <= 0) return hipSuccess;
  if (width_bytes % 4 || reinterpret_cast<uintptr_t>(src) % 4 || reinterpret_cast<uintptr_t>(dst) % 4)
    return hipErrorInvalidValue;
  const int ww = width_bytes / 4;
  launch("unpack_rows", unpack_rows_kernel, blocks((size_t)P * S_dst * ww), dim3(256), s,
         static_cast<const uint32_t *>(src), ww, tok, mot, P, first, S_dst, static_cast<uint32_t *>(dst));
  return hipGetLastError();
}

hipError_t convert_f16(const void *src, int src_type, f16 *dst, size_t n, int32_t *bad, hipStream_t s) {
  if (n == 0) return hipSuccess;
  launch("convert", convert_kernel<f16>, blocks(n), dim3(256), s, src, src_type, dst, n, bad);
  return hipGetLastError();
}

hipError_t convert_f32(const void *src, int src_type, float *dst, size_t n, int32_t *bad, hipStream_t s) {
  if (n == 0) return hipSuccess;
  launch("convert", convert_kernel<float>, blocks(n), dim3(256), s, src, src_type, dst, n, bad);
  return hipGetLastError();
}

template <typename T> hipError_t fill_zero(T *dst, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  launch("fill_zero", fill_zero_kernel<T>, blocks(n), dim3(256), s, dst, n);
  return hipGetLastError();
}
template hipError_t fill_zero<f16>(f16 *, size_t, hipStream_t);
template hipError_t fill_zero<float>(float *, size_t, hipStream_t);

hipError_t step_advance(int32_t *step, hipStream_t s) {
  launch("step_advance", step_advance_kernel, dim3(1), dim3(1), s, step);
  return hipGetLastError();
}

hipError_t set_int(int32_t *dst, int32_t v, hipStream_t s) {
  launch("set_int", set_int_kernel, dim3(1), dim3(1), s, dst, v);
  return hipGetLastError();
}

#define KMD_INST(T)                                                                                          \
  template hipError_t sinusoid<T>(const int32_t *, int, T *, hipStream_t);                                   \
  template hipError_t pad_cols<T>(const T *, int, int, T *, int, hipStream_t);                               \
  template hipError_t text_rows<T>(const float *, int, T *, hipStream_t);                                    \
  template hipError_t gather_root<T>(const float *, int, int, int, const int32_t *, T *, int, hipStream_t);  \
  template hipError_t assemble_tokens<T>(const float *, const T *, const int32_t *, const T *, const float *, \
                                         T *, int, int, const int32_t *, const int32_t *, hipStream_t);      \
  template hipError_t g2l_gather<T>(const float *, const float *, const float *, const uint8_t *, int, int, int, \
                                    const int32_t *, const int32_t *, T *, int, float *, hipStream_t);
KMD_INST(f16)
KMD_INST(float)
#undef KMD_INST

}  // namespace kmd
