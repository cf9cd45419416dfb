// Multi-head self-attention with key masking (Kimodo WebGPU README, "WGSL
// compute shaders" table, attention.wgsl row; the qkv_split.wgsl step of the
// same table is not needed: Q, K and V are read in place from the
// fused projection rows [q | k | v], head j at columns 128j .. 128j+127 of each).
//
// Three kernels: attention_kernel (below; fp32, and the reference layout of
// the math), attention_f16_kernel (fp16, 32 queries per wavefront, for grids
// of at least one workgroup per CU) and attention_f16_q16_kernel (fp16, 16
// queries per wavefront, for 1 to 8 sequences, where twice the wavefronts
// hide more latency).
//
// fp32: per (sequence p, head h, 64-query tile) one 256-thread workgroup; each of
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
                                                        T *__restrict__ out, const int32_t *__restrict__ tok,
                                                        const int32_t *__restrict__ mot, int S, int S_pad,
                                                        float scale_log2) {
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
  // sequence p: its n_valid tokens at packed rows tok[p] ..
  const int n_valid = mot[p + 1] - mot[p] + 2;
  const int q_tile0 = blockIdx.x * QT;
  if (q_tile0 >= n_valid) return;  // no token rows in this tile
  const T *seq = qkv + (size_t)tok[p] * QKV_LD;
  const T *vhead = vt + ((size_t)p * (D_MODEL / D_HEAD) + head) * D_HEAD * S_pad;  // [d][S_pad]
  T *oseq = out + (size_t)tok[p] * D_MODEL + head * D_HEAD;

  const int q = q_tile0 + wave * 16 + l16;
  const bool q_ok = q < n_valid;
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
    // Vt positions past the sequence's keys hold whatever an earlier call
    // left there; they are stored as exact zeros, so that their zero weights
    // give zero products whatever those values are.
    for (int idx = tid; idx < D_HEAD * (KB / CH); idx += 256) {
      const int d = idx / (KB / CH), c = (idx % (KB / CH)) * CH;
      uint4 raw = *reinterpret_cast<const uint4 *>(vhead + (size_t)d * S_pad + j0 + c);
      const int nv = n_valid - (j0 + c);  // valid keys in this 16-byte chunk
      if (nv < CH) {
        T e[CH];
        __builtin_memcpy(e, &raw, 16);
#pragma unroll
        for (int i = 0; i < CH; ++i) e[i] = i < nv ? e[i] : T(0);
        __builtin_memcpy(&raw, e, 16);
      }
      *reinterpret_cast<uint4 *>(v_lds + d * V_PITCH + c * ES) = raw;
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

// fp16 kernel. One workgroup per (sequence p, head, chunk of up to 384
// queries): NW <= 12 wavefronts of 32 queries each, so a sequence of up to
// 382 tokens is one chunk and its K and V stream through LDS once per head.
// One workgroup per CU (167 VGPRs: three wavefronts per SIMD; the output
// staging takes 104 KB of LDS). Key blocks of 64 arrive by direct-to-LDS
// loads (buffer_load ... lds, 16 bytes per lane) in two stages: the loads of
// block b+1 are issued when block b starts. K rows (256 bytes) are stored
// with 16-byte chunk c at c ^ sw23(row & 15) (sw23 swaps bits 2 and 3, the
// order in which the MFMA rows take the keys below), Vt rows (64 keys, 128
// bytes) with chunk c at c ^ swz8(d): each 16-byte fragment read then hits
// disjoint banks in every group of 8 lanes and of 16 lanes.
//
// Per wavefront and key block, on the 32x32x16 MFMA:
//   S^T[64 keys][32 queries] = K Q^T: two 32-key blocks x 8 steps of 16 d;
//     the Q fragments (32 queries x 128 d) stay in registers. Output row
//     i of a 32-key block is fed the K row with bits 2 and 3 of i swapped,
//     so lane l (query l % 32, g = l / 32) ends up with the scores of keys
//     32 kb + 16 h + 8 g + 0..7 in accumulator entries 8 h + 0..7.
//   Online softmax in fp32 (exp2, scale folded in): the two lanes of a query
//     (l, l ^ 32) meet in one cross-lane step for the block maximum; each
//     keeps its own partial sum until the end.
//   O^T[128 d][32 queries] += Vt P^T: four d blocks x 4 steps of 16 keys. The
//     scores a lane holds are exactly the P^T fragment it must supply (step
//     j = 2 kb + h: keys 16 j + 8 g + 0..7), so P needs no shuffle; the Vt
//     fragment is the same 8 consecutive keys of row d, one 16-byte chunk.
// Each K and Vt fragment read from LDS feeds 32 queries (16x16 tiles would
// feed 16), which halves the LDS traffic per flop of the 16-query form.
// Masked keys (>= length + 2) get -inf and zero Vt entries. The output goes
// through LDS and is stored as whole 256-byte rows of the head's slice.
// Wavefronts whose queries are all padding skip the math (they still issue
// loads and meet the barriers). Workgroup i serves head i % 8, so XCD x
// serves head x.
constexpr int ATT_MAX_WAVES = 12, ATT_QW = 32;  // wavefronts per workgroup, queries per wavefront
constexpr int ATT_CHUNK_Q = ATT_MAX_WAVES * ATT_QW;

constexpr int WAIT_ALL = waitcnt_imm(0, 0);

// Zeroes the Vt entries of keys nv .. 63 of a staged 64-key block (D_HEAD
// rows of 128 bytes, 16-byte chunk c of row d at c ^ swz8(d)). Every thread
// of the workgroup calls it; eight consecutive threads cover one row.
__device__ __forceinline__ void zero_vt_tail(char *vs, int nv, int tid, int n_threads) {
  for (int e = tid; e < D_HEAD * 8; e += n_threads) {
    const int d = e >> 3, c = e & 7, k0 = 8 * c;
    if (k0 + 8 <= nv) continue;
    f16x8 *chunk = reinterpret_cast<f16x8 *>(vs + d * (KB * 2) + ((c ^ swz8(d)) * 16));
    f16x8 v = k0 >= nv ? zero8<f16>() : *chunk;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (k0 + i >= nv) v[i] = (f16)0.f;
    *chunk = v;
  }
}

__global__ __launch_bounds__(64 * ATT_MAX_WAVES, 1) void attention_f16_kernel(
    const f16 *__restrict__ qkv, const f16 *__restrict__ vt, f16 *__restrict__ out,
    const int32_t *__restrict__ tok, const int32_t *__restrict__ mot, int P, int S, int S_pad, int n_chunks,
    int q_chunk, float scale_log2) {
  constexpr int K_ROW = D_HEAD * 2;          // 256 bytes per key row
  constexpr int V_ROW = KB * 2;              // 128 bytes per d row of a 64-key block
  constexpr int K_STAGE = KB * K_ROW;        // 16 KB
  constexpr int STAGE = K_STAGE + D_HEAD * V_ROW;  // + 16 KB
  constexpr int O_PITCH = D_HEAD * 2 + 16;   // staged output row
  constexpr int LDS = 2 * STAGE > ATT_MAX_WAVES * ATT_QW * O_PITCH ? 2 * STAGE : ATT_MAX_WAVES * ATT_QW * O_PITCH;
  __shared__ __attribute__((aligned(1024))) char lds[LDS];

  const int head = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int p = slot / n_chunks, chunk = slot - p * n_chunks;
  if (p >= P) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), NW = blockDim.x / 64;
  const int l32 = lane & 31, g = lane >> 5;
  const int t0 = tok[p], n_valid = mot[p + 1] - mot[p] + 2;  // sequence p's tokens, from packed row t0
  const int q_base = chunk * q_chunk + wave * ATT_QW;
  const bool active = q_base < n_valid;

  // Buffer resources: the sequence's K columns of this head (rows past its
  // tokens read as zero) and its Vt block [128][S_pad].
  const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(qkv + (size_t)t0 * QKV_LD + D_MODEL + head * D_HEAD), (short)0, n_valid * QKV_LD * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(vt + ((size_t)p * 8 + head) * D_HEAD * S_pad), (short)0, D_HEAD * S_pad * 2, 0x00020000);
  // Load instruction i < 16: K rows 4i .. 4i+3 of the block; i >= 16: Vt rows
  // d = 8(i-16) .. +7. Lane l writes LDS byte 16 l of the instruction's 1 KB.
  const int k_row = lane >> 4, k_chunk = lane & 15;
  auto sw23 = [](int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); };
  auto issue = [&](int blk, int stage) {
    char *base = lds + stage * STAGE;
    for (int i = wave; i < 32; i += NW) {
      if (i < 16) {
        const int r = 4 * i + k_row;
        const int voff = (KB * blk + r) * QKV_LD * 2 + ((k_chunk ^ sw23(r & 15)) * 16);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(k_rsrc, (__attribute__((address_space(3))) void *)(base + i * 1024),
                                                 16, voff, 0, 0, 0);
      } else {
        const int d = 8 * (i - 16) + (lane >> 3);
        const int voff = d * S_pad * 2 + (KB * blk + 8 * ((lane & 7) ^ swz8(d))) * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            v_rsrc, (__attribute__((address_space(3))) void *)(base + K_STAGE + (i - 16) * 1024), 16, voff, 0, 0, 0);
      }
    }
  };

  // Q^T fragments: query q_base + l32, d = 16 ks + 8 g .. + 7.
  const int q = q_base + l32;
  const bool q_ok = active && q < n_valid;
  f16x8 qf[8];
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    qf[ks] = q_ok ? load8(qkv + ((size_t)t0 + q) * QKV_LD + head * D_HEAD + 16 * ks + 8 * g) : zero8<f16>();
  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int n_blk = (n_valid + KB - 1) / KB;
  issue(0, 0);
  for (int b = 0; b < n_blk; ++b) {
    const int j0 = b * KB;
    __builtin_amdgcn_s_waitcnt(WAIT_ALL);
    __builtin_amdgcn_s_barrier();
    if (b + 1 < n_blk) issue(b + 1, (b + 1) & 1);
    // The block that holds the sequence's last key (the same block for the
    // whole workgroup; no loads are in flight after it): Vt entries past that
    // key hold whatever an earlier call left there. They are zeroed, so the
    // zero weights of those keys give zero products whatever the values were.
    const int nv = n_valid - j0;  // valid keys of this block (>= 64: all)
    if (nv < KB) {
      zero_vt_tail(lds + (b & 1) * STAGE + K_STAGE, nv, tid, blockDim.x);
      __builtin_amdgcn_s_waitcnt(WAIT_ALL);
      __builtin_amdgcn_s_barrier();
    }
    if (!active) continue;
    const char *ks_lds = lds + (b & 1) * STAGE;
    const char *vs = ks_lds + K_STAGE;

    // S^T = K Q^T: key block kb, output row l32 takes key row kr = 32 kb +
    // sw23(l32), d chunk 2 ks + g, stored at chunk (2 ks + g) ^ (l32 & 15).
    // The K fragments of step ks+1 are read while step ks's MFMAs run.
    f32x16 sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.f;
    f16x8 kf[2][2];
    auto read_k = [&](int ks, int slot) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int kr = 32 * kb + sw23(l32);
        kf[slot][kb] = load8(reinterpret_cast<const f16 *>(ks_lds + kr * K_ROW + (((2 * ks + g) ^ (l32 & 15)) * 16)));
      }
    };
    read_k(0, 0);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks < 7) read_k(ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sacc[kb] = mfma32(kf[ks & 1][kb], qf[ks], sacc[kb]);
    }
    // masks: 0x100 LDS read, 0x008 MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
    for (int ks = 0; ks < 7; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);

    // sacc[kb][8 h + e]: raw score of key j0 + 32 kb + 16 h + 8 g + e. Keys
    // past the sequence (only in its last block) get -inf.
    if (j0 + KB > n_valid) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (j0 + 32 * kb + 16 * h + 8 * g + e >= n_valid) sacc[kb][8 * h + e] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE)) * scale_log2;  // the scale is positive: it keeps the order
    // The reference maximum m_run moves only when a query's block maximum
    // exceeds it by more than 8 (in log2 units), so most blocks skip the
    // rescale of O and l (decided for the whole wavefront). A reference up to
    // 8 below the true maximum leaves the weights exp2(s - m_run) at most
    // 256: within fp16, with the same relative rounding as weights <= 1.
    if (__builtin_amdgcn_ballot_w64(mx > m_run + 8.f)) {
      const float m_new = fmaxf(m_run, mx);
      // exponents are <= 0 or -inf: the bare exp2 instruction is exact
      // enough and maps -inf to 0
      const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= corr;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] *= corr;
    }
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], scale_log2, -m_run));
        psum += sacc[kb][r];
      }
    l_run += psum;

    // O^T += Vt P^T. Step j = 2 kb + h covers keys 16 j + 8 g + 0..7: the
    // lane's own scores sacc[kb][8 h + 0..7], and logical chunk 2 j + g of
    // Vt row d = 32 db + l32 (zero past the sequence's last key). The loop
    // has no branch, so each Vt read stays in flight for one MFMA.
    f16x8 pf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[j][e] = (f16)sacc[j >> 1][8 * (j & 1) + e];
    f16x8 vf[2];
    auto read_v = [&](int step, int slot) {
      const int j = step >> 2, d = 32 * (step & 3) + l32;
      vf[slot] = *reinterpret_cast<const f16x8 *>(vs + d * V_ROW + (((2 * j + g) ^ swz8(d)) * 16));
    };
    read_v(0, 0);
#pragma unroll
    for (int step = 0; step < 16; ++step) {
      if (step < 15) read_v(step + 1, (step + 1) & 1);
      o[step & 3] = mfma32(vf[step & 1], pf[step >> 2], o[step & 3]);
    }
  }

  // Output: O^T lane layout (query l32, d = 32 db + 8 qq + 4 g + r) -> LDS
  // rows [query][d] -> 16-byte chunks of whole rows.
  float l_tot = l_run + __shfl_xor(l_run, 32, WAVE);
  const float inv = active ? 1.f / l_tot : 0.f;
  __builtin_amdgcn_s_waitcnt(WAIT_ALL);
  __builtin_amdgcn_s_barrier();
  char *ow = lds + wave * ATT_QW * O_PITCH;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      *reinterpret_cast<f16x4 *>(ow + l32 * O_PITCH + (32 * db + 8 * qq + 4 * g) * 2) =
          f16x4{(f16)(o[db][4 * qq] * inv), (f16)(o[db][4 * qq + 1] * inv), (f16)(o[db][4 * qq + 2] * inv),
                (f16)(o[db][4 * qq + 3] * inv)};
#pragma unroll
  for (int r0 = 0; r0 < ATT_QW; r0 += 4) {
    const int ql = r0 + (lane >> 4), qq = q_base + ql, c = lane & 15;
    const f16x8 v = *reinterpret_cast<const f16x8 *>(ow + ql * O_PITCH + c * 16);
    if (qq < n_valid && qq < (chunk + 1) * q_chunk)
      *reinterpret_cast<f16x8 *>(out + ((size_t)t0 + qq) * D_MODEL + head * D_HEAD + 8 * c) = v;
  }
}

// fp16 kernel for small grids (fewer workgroups of 128-query chunks than
// CUs: 1 to 8 sequences). One workgroup per (sequence p, head, chunk of up to 256
// queries): NW wavefronts of 16 queries each, so K and V of the sequence are
// read once per head instead of once per query tile. Key blocks of 64 are
// loaded straight into LDS (buffer_load ... lds, 16 bytes per lane) in two
// stages: the loads of block b+1 are issued when block b starts, so they land
// during block b's MFMA work. K rows (256 bytes) are stored with 16-byte chunk
// c at c ^ (row & 15) and Vt rows (64 keys, 128 bytes) with chunk c at
// c ^ (d & 7), so the fragment reads of 16 consecutive rows spread over the
// banks. The math per wavefront is the fp32 kernel's at the top of this file
// (S^T = K Q^T, here with the 16x16x32 MFMA, online softmax per lane, O^T +=
// Vt P^T). The output goes
// through LDS so that each store writes whole 256-byte rows of the head's
// slice. Wavefronts whose queries are all padding skip the math (they still
// issue loads and meet the barriers) and write zeros. Workgroups are mapped
// so that XCD x serves head x: blockIdx.x % 8 is the head.
constexpr int Q16_MAX_WAVES = 16, Q16_QW = 16;  // wavefronts per workgroup, queries per wavefront
// Smallest query chunk worth splitting for when there are few sequences (3
// wavefronts): the grid grows while it is under one workgroup per CU. 1 clip
// (2 x 152 tokens) takes 4 chunks of 48 (1.98 ms per step against 2.00 with
// chunks of 32 and 2.05 with one chunk); 8 sequences of 92 tokens take 2
// chunks of 48 (2.143 ms per pass against 2.157 with one). Each chunk walks
// all the keys on its own (K and V come from L2).
constexpr int Q16_MIN_CHUNK_Q = 48;
// At most this many queries per workgroup (8 wavefronts) before the split.
constexpr int Q16_CHUNK_Q = 128;

__global__ __launch_bounds__(64 * Q16_MAX_WAVES) void attention_f16_q16_kernel(
    const f16 *__restrict__ qkv, const f16 *__restrict__ vt, f16 *__restrict__ out,
    const int32_t *__restrict__ tok, const int32_t *__restrict__ mot, int P, int S, int S_pad, int n_chunks,
    int q_chunk, float scale_log2) {
  constexpr int K_ROW = D_HEAD * 2;          // 256 bytes per key row
  constexpr int V_ROW = KB * 2;              // 128 bytes per d row of a 64-key block
  constexpr int K_STAGE = KB * K_ROW;        // 16 KB
  constexpr int STAGE = K_STAGE + D_HEAD * V_ROW;  // + 16 KB
  constexpr int O_PITCH = D_HEAD * 2 + 16;   // staged output row
  constexpr int LDS = 2 * STAGE > Q16_MAX_WAVES * Q16_QW * O_PITCH ? 2 * STAGE : Q16_MAX_WAVES * Q16_QW * O_PITCH;
  __shared__ __attribute__((aligned(1024))) char lds[LDS];

  const int head = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int p = slot / n_chunks, chunk = slot - p * n_chunks;
  if (p >= P) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), NW = blockDim.x / 64;
  const int l16 = lane & 15, g = lane >> 4;
  const int t0 = tok[p], n_valid = mot[p + 1] - mot[p] + 2;  // sequence p's tokens, from packed row t0
  const int q_base = chunk * q_chunk + wave * Q16_QW;
  const bool active = q_base < n_valid;

  // Buffer resources: the sequence's K columns of this head (rows past S read
  // as zero) and its Vt block [128][S_pad].
  const __amdgpu_buffer_rsrc_t k_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(qkv + (size_t)t0 * QKV_LD + D_MODEL + head * D_HEAD), (short)0, n_valid * QKV_LD * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t v_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(vt + ((size_t)p * 8 + head) * D_HEAD * S_pad), (short)0, D_HEAD * S_pad * 2, 0x00020000);
  // Load instruction i < 16: K rows 4i .. 4i+3 of the block; i >= 16: Vt rows
  // d = 8(i-16) .. +7. Lane l writes LDS byte 16 l of the instruction's 1 KB.
  const int k_row = lane >> 4, k_chunk = lane & 15;  // swizzled with the row below
  auto issue = [&](int blk, int stage) {
    char *base = lds + stage * STAGE;
    for (int i = wave; i < 32; i += NW) {
      if (i < 16) {
        const int r = 4 * i + k_row;
        const int voff = (KB * blk + r) * QKV_LD * 2 + ((k_chunk ^ (r & 15)) * 16);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(k_rsrc, (__attribute__((address_space(3))) void *)(base + i * 1024),
                                                 16, voff, 0, 0, 0);
      } else {
        const int d = 8 * (i - 16) + (lane >> 3);
        const int voff = d * S_pad * 2 + (KB * blk + 8 * ((lane & 7) ^ (d & 7))) * 2;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            v_rsrc, (__attribute__((address_space(3))) void *)(base + K_STAGE + (i - 16) * 1024), 16, voff, 0, 0, 0);
      }
    }
  };

  const int q = q_base + l16;
  const bool q_ok = active && q < n_valid;
  f16x8 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    qf[kk] = q_ok ? load8(qkv + ((size_t)t0 + q) * QKV_LD + head * D_HEAD + 32 * kk + 8 * g) : zero8<f16>();
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  const int n_blk = (n_valid + KB - 1) / KB;
  issue(0, 0);
  for (int b = 0; b < n_blk; ++b) {
    const int j0 = b * KB;
    __builtin_amdgcn_s_waitcnt(WAIT_ALL);
    __builtin_amdgcn_s_barrier();
    if (b + 1 < n_blk) issue(b + 1, (b + 1) & 1);
    if (!active) continue;
    const char *ks = lds + (b & 1) * STAGE;
    const char *vs = ks + K_STAGE;

    // S^T = K Q^T over 4 key sub-blocks of 16 with independent accumulators,
    // k-outer so that consecutive MFMAs do not depend on each other; the K
    // fragments of step kk+1 are read while step kk's MFMAs run. Row r =
    // 16 sb + l16 has r & 15 = l16.
    f32x4 sacc[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) sacc[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
    f16x8 kf[2][4];
    auto read_k = [&](int kk, int slot) {
#pragma unroll
      for (int sb = 0; sb < 4; ++sb)
        kf[slot][sb] = load8(reinterpret_cast<const f16 *>(ks + (16 * sb + l16) * K_ROW + (((4 * kk + g) ^ l16) * 16)));
    };
    read_k(0, 0);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk < 3) read_k(kk + 1, (kk + 1) & 1);
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) sacc[sb] = mfma8(kf[kk & 1][sb], qf[kk], sacc[sb]);
    }
    // masks: 0x100 LDS read, 0x008 MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int kk = 0; kk < 3; ++kk)
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);

    float s[4][4];
    float mx = -INFINITY;
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int key = j0 + 16 * sb + 4 * g + r4;
        s[sb][r4] = key < n_valid ? sacc[sb][r4] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[sb][r4]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, WAVE));
    mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
    const float m_new = fmaxf(m_run, mx);
    // exponents are <= 0 or -inf: the bare exp2 instruction is exact enough
    // and maps -inf to 0
    const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int sb = 0; sb < 4; ++sb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        s[sb][r4] = __builtin_amdgcn_exp2f(s[sb][r4] - m_new);
        psum += s[sb][r4];
      }
    l_run = l_run * corr + psum;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] *= corr;

    // O^T += Vt P^T. k-slots of half hf for group g: keys 32 hf + {4g .. 4g+3,
    // 16+4g .. 16+4g+3}, i.e. 8-byte halves of logical Vt chunks 4hf + g/2 and
    // 4hf + 2 + g/2. The 16 (hf, db) steps read their V fragment one step ahead.
    f16x8 pf[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        pf[hf][r4] = (f16)s[2 * hf][r4];
        pf[hf][4 + r4] = (f16)s[2 * hf + 1][r4];
      }
    // In the block that holds the sequence's last key, Vt positions past it
    // hold whatever an earlier call left there: their fragment entries are
    // replaced by exact zeros, so that the zero weights of those keys give
    // zero products whatever the values are.
    const int nv = n_valid - j0;  // valid keys of this block (>= 64: all)
    f16x8 vf[2];
    auto read_v = [&](int step, int slot) {
      const int hf = step >> 3, db = step & 7;
      const int c_lo = 4 * hf + (g >> 1), half = (g & 1) * 8, d = 16 * db + l16;
      const char *vrow = vs + d * V_ROW;
      const f16x4 lo = *reinterpret_cast<const f16x4 *>(vrow + ((c_lo ^ (d & 7)) * 16) + half);
      const f16x4 hi = *reinterpret_cast<const f16x4 *>(vrow + (((c_lo + 2) ^ (d & 7)) * 16) + half);
      f16x8 v = f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      if (nv < KB) {
        const int k_lo = 32 * hf + 4 * g;  // keys k_lo .. k_lo + 3 and k_lo + 16 .. k_lo + 19
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = k_lo + e < nv ? v[e] : (f16)0.f;
          v[4 + e] = k_lo + 16 + e < nv ? v[4 + e] : (f16)0.f;
        }
      }
      vf[slot] = v;
    };
    read_v(0, 0);
#pragma unroll
    for (int step = 0; step < 16; ++step) {
      if (step < 15) read_v(step + 1, (step + 1) & 1);
      o[step & 7] = mfma8(vf[step & 1], pf[step >> 3], o[step & 7]);
    }
  }

  // Output: O^T lane layout (query l16, d = 16 db + 4 g + r) -> LDS rows
  // [query][d] -> 16-byte chunks of whole rows.
  float l_tot = l_run + __shfl_xor(l_run, 16, WAVE);
  l_tot += __shfl_xor(l_tot, 32, WAVE);
  const float inv = active ? 1.f / l_tot : 0.f;
  __builtin_amdgcn_s_waitcnt(WAIT_ALL);
  __builtin_amdgcn_s_barrier();
  char *ow = lds + wave * Q16_QW * O_PITCH;
#pragma unroll
  for (int db = 0; db < 8; ++db)
    *reinterpret_cast<f16x4 *>(ow + l16 * O_PITCH + (16 * db + 4 * g) * 2) =
        f16x4{(f16)(o[db][0] * inv), (f16)(o[db][1] * inv), (f16)(o[db][2] * inv), (f16)(o[db][3] * inv)};
#pragma unroll
  for (int r0 = 0; r0 < Q16_QW; r0 += 4) {
    const int ql = r0 + (lane >> 4), qq = q_base + ql, c = lane & 15;
    const f16x8 v = *reinterpret_cast<const f16x8 *>(ow + ql * O_PITCH + c * 16);
    if (qq < n_valid && qq < (chunk + 1) * q_chunk)
      *reinterpret_cast<f16x8 *>(out + ((size_t)t0 + qq) * D_MODEL + head * D_HEAD + 8 * c) = v;
  }
}

}  // namespace

template <typename T>
hipError_t attention(const T *qkv, const T *vt, T *out, const int32_t *tok, const int32_t *mot, int P, int S,
                     int S_pad, hipStream_t stream) {
  if (P <= 0 || S <= 0) return hipSuccess;
  if (S_pad % KB != 0 || S_pad < S) return hipErrorInvalidValue;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)D_HEAD);
  if constexpr (sizeof(T) == 2) {
    // Fewer 128-query chunks than CUs (1 to 8 sequences): the 16-query
    // wavefronts of attention_f16_q16_kernel give the key loops twice the
    // wavefronts (1 clip: 11.1 -> 8.8 us per launch, 1.96 -> 1.90 ms per step;
    // 4 takes of 90 frames: 2.22 -> 2.17 ms per pass).
    if (8 * P * ((S + Q16_CHUNK_Q - 1) / Q16_CHUNK_Q) < 256) {
      int n_chunks = (S + Q16_CHUNK_Q - 1) / Q16_CHUNK_Q;
      auto chunk_q = [&](int n) { return ((S + n - 1) / n + Q16_QW - 1) / Q16_QW * Q16_QW; };
      while (8 * P * n_chunks < 256 && chunk_q(n_chunks + 1) >= Q16_MIN_CHUNK_Q &&
             chunk_q(n_chunks + 1) < chunk_q(n_chunks))
        ++n_chunks;
      const int q_chunk = chunk_q(n_chunks);
      n_chunks = (S + q_chunk - 1) / q_chunk;  // no chunk wholly past S
      launch("attention", attention_f16_q16_kernel, dim3(8 * P * n_chunks), dim3(64 * (q_chunk / Q16_QW)), stream,
             qkv, vt, out, tok, mot, P, S, S_pad, n_chunks, q_chunk, scale_log2);
      return hipGetLastError();
    }
    // the fewest chunks of at most ATT_CHUNK_Q queries, balanced in whole
    // wavefronts (182 tokens: one chunk of 192; 302 tokens: one chunk of 320;
    // 702 tokens: 2 chunks of 352)
    int n_chunks = (S + ATT_CHUNK_Q - 1) / ATT_CHUNK_Q;
    const int q_chunk = ((S + n_chunks - 1) / n_chunks + ATT_QW - 1) / ATT_QW * ATT_QW;
    n_chunks = (S + q_chunk - 1) / q_chunk;  // no chunk wholly past S
    dim3 grid(8 * P * n_chunks);
    launch("attention", attention_f16_kernel, grid, dim3(64 * (q_chunk / ATT_QW)), stream, qkv, vt, out, tok, mot, P,
           S, S_pad, n_chunks, q_chunk, scale_log2);
  } else {
    dim3 grid((S + QT - 1) / QT, D_MODEL / D_HEAD, P);
    launch("attention", attention_kernel<T>, grid, dim3(256), stream, qkv, vt, out, tok, mot, S, S_pad,
           scale_log2);
  }
  return hipGetLastError();
}

template hipError_t attention<f16>(const f16 *, const f16 *, f16 *, const int32_t *, const int32_t *, int, int, int,
                                   hipStream_t);
template hipError_t attention<float>(const float *, const float *, float *, const int32_t *, const int32_t *, int,
                                     int, int, hipStream_t);

}  // namespace kmd
