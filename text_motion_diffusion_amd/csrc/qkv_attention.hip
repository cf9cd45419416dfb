// Fused QKV projection + masked self-attention of one head of one sequence,
// for sequences of up to 160 tokens (fp16). The projection is the Linear of
// the encoder layer's self-attention with a fused [Wq; Wk; Wv] weight (Kimodo
// WebGPU README, "WGSL compute shaders" table, linear.wgsl and qkv_split.wgsl
// rows); the attention is its multi-head self-attention with
// key masking (same table, attention.wgsl row). Fusing them keeps Q, K and V of
// the head in LDS: they never go to HBM.
//
// One workgroup of 12 wavefronts per (sequence p, head); each XCD serves two
// heads of the sequences of one parity, so its L2 holds two heads' weight
// slices and half of the token rows.
//   1. Projection: the sequence's packed token rows (up to 160; rows past
//      its tokens read as zero) times the head's 384 weight rows (Q, K, V
//      blocks of 128). The main loop is the one of the projection GEMMs:
//      64-deep k-tiles in two LDS stages loaded straight into LDS, swz8 chunk
//      swizzle, 32x32x16 MFMAs; wavefront w owns columns 32w .. 32w+31 (160 x
//      32, 5 blocks). The V wavefronts (8..11) issue the MFMAs with swapped
//      operands, so their lanes hold the transposed layout of step 2.
//   2. Bias, fp16, and into LDS: Q and K as [160][128] rows of 256 bytes with
//      16-byte chunk c at c ^ (row & 15); V transposed as three blocks of
//      [128 d][64 keys] with chunk c at c ^ (d & 7) (keys past 160 zero),
//      4 consecutive keys per 8-byte store.
//   3. Attention: wavefronts 0..9 take 16 queries each, S^T = K Q^T with
//      16x16x32 MFMAs, online softmax per lane in fp32 (exp2 with the scale
//      folded into one FMA; the reference maximum moves only when a block's
//      maximum exceeds it by more than 8, so most blocks skip the rescale),
//      O^T += Vt P^T; keys >= length + 2 get -inf.
//   4. O / l through LDS, stored as whole 256-byte rows of the head's slice.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace kmd {
namespace {

constexpr int D = 1024, DH = 128, QKV_N = 3 * D;
constexpr int MAX_MB = 5;                         // row blocks of 32: up to 160 token rows
constexpr int COLS = 3 * DH;                      // the head's Q, K, V weight rows
constexpr int NW = 12;                            // wavefronts
constexpr int KTB = 128;                          // bytes of one 64-deep k-tile row
constexpr int V_BLK = DH * 128;                   // one [128][64] Vt block
constexpr int O_PITCH = DH * 2 + 16;
constexpr int QW = 16;                            // queries per attention wavefront

// MB row blocks of 32 token rows: the launch's longest sequence rounded up, so
// short sequences skip the projection of rows they do not have. The values
// in the comments are those of MB = 5.
template <int MB>
__global__ __launch_bounds__(64 * NW) void qkv_attention_kernel(const f16 *__restrict__ h, const f16 *__restrict__ wqkv,
                                                                const float *__restrict__ bqkv, f16 *__restrict__ out,
                                                                const int32_t *__restrict__ tok,
                                                                const int32_t *__restrict__ mot, int P, int S,
                                                                float scale_log2) {
  constexpr int ROWS = 32 * MB;                     // token rows per workgroup
  constexpr int STAGE = (ROWS + COLS) * KTB;        // 69632
  constexpr int NI = (ROWS + COLS) / 8;             // 68 load instructions per k-tile
  constexpr int LW = (NI + NW - 1) / NW;            // 6 per wavefront
  constexpr int NVB = (ROWS + 63) / 64;             // 3 Vt blocks of 64 keys
  // K rows past ROWS (keys of the last block that masking drops) read into the
  // V region; only V's keys past ROWS must be zeroed
  constexpr int Q_OFF = 0, K_OFF = ROWS * 256, V_OFF = 2 * ROWS * 256;
  constexpr int ATT_BYTES = V_OFF + NVB * V_BLK;    // 131072
  constexpr int MAIN = 2 * STAGE > ATT_BYTES ? 2 * STAGE : ATT_BYTES;
  static_assert(MB >= 1 && MB <= MAX_MB, "1 to 5 row blocks");
  static_assert(ROWS / QW * QW * O_PITCH <= MAIN, "output staging fits");
  __shared__ __attribute__((aligned(1024))) char lds[MAIN + COLS * 4];
  float *bias_l = reinterpret_cast<float *>(lds + MAIN);
  // XCD x = blockIdx % 8 serves heads 2 (x & 3) and 2 (x & 3) + 1 of the
  // sequences of parity x >> 2: its L2 holds two heads' weights and half of
  // the token rows instead of one head's and all of them.
  const int xcd = blockIdx.x % 8, j = blockIdx.x / 8;
  const int head = 2 * (xcd & 3) + (j & 1), p = (xcd >> 2) + 2 * (j >> 1);
  if (p >= P) return;  // an odd P leaves one slot per XCD of one parity empty
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int t0 = tok[p], n_valid = mot[p + 1] - mot[p] + 2;  // sequence p's tokens, from packed row t0
  for (int c = tid; c < COLS; c += 64 * NW) bias_l[c] = bqkv[(c / DH) * D + head * DH + c % DH];

  // ---- 1. projection ------------------------------------------------------
  // Tile row 8i + lane/8 of load instruction i: token row (i < 20) or weight
  // row (c / 128) * 1024 + head * 128 + c % 128 for c = 8i - 160 + lane/8.
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)(h + (size_t)t0 * D), (short)0, n_valid * D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t w_rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void *)wqkv, (short)0, QKV_N * D * 2, 0x00020000);
  const int lr = lane >> 3;
  const int c0 = ((lane & 7) ^ swz8(8 * (wave & 1) + lr)) * 16;
  auto issue = [&](int kt, int stage) {
#pragma unroll
    for (int j = 0; j < LW; ++j) {
      const int i = j * NW + wave < NI ? j * NW + wave : NI - 1 - ((NI - 1 - wave) & 1);
      auto *dst = (__attribute__((address_space(3))) void *)(lds + stage * STAGE + i * 1024);
      const int r8 = 8 * i;
      const bool is_a = r8 < ROWS;
      const int wr = r8 - ROWS;
      const int grow = (wr >> 7) * D + head * DH + (wr & (DH - 1));
      __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? a_rsrc : w_rsrc, dst, 16,
                                               is_a ? (r8 + lr) * D * 2 + c0 : (grow + lr) * D * 2 + c0,
                                               kt * KTB, 0, 0);
    }
  };

  f32x16 acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  const int sw = swz8(l32 & 15);
  const int a_row = l32 * KTB, w_row = (ROWS + 32 * wave + l32) * KTB;
  f16x8 af[2][MB], wf[2];
  auto read_frags = [&](int stage, int ks, int slot) {
    const char *base = lds + stage * STAGE;
    const int chunk = ((2 * ks + g) ^ sw) * 16;
#pragma unroll
    for (int i = 0; i < MB; ++i) af[slot][i] = load8(reinterpret_cast<const f16 *>(base + a_row + i * 32 * KTB + chunk));
    wf[slot] = load8(reinterpret_cast<const f16 *>(base + w_row + chunk));
  };
  const int nk = D / 64;
  issue(0, 0);
  // The V wavefronts (8..11) multiply with the operands swapped, A W^T
  // instead of W A^T: each lane then ends with 4 consecutive tokens of one
  // head-dim column, the layout of the transposed V block in LDS (one 8-byte
  // store per 4 tokens instead of 4 2-byte ones). Two copies of the loop,
  // chosen once per wavefront.
  auto main_loop = [&](auto swap) {
  for (int kt = 0; kt < nk; ++kt) {
    const int s = kt & 1;
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __builtin_amdgcn_s_barrier();
    issue(min(kt + 1, nk - 1), s ^ 1);
    read_frags(s, 0, 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3) read_frags(s, ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int i = 0; i < MB; ++i)
        acc[i] = decltype(swap)::value ? mfma32(af[ks & 1][i], wf[ks & 1], acc[i])
                                       : mfma32(wf[ks & 1], af[ks & 1][i], acc[i]);
    }
    // masks: 0x010 VMEM, 0x100 LDS read, 0x008 MFMA
    __builtin_amdgcn_sched_group_barrier(0x010, LW, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, MB + 1, 0);
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
      for (int i = 1; i < MB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, MB, 0);
  }
  };
  if (wave >= 8)
    main_loop(std::true_type{});
  else
    main_loop(std::false_type{});
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  __builtin_amdgcn_s_barrier();

  // ---- 2. Q, K, Vt into LDS ------------------------------------------------
  {
    const int blk = wave >> 2, cb = 32 * (wave & 3);
    if (blk < 2) {
      // Q, K: acc[i][4 q + r] is token m = 32 i + l32, head-dim column
      // cb + 8 q + 4 g + r
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int m = 32 * i + l32;
        char *row = lds + (blk == 0 ? Q_OFF : K_OFF) + m * 256;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int d0 = cb + 8 * q + 4 * g;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[i][4 * q + r] + bias_l[blk * DH + d0 + r];
          *reinterpret_cast<f16x4 *>(row + ((((cb >> 3) + q) ^ (m & 15)) * 16) + 8 * g) =
              f16x4{(f16)v[0], (f16)v[1], (f16)v[2], (f16)v[3]};
        }
      }
    } else {
      // V (operands swapped): acc[i][4 q + r] is token 32 i + 8 q + 4 g + r,
      // head-dim column d = cb + l32; the 4 tokens share one 16-byte chunk of
      // the Vt row (they start on a multiple of 4)
      const int d = cb + l32;
      const float b = bias_l[2 * DH + d];
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = 32 * i + 8 * q + 4 * g, kb = m >> 6, k = m & 63;
          *reinterpret_cast<f16x4 *>(lds + V_OFF + kb * V_BLK + d * 128 + (((k >> 3) ^ (d & 7)) * 16) + (k & 7) * 2) =
              f16x4{(f16)(acc[i][4 * q] + b), (f16)(acc[i][4 * q + 1] + b), (f16)(acc[i][4 * q + 2] + b),
                    (f16)(acc[i][4 * q + 3] + b)};
        }
    }
    // keys ROWS .. 64 NVB - 1 of the last Vt block (160 .. 191): zeros (their
    // probabilities are 0, the values must be finite)
    if constexpr (ROWS % 64 != 0) {
      for (int e = tid; e < DH * 4; e += 64 * NW) {
        const int d = e >> 2, k = 32 + 8 * (e & 3);
        *reinterpret_cast<uint4 *>(lds + V_OFF + (NVB - 1) * V_BLK + d * 128 + (((k >> 3) ^ (d & 7)) * 16)) =
            make_uint4(0, 0, 0, 0);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  __builtin_amdgcn_s_barrier();

  // ---- 3. attention ------------------------------------------------------
  const int l16 = lane & 15, g4 = lane >> 4;
  const int q_base = wave * QW;
  const bool active = wave < ROWS / QW && q_base < n_valid;
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  if (active) {
    const int q = q_base + l16;
    f16x8 qf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      qf[kk] = load8(reinterpret_cast<const f16 *>(lds + Q_OFF + q * 256 + (((4 * kk + g4) ^ (q & 15)) * 16)));
    const int n_blk = (n_valid + 63) / 64;
    for (int b = 0; b < n_blk; ++b) {
      const int j0 = 64 * b;
      const char *ks = lds + K_OFF + j0 * 256;
      const char *vs = lds + V_OFF + b * V_BLK;
      f32x4 sacc[4];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb) sacc[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
      f16x8 kf[2][4];
      auto read_k = [&](int kk, int slot) {
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
          kf[slot][sb] = load8(reinterpret_cast<const f16 *>(ks + (16 * sb + l16) * 256 + (((4 * kk + g4) ^ l16) * 16)));
      };
      read_k(0, 0);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (kk < 3) read_k(kk + 1, (kk + 1) & 1);
#pragma unroll
        for (int sb = 0; sb < 4; ++sb) sacc[sb] = mfma8(kf[kk & 1][sb], qf[kk], sacc[sb]);
      }
      // raw scores; keys past the sequence (only in its last block) get -inf
      float sc[4][4];
#pragma unroll
      for (int sb = 0; sb < 4; ++sb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) sc[sb][r4] = sacc[sb][r4];
      if (j0 + 64 > n_valid) {
#pragma unroll
        for (int sb = 0; sb < 4; ++sb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
            if (j0 + 16 * sb + 4 * g4 + r4 >= n_valid) sc[sb][r4] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int sb = 0; sb < 4; ++sb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) mx = fmaxf(mx, sc[sb][r4]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, WAVE));
      mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE)) * scale_log2;  // a positive scale keeps the order
      // The reference maximum moves only when a query's block maximum exceeds
      // it by more than 8 (log2 units), decided for the whole wavefront: the
      // weights exp2(s - m_run) then stay <= 256 (fp16-safe, same relative
      // rounding), and most blocks skip the rescale of O and l.
      if (__builtin_amdgcn_ballot_w64(mx > m_run + 8.f)) {
        const float m_new = fmaxf(m_run, mx);
        const float corr = __builtin_amdgcn_exp2f(m_run - m_new);  // arguments <= 0 or -inf
        m_run = m_new;
        l_run *= corr;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] *= corr;
      }
      float psum = 0.f;
#pragma unroll
      for (int sb = 0; sb < 4; ++sb)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          sc[sb][r4] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[sb][r4], scale_log2, -m_run));
          psum += sc[sb][r4];
        }
      l_run += psum;
      // k-slots of half hf for group g4: keys 32 hf + {4 g4 .. +3, 16 + 4 g4 .. +3}
      f16x8 pf[2];
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          pf[hf][r4] = (f16)sc[2 * hf][r4];
          pf[hf][4 + r4] = (f16)sc[2 * hf + 1][r4];
        }
      f16x8 vf[2];
      auto read_v = [&](int step, int slot) {
        const int hf = step >> 3, db = step & 7;
        const int c_lo = 4 * hf + (g4 >> 1), half = (g4 & 1) * 8, d = 16 * db + l16;
        const char *vrow = vs + d * 128;
        const f16x4 lo = *reinterpret_cast<const f16x4 *>(vrow + ((c_lo ^ (d & 7)) * 16) + half);
        const f16x4 hi = *reinterpret_cast<const f16x4 *>(vrow + (((c_lo + 2) ^ (d & 7)) * 16) + half);
        vf[slot] = f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      };
      read_v(0, 0);
#pragma unroll
      for (int step = 0; step < 16; ++step) {
        if (step < 15) read_v(step + 1, (step + 1) & 1);
        o[step & 7] = mfma8(vf[step & 1], pf[step >> 3], o[step & 7]);
      }
    }
  }
  float l_tot = l_run + __shfl_xor(l_run, 16, WAVE);
  l_tot += __shfl_xor(l_tot, 32, WAVE);
  const float inv = active ? 1.f / l_tot : 0.f;
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  __builtin_amdgcn_s_barrier();

  // ---- 4. output ----------------------------------------------------------
  if (wave < ROWS / QW) {
    char *ow = lds + wave * QW * O_PITCH;
#pragma unroll
    for (int db = 0; db < 8; ++db)
      *reinterpret_cast<f16x4 *>(ow + l16 * O_PITCH + (16 * db + 4 * g4) * 2) =
          f16x4{(f16)(o[db][0] * inv), (f16)(o[db][1] * inv), (f16)(o[db][2] * inv), (f16)(o[db][3] * inv)};
#pragma unroll
    for (int r0 = 0; r0 < QW; r0 += 4) {
      const int ql = r0 + (lane >> 4), qq = q_base + ql, c = lane & 15;
      const f16x8 v = *reinterpret_cast<const f16x8 *>(ow + ql * O_PITCH + c * 16);
      if (qq < n_valid) *reinterpret_cast<f16x8 *>(out + ((size_t)t0 + qq) * D + head * DH + 8 * c) = v;
    }
  }
}

}  // namespace

hipError_t qkv_attention(const f16 *h, const f16 *wqkv, const float *bqkv, f16 *out, const int32_t *tok,
                         const int32_t *mot, int P, int S, hipStream_t stream) {
  if (P <= 0 || S <= 0) return hipSuccess;
  if (S > 32 * MAX_MB) return hipErrorInvalidValue;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)DH);
  const dim3 grid(8 * ((P + 1) & ~1)), block(64 * NW);
  switch ((S + 31) / 32) {
    case 1: launch("qkv_attention", qkv_attention_kernel<1>, grid, block, stream, h, wqkv, bqkv, out, tok, mot, P, S,
                   scale_log2); break;
    case 2: launch("qkv_attention", qkv_attention_kernel<2>, grid, block, stream, h, wqkv, bqkv, out, tok, mot, P, S,
                   scale_log2); break;
    case 3: launch("qkv_attention", qkv_attention_kernel<3>, grid, block, stream, h, wqkv, bqkv, out, tok, mot, P, S,
                   scale_log2); break;
    case 4: launch("qkv_attention", qkv_attention_kernel<4>, grid, block, stream, h, wqkv, bqkv, out, tok, mot, P, S,
                   scale_log2); break;
    default: launch("qkv_attention", qkv_attention_kernel<5>, grid, block, stream, h, wqkv, bqkv, out, tok, mot, P, S,
                    scale_log2); break;
  }
  return hipGetLastError();
}

}  // namespace kmd
