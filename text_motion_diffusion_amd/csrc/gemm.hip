// Dense projection GEMMs of the denoiser (QKV, attention output, FFN, input and
// output heads, text and timestep MLPs): C = epi(A W^T + b) with W in the torch
// Linear layout [out, in] (Kimodo WebGPU README, "WGSL compute shaders" table,
// linear.wgsl row; its gelu.wgsl and silu.wgsl steps are folded into the epilogue).
//
// gfx950 design. A workgroup of WGM x WGN wavefronts (times KS k-groups)
// computes a BM x BN tile of C; each wavefront owns a (BM/WGM) x (BN/WGN)
// sub-tile held as 32x32 MFMA accumulator blocks in fp32. The MFMA is issued
// as D = W_tile * A_tile^T, so each lane ends with runs of 4 consecutive
// output columns of one row. K is consumed in k-tiles of 128 bytes per row
// (64 fp16 or 32 fp32 values), two LDS stages deep, so the loads of tile k+1
// are in flight while tile k is multiplied.
//
// fp16 path (gemm_tile_dma): operands go HBM -> LDS by direct buffer loads
// (16 bytes per lane, no register staging); LDS rows are 128 bytes with
// 16-byte chunks XOR-swizzled by swz8(row) so the fragment reads of 8
// consecutive rows hit disjoint banks. Rows past M or N lie outside the
// buffer resource's range and read as zero. Per 16-deep k-step the LDS
// fragment reads of the next k-step are issued before this k-step's MFMAs (a
// pinned schedule). With KS = 2 the two k-groups of wavefronts take the two
// halves of K and are summed through LDS before the epilogue. The epilogue
// adds the bias (preloaded into LDS), applies GELU/SiLU, and writes fp16 rows
// through LDS as 16-byte chunks; the QKV role writes its V third transposed
// into vt[p][head][d][s_pad], also staged through LDS. Tile shapes by M and
// role: 256x256 and 192x256 for large M and 192x256 for QKV below it, 160x128 (two workgroups
// per CU) for FFN1, and four-stage 160x128 or 128x128 tiles for the N = 1024
// products (OUT, FFN2).
//
// Split-K (fp16, few output tiles: 1 to 4 sequences): the k-tiles are divided
// among workgroups that write fp32 partial sums; a reduction kernel (or the
// LayerNorm that consumes the projection) adds them in split order, then the
// bias and the epilogue.
//
// fp32 path (gemm_tile): register-staged 128x128 tiles on the 32x32x2 fp32
// MFMA, rows padded by 16 bytes in LDS.
//
// Tile order is XCD-aware: workgroups are handed to the 8 XCDs round robin, so
// workgroup i is mapped to tile (i % 8) * ceil(tiles / 8) + i / 8; each XCD then
// works on a contiguous band of tiles (row-major, N fastest) that shares A rows
// and W panels in its own L2.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace kmd {
namespace {

// EPI_PARTIAL: split-K partial sums, fp32, no bias (the reduction adds it).
enum { EPI_BIAS = 0, EPI_BIAS_GELU = 1, EPI_BIAS_SILU = 2, EPI_QKV = 3, EPI_PARTIAL = 4 };
constexpr int ROW_BYTES = 128;
constexpr int PITCH = ROW_BYTES + 16;
constexpr int NUM_XCD = 8;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));


// Epilogue of one 32x32 accumulator block: lane holds column l32 of rows
// 8q + 4g + r (q, r = 0..3) of D = W_tile A_tile^T, i.e. output row m and the
// four output columns n .. n+3 for each q. EPI_QKV writes columns >= 2 * 1024
// (the V projection) transposed into vt[p][head][d][s_pad] (token (p, s) of row
// m from aux.pk.row_ps), where consecutive lanes hold consecutive tokens, so
// within a sequence each of the four stores is a contiguous 64-byte run.
template <int EPI, typename TO>
__device__ __forceinline__ void store_block(const f32x16 &acc, const float *__restrict__ bias, TO *__restrict__ C,
                                            int ldc, int m, int n_base, int M, int N, int vec_store,
                                            const GemmAux &aux) {
  if (m >= M) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int n = n_base + 8 * q;
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float x = acc[4 * q + r];
      if (EPI != EPI_PARTIAL && n + r < N) x += bias[n + r];
      if (EPI == EPI_BIAS_GELU) x = gelu_erf(x);
      if (EPI == EPI_BIAS_SILU) x = silu(x);
      v[r] = x;
    }
    if (EPI == EPI_QKV && n >= 2 * 1024) {
      const int ps = aux.pk.row_ps[m], p = ps >> 16, sq = ps & 0xffff, hd = n - 2 * 1024;
      TO *dst = static_cast<TO *>(aux.vt) + ((size_t)p * 1024 + hd) * aux.seq_pad + sq;
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(size_t)r * aux.seq_pad] = from_f32<TO>(v[r]);
      continue;
    }
    TO *dst = C + (size_t)m * ldc + n;
    if (vec_store && n + 3 < N) {
      if constexpr (sizeof(TO) == 4) {
        *reinterpret_cast<f32x4 *>(dst) = f32x4{v[0], v[1], v[2], v[3]};
      } else {
        *reinterpret_cast<f16x4 *>(dst) =
            f16x4{from_f32<TO>(v[0]), from_f32<TO>(v[1]), from_f32<TO>(v[2]), from_f32<TO>(v[3])};
      }
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < N) dst[r] = from_f32<TO>(v[r]);
    }
  }
}

// Coalesced fp16 epilogue of one wavefront's (32 MB) x (32 NB) sub-tile
// through its own LDS region: the accumulators (bias and activation applied)
// are written as fp16 rows, then read back as 16-byte chunks and stored so
// that each store instruction writes whole row segments of 32 NB * 2 bytes,
// instead of 16-byte pieces of 32 different rows. Needs N % 8 == 0, ldc % 8
// == 0 and a 16-byte aligned C. LDS operations of one wavefront complete in
// order, so the read-back sees the writes without a barrier.
template <int MB, int NB>
constexpr int epi_pitch() { return 64 * NB + 16; }  // bytes per staged row

// bias_l: the wavefront's WTN bias values in LDS (zero past N).
template <int EPI, int MB, int NB>
__device__ __forceinline__ void store_tile_lds(const f32x16 (&acc)[MB][NB], char *lds, const float *bias_l,
                                               f16 *__restrict__ C, int ldc, int m_base, int n_base, int M, int N) {
  constexpr int WTM = 32 * MB, WTN = 32 * NB, PITCH = epi_pitch<MB, NB>();
  const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nl = 32 * j + 8 * q + 4 * g;
      const float4 b4 = *reinterpret_cast<const float4 *>(bias_l + nl);
      const float b[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        f16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = acc[i][j][4 * q + r] + b[r];
          if (EPI == EPI_BIAS_GELU) x = gelu_erf(x);
          if (EPI == EPI_BIAS_SILU) x = silu(x);
          v[r] = (f16)x;
        }
        *reinterpret_cast<f16x4 *>(lds + (32 * i + l32) * PITCH + nl * 2) = v;
      }
    }
  constexpr int CPR = WTN / 8, RPI = 64 / CPR;  // 16-byte chunks per row, rows per instruction
  const int cr = lane / CPR, cc = lane % CPR;   // lanes past RPI rows (CPR not dividing 64) stay idle
#pragma unroll
  for (int r0 = 0; r0 < WTM; r0 += RPI) {
    const int rl = r0 + cr, m = m_base + rl, n = n_base + 8 * cc;
    if (cr < RPI && rl < WTM) {
      const f16x8 v = *reinterpret_cast<const f16x8 *>(lds + rl * PITCH + cc * 16);
      if (m < M && n < N) *reinterpret_cast<f16x8 *>(C + (size_t)m * ldc + n) = v;
    }
  }
}

// fp32 partial sums of a wavefront's sub-tile, staged the same way: rows of
// WTN floats at a pitch of WTN + 4 (16 rows written at one column offset hit
// 16 distinct 16-byte bank slots), stored back as whole row segments of
// WTN * 4 bytes, 16 bytes per lane. Needs N % 4 == 0 and 16-byte rows.
template <int MB, int NB>
constexpr int part_pitch() { return 128 * NB + 16; }  // bytes per staged row
template <int MB, int NB>
__device__ __forceinline__ void store_partial_lds(const f32x16 (&acc)[MB][NB], char *lds, float *__restrict__ P,
                                                  int ldp, int m_base, int n_base, int M, int N) {
  constexpr int WTM = 32 * MB, WTN = 32 * NB, PITCH = part_pitch<MB, NB>();
  const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int nl = 32 * j + 8 * q + 4 * g;
#pragma unroll
      for (int i = 0; i < MB; ++i)
        *reinterpret_cast<float4 *>(lds + (32 * i + l32) * PITCH + nl * 4) =
            float4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
    }
  constexpr int CPR = WTN / 4, RPI = 64 / CPR;  // 16-byte chunks per row, rows per instruction
  const int cr = lane / CPR, cc = lane % CPR;
#pragma unroll
  for (int r0 = 0; r0 < WTM; r0 += RPI) {
    const int rl = r0 + cr, m = m_base + rl, n = n_base + 4 * cc;
    if (rl < WTM) {
      const float4 v = *reinterpret_cast<const float4 *>(lds + rl * PITCH + cc * 16);
      if (m < M && n < N) *reinterpret_cast<float4 *>(P + (size_t)m * ldp + n) = v;
    }
  }
}

// The V part of the QKV projection, stored transposed into vt[p][hd][s_pad]
// through the wavefront's LDS region. Sequences start on multiples of 8 packed
// rows and sub-tiles on multiples of 32, so a sub-tile's 32 MB rows are 4 MB
// runs of 8 rows, each inside one sequence (its dead rows included). Lane k <
// 4 MB of each 16 reads 16 bytes of one staged head-dim row of run k and
// writes the run's 8 tokens with one store; head-dim rows are staged 64 (or
// 32) at a time. A run at or past row M (a multiple of 8) is not stored.
template <int MB>
constexpr int vt_pitch() { return 16 * 4 * MB + 16; }  // bytes per staged head-dim row

// The first token of run k = lane % 16 of a sub-tile, looked up before the
// main loop (clamped to a valid row, so the load needs no branch) and used
// only in the epilogue, so the loop hides its latency.
struct VtRun {
  int ps;     // (p << 16) | s of the run's first row
  bool live;  // the run exists and starts below M
};

template <int MB>
__device__ __forceinline__ VtRun plan_vt(int m_base, int M, const Packing &pk, bool staged) {
  const int k = threadIdx.x & 15, m = m_base + 8 * k;
  VtRun r;
  r.live = staged && k < 4 * MB && m < M;
  r.ps = pk.row_ps[min(m, M - 1)];
  return r;
}

template <int MB, int NB>
__device__ __forceinline__ void store_vt_lds(const f32x16 (&acc)[MB][NB], char *lds, const float *bias_l,
                                             f16 *__restrict__ vt, int m_base, int n_base, int M, const VtRun &run,
                                             int seq_pad) {
  constexpr int WTN = 32 * NB;
  constexpr int HR = WTN % 64 == 0 ? 64 : 32;  // head-dim rows per pass
  constexpr int PITCH = vt_pitch<MB>();
  static_assert(4 * MB <= 16, "at most 16 runs per row");
  if (m_base >= M) return;  // a sub-tile past the last row: nothing to store
  const int lane = threadIdx.x & 63, l32 = lane & 31, g = lane >> 5;
  const int k = lane & 15, rsub = lane >> 4;
  f16 *const vseq = vt + (size_t)(run.ps >> 16) * 1024 * seq_pad + (run.ps & 0xffff);
#pragma unroll
  for (int h0 = 0; h0 < WTN; h0 += HR) {
#pragma unroll
    for (int j = h0 / 32; j < (h0 + HR) / 32; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nl = 32 * j + 8 * q + 4 * g;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float b = bias_l[nl + r];
#pragma unroll
          for (int i = 0; i < MB; ++i)
            *reinterpret_cast<f16 *>(lds + (nl + r - h0) * PITCH + (32 * i + l32) * 2) =
                (f16)(acc[i][j][4 * q + r] + b);
        }
      }
#pragma unroll
    for (int r0 = 0; r0 < HR; r0 += 4) {
      const int hr = r0 + rsub, hd = n_base - 2 * 1024 + h0 + hr;
      if (run.live)
        *reinterpret_cast<f16x8 *>(vseq + (size_t)hd * seq_pad) =
            *reinterpret_cast<const f16x8 *>(lds + hr * PITCH + 16 * k);
    }
  }
}

template <typename T, int BM, int BN, int WGM, int WGN, int EPI, typename TO>
__device__ __forceinline__ void gemm_tile(const T *__restrict__ A, int lda, const T *__restrict__ W, int ldw,
                                          const float *__restrict__ bias, TO *__restrict__ C, int ldc, int M, int N,
                                          int K, int vec_store, const GemmAux &aux) {
  typedef typename Vec8<T>::type V8;
  constexpr int BK = ROW_BYTES / (int)sizeof(T);
  constexpr int FRAG = 8 * (int)sizeof(T);  // bytes of one 8-element fragment
  constexpr int KSTEPS = ROW_BYTES / (2 * FRAG);
  constexpr int FRAG_PER_MFMA = sizeof(T) == 2 ? 16 : 2;  // k per MFMA instruction
  constexpr int ROWS = BM + BN;
  constexpr int STAGE = ROWS * PITCH;
  constexpr int NT = 64 * WGM * WGN;                  // threads
  constexpr int WTM = BM / WGM, WTN = BN / WGN;       // wavefront tile
  constexpr int MB = WTM / 32, NB = WTN / 32;         // 32x32 blocks per wavefront
  constexpr int RPP = NT / 8;                         // tile rows loaded per pass
  static_assert(BM % RPP == 0 && BN % RPP == 0, "tile rows must be a multiple of the rows per pass");
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int wm = wave / WGN, wn = wave % WGN;

  // XCD-aware tile index, row-major over (M tiles, N tiles).
  const int n_tiles = (N + BN - 1) / BN, tiles = n_tiles * ((M + BM - 1) / BM);
  const int wg = blockIdx.x, per_xcd = (tiles + NUM_XCD - 1) / NUM_XCD;
  const int tile = (wg % NUM_XCD) * per_xcd + wg / NUM_XCD;
  if (tile >= tiles) return;
  const int m0 = (tile / n_tiles) * BM, n0 = (tile % n_tiles) * BN;

  // Global -> register staging: chunk j of thread t is tile row 32 j + t / 8,
  // 16-byte chunk t % 8; rows [0, BM) are A, rows [BM, BM + BN) are W. The
  // next k-tile is loaded at the top of an iteration and written to the other
  // LDS buffer at its end, so a whole k-tile of MFMA work hides the latency.
  // Loads go through buffer resources that end at the last valid row of the
  // tile: rows past M (or N) lie beyond the resource range and read as zero,
  // with no branch. The row offset is in the per-lane offset, which the range
  // check covers; the scalar offset only carries the k position in the row.
  const int ld_row = tid >> 3, ld_ch = tid & 7;
  const int a_valid = min(M - m0, BM), w_valid = min(N - n0, BN);
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(A + (size_t)m0 * lda), (short)0, a_valid * lda * (int)sizeof(T), 0x00020000);
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(W + (size_t)n0 * ldw), (short)0, w_valid * ldw * (int)sizeof(T), 0x00020000);
  const int a_off = ld_row * lda * (int)sizeof(T) + ld_ch * 16, a_step = RPP * lda * (int)sizeof(T);
  const int w_off = ld_row * ldw * (int)sizeof(T) + ld_ch * 16, w_step = RPP * ldw * (int)sizeof(T);
  u32x4 stage[(BM + BN) / RPP];
  auto gload = [&](int kt) {
#pragma unroll
    for (int j = 0; j < BM / RPP; ++j)
      stage[j] = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, a_off + j * a_step, kt * ROW_BYTES, 0);
#pragma unroll
    for (int j = 0; j < BN / RPP; ++j)
      stage[BM / RPP + j] = __builtin_amdgcn_raw_buffer_load_b128(w_rsrc, w_off + j * w_step, kt * ROW_BYTES, 0);
  };
  auto sstore = [&](int buf) {
    char *base = smem + buf * STAGE + ld_row * PITCH + ld_ch * 16;
#pragma unroll
    for (int j = 0; j < (BM + BN) / RPP; ++j) *reinterpret_cast<u32x4 *>(base + RPP * j * PITCH) = stage[j];
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // LDS fragments of k-step ks+1 are read while the MFMAs of k-step ks run.
  V8 af[2][MB], wf[2][NB];
  auto read_frags = [&](int buf, int ks, int slot) {
    const char *a_base = smem + buf * STAGE + (wm * WTM + l32) * PITCH + g * FRAG + ks * 2 * FRAG;
    const char *w_base = smem + buf * STAGE + (BM + wn * WTN + l32) * PITCH + g * FRAG + ks * 2 * FRAG;
#pragma unroll
    for (int i = 0; i < MB; ++i) af[slot][i] = load8(reinterpret_cast<const T *>(a_base + i * 32 * PITCH));
#pragma unroll
    for (int j = 0; j < NB; ++j) wf[slot][j] = load8(reinterpret_cast<const T *>(w_base + j * 32 * PITCH));
  };
  // The scheduling groups pin that order: per k-step, first the LDS reads of
  // the next k-step, then the MFMAs of this one (mask 0x100 = LDS reads,
  // 0x008 = MFMA), so LDS latency overlaps MFMA work.
  auto compute = [&](int buf) {
    read_frags(buf, 0, 0);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if (ks + 1 < KSTEPS) read_frags(buf, ks + 1, (ks + 1) & 1);
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[i][j] = mfma32(wf[ks & 1][j], af[ks & 1][i], acc[i][j]);
      if (ks + 1 < KSTEPS) __builtin_amdgcn_sched_group_barrier(0x100, MB + NB, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, MB * NB * (16 / FRAG_PER_MFMA), 0);
    }
  };

  const int nk = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) gload(kt + 1);
    compute(kt & 1);
    if (more) sstore((kt + 1) & 1);
    __syncthreads();
  }

  // Epilogue: block (i, j) is output row m0 + wm*WTM + 32i + l32, columns from
  // n0 + wn*WTN + 32j + 4g.
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
      store_block<EPI, TO>(acc[i][j], bias, C, ldc, m0 + wm * WTM + 32 * i + l32, n0 + wn * WTN + 32 * j + 4 * g, M, N,
                           vec_store, aux);
}

// fp16 main loop with direct-to-LDS loads. A k-tile is 64 deep (128 bytes per
// row); two LDS stages alternate, and the loads of k-tile kt+1 are issued at
// the top of iteration kt, so they have a whole k-tile of MFMA work to land.
// buffer_load ... lds writes each wavefront's 64 lanes x 16 bytes to 1 KB of
// consecutive LDS, i.e. 8 tile rows of 8 chunks; lane i fetches the logical
// chunk (i % 8) ^ swz8(row), so a row's chunks sit XOR-permuted in LDS and the
// fragment reads (one chunk of 16 consecutive rows per 16-lane group) hit
// disjoint banks: swz8(r) = ((r >> 1) ^ ((r & 1) << 2)) & 7 gives 8 distinct
// chunks for rows 0..7 (8-lane / 128-byte service groups) and for each parity
// class of rows 0..15 (16-lane / 256-byte groups). Each 32x32x16 MFMA takes a
// 16-byte fragment of A and of W; per 16-deep k-step the fragments of the
// next k-step are read interleaved with this k-step's MFMAs, pinned with
// scheduling group barriers (the default schedule serialises reads and MFMAs).
// The loop body has no branch (the last iterations re-load the last k-tile
// into a stage that is not read again), which keeps it one scheduling region.
// NST LDS stages keep NST - 1 k-tiles in flight.

template <int BM, int BN, int WGM, int WGN, int KS, int EPI, typename TO, int NST = 2>
__device__ __forceinline__ void gemm_tile_dma(const f16 *__restrict__ A, int lda, const f16 *__restrict__ W, int ldw,
                                              const float *__restrict__ bias, TO *__restrict__ C, int ldc, int M,
                                              int N, int K, int vec_store, const GemmAux &aux) {
  constexpr int NWM = WGM * WGN;                  // wavefronts per k-group (one output tile)
  constexpr int WTM = BM / WGM, WTN = BN / WGN;   // wavefront tile
  constexpr int MB = WTM / 32, NB = WTN / 32;     // 32x32 blocks per wavefront
  constexpr int KTB = 128;                        // bytes of one k-tile row: 64 fp16
  constexpr int STAGE_G = (BM + BN) * KTB;        // one k-group's k-tile
  constexpr int STAGE = KS * STAGE_G;
  constexpr int NI = (BM + BN) / 8;               // 1 KB load instructions per k-tile (8 rows each)
  constexpr int LW = (NI + NWM - 1) / NWM;        // per wavefront
  static_assert(NWM % 2 == 0 && BM % 16 == 0 && BN % 8 == 0 && MB >= 1 && NB >= 1 && (KS == 1 || KS == 2),
                "even wavefront count (one row parity per wavefront), 16-row aligned A/W boundary");
  // Staged epilogues, one region per wavefront of k-group 0 (the transposed V
  // store only in the QKV projection), then the k-group 1 partial sums.
  constexpr int EPI_LDS = NWM * WTM * epi_pitch<MB, NB>();
  constexpr int VT_LDS = EPI == EPI_QKV && (MB == 2 || MB == 3) ? NWM * 64 * vt_pitch<MB>() : 0;
  constexpr int PART_LDS = EPI == EPI_PARTIAL ? NWM * WTM * part_pitch<MB, NB>() : 0;
  constexpr int OUT_LDS = EPI_LDS > VT_LDS ? (EPI_LDS > PART_LDS ? EPI_LDS : PART_LDS)
                                           : (VT_LDS > PART_LDS ? VT_LDS : PART_LDS);
  constexpr int RED_LDS = KS == 2 ? NWM * MB * NB * 16 * 64 * 4 : 0;
  constexpr int MAIN_LDS = NST * STAGE > OUT_LDS + RED_LDS ? NST * STAGE : OUT_LDS + RED_LDS;
  static_assert(NST >= 2 && (NST - 2) * LW <= 63, "stages: vmcnt holds the loads of NST - 2 k-tiles");
  __shared__ __attribute__((aligned(1024))) char smem[MAIN_LDS + BN * 4];  // + the tile's bias
  float *bias_l = reinterpret_cast<float *>(smem + MAIN_LDS);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: selects LDS targets
  const int kg = wave / NWM, wq = wave % NWM;                   // k-group, wavefront in the group
  const int l32 = lane & 31, g = lane >> 5;
  const int wm = wq / WGN, wn = wq % WGN;

  const int n_tiles = (N + BN - 1) / BN, tiles = n_tiles * ((M + BM - 1) / BM);
  const int per_xcd = (tiles + NUM_XCD - 1) / NUM_XCD;
  const int tile = (blockIdx.x % NUM_XCD) * per_xcd + blockIdx.x / NUM_XCD;
  if (tile >= tiles) return;
  const int m0 = (tile / n_tiles) * BM, n0 = (tile % n_tiles) * BN;
  // the transposed V store's table lookup, issued now and consumed in the
  // epilogue (the main loop hides its latency)
  constexpr bool VT_STAGED = EPI == EPI_QKV && (MB == 2 || MB == 3) && sizeof(TO) == 2;
  const bool vt_staged = VT_STAGED && n0 >= 2 * 1024 && aux.seq_pad % 8 == 0 && M % 8 == 0;
  VtRun vrun{0, false};
  if constexpr (VT_STAGED) vrun = plan_vt<MB>(m0 + wm * WTM, M, aux.pk, vt_staged);
  // The tile's bias goes to LDS now (read back after many barriers), so the
  // epilogue does not wait on global loads.
  for (int c = tid; c < BN; c += 64 * NWM * KS) bias_l[c] = EPI != EPI_PARTIAL && n0 + c < N ? bias[n0 + c] : 0.f;

  // Rows past M (or N) lie beyond the resource range and read as zero. The
  // row offset is in the per-lane offset, which the range check covers; the
  // scalar offset only carries the k position in the row.
  const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(A + (size_t)m0 * lda), (short)0, min(M - m0, BM) * lda * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t w_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(W + (size_t)n0 * ldw), (short)0, min(N - n0, BN) * ldw * 2, 0x00020000);
  // Load instruction i covers tile rows 8i .. 8i+7 (A rows below BM, then W
  // rows); wavefront q of a k-group issues i = q, q + NWM, ... for that
  // group's k-tile. The swizzle depends on row & 15 = 8 (i & 1) + lane / 8,
  // the same for all of a wavefront's i because NWM is even. Where NWM does
  // not divide NI, a wavefront's surplus load repeats the last instruction of
  // its parity (the same bytes to the same LDS), so the loop has no branch.
  const int lr = lane >> 3;
  const int c0 = ((lane & 7) ^ swz8(8 * (wq & 1) + lr)) * 16;
  const int va = lr * lda * 2 + c0, vw = lr * ldw * 2 + c0;
  auto issue = [&](int kt, int stage) {
#pragma unroll
    for (int j = 0; j < LW; ++j) {
      const int i = j * NWM + wq < NI ? j * NWM + wq : NI - 1 - ((NI - 1 - wq) & 1);
      auto *dst = (__attribute__((address_space(3))) void *)(smem + stage * STAGE + kg * STAGE_G + i * 1024);
      if constexpr (NI % NWM == 0 && BM % (8 * NWM) == 0) {
        // the j-th load of every wavefront is on the same side of the A/W boundary
        if (j < BM / (8 * NWM))
          __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, dst, 16, va + 8 * i * lda * 2, kt * KTB, 0, 0);
        else
          __builtin_amdgcn_raw_ptr_buffer_load_lds(w_rsrc, dst, 16, vw + (8 * i - BM) * ldw * 2, kt * KTB, 0, 0);
      } else {
        const bool is_a = 8 * i < BM;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? a_rsrc : w_rsrc, dst, 16,
                                                 is_a ? va + 8 * i * lda * 2 : vw + (8 * i - BM) * ldw * 2,
                                                 kt * KTB, 0, 0);
      }
    }
  };

  f32x16 acc[MB][NB];
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int sw = swz8(l32 & 15);  // fragment rows are 16-aligned + l32
  const int a_row = (wm * WTM + l32) * KTB, w_row = (BM + wn * WTN + l32) * KTB;
  f16x8 af[2][MB], wf[2][NB];
  // More fragments than MFMAs per k-step (a 32 x 64 wavefront tile: 3 reads,
  // 2 MFMAs) in the few-tile shapes, one small workgroup per CU: the W
  // fragments are read first, so that the schedule below can issue them with
  // the step's first MFMA and no MFMA waits for a fragment read just before
  // it. (The 160 x 32 wavefront tiles of the two-stage shapes keep the plain
  // order: two wavefronts per SIMD hide that wait, and the early read made
  // the two-chain 32-clip step 1.4% slower.)
  constexpr bool READS_OVER = MB + NB > MB * NB && NST > 2;
  auto read_frags = [&](int stage, int ks, int slot) {
    const char *base = smem + stage * STAGE + kg * STAGE_G;
    const int chunk = ((2 * ks + g) ^ sw) * 16;
    if constexpr (READS_OVER) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
        wf[slot][j] = load8(reinterpret_cast<const f16 *>(base + w_row + j * 32 * KTB + chunk));
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) af[slot][i] = load8(reinterpret_cast<const f16 *>(base + a_row + i * 32 * KTB + chunk));
    if constexpr (!READS_OVER) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
        wf[slot][j] = load8(reinterpret_cast<const f16 *>(base + w_row + j * 32 * KTB + chunk));
    }
  };
  auto mfmas = [&](int slot) {
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = mfma32(wf[slot][j], af[slot][i], acc[i][j]);
  };

  // Iteration t: wait for this wavefront's loads of k-tile t (those of the
  // NST - 2 later k-tiles may still be in flight) and barrier (all loads of t
  // visible; every wavefront is done reading t-1's stage), refill that stage
  // with t + NST - 1, then 4 k-steps of fragment reads + MFMAs. With KS = 2
  // the two k-groups run this loop in step on the two halves of K (k-tiles
  // kg * nk/2 + t), each in its own half of every stage.
  const int nkg = K / 64 / KS, kbase = kg * nkg;
#pragma unroll
  for (int j = 0; j < NST - 1; ++j) issue(kbase + min(j, nkg - 1), j);
  for (int kt = 0; kt < nkg; ++kt) {
    const int s = kt % NST;
    __builtin_amdgcn_s_waitcnt(waitcnt_imm((NST - 2) * LW, 0));
    __builtin_amdgcn_s_barrier();
    issue(kbase + min(kt + NST - 1, nkg - 1), (kt + NST - 1) % NST);
    read_frags(s, 0, 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks < 3) read_frags(s, ks + 1, (ks + 1) & 1);
      mfmas(ks & 1);
    }
    // Schedule (masks: 0x010 VMEM, 0x100 LDS read, 0x008 MFMA): the loads,
    // the first k-step's fragments, then per k-step the next fragments one
    // per MFMA, then the rest of the MFMAs. With more fragments than MFMAs,
    // the surplus goes with the first MFMA, so every fragment is read while
    // at least one MFMA of the current step still runs.
    constexpr int NR = MB + NB, NM = MB * NB;
    __builtin_amdgcn_sched_group_barrier(0x010, LW, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
      if constexpr (READS_OVER) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, NR - NM + 1, 0);
#pragma unroll
        for (int i = 1; i < NM; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NR; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        if constexpr (NM >= NR) __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
  }

  // Every wavefront is done with the k-tile stages: LDS is free for the
  // k-group reduction and the staged epilogue.
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  __builtin_amdgcn_s_barrier();
  if constexpr (KS == 2) {
    // k-group 1 hands its partial sums to its partner in k-group 0 through
    // LDS (16 bytes per lane, consecutive lanes consecutive), then leaves.
    float4 *red = reinterpret_cast<float4 *>(smem + OUT_LDS) + wq * MB * NB * 4 * 64 + lane;
    if (kg == 1) {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4)
            red[((i * NB + j) * 4 + r4) * 64] = float4{acc[i][j][4 * r4], acc[i][j][4 * r4 + 1],
                                                       acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]};
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __builtin_amdgcn_s_barrier();
    if (kg == 1) return;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const float4 v = red[((i * NB + j) * 4 + r4) * 64];
          acc[i][j][4 * r4] += v.x;
          acc[i][j][4 * r4 + 1] += v.y;
          acc[i][j][4 * r4 + 2] += v.z;
          acc[i][j][4 * r4 + 3] += v.w;
        }
  }
  // Epilogue. fp16 outputs with 16-byte rows and split-K partial sums go
  // through LDS; the V part of the QKV projection through its transposed
  // staging; other fp32 outputs are stored straight from the accumulators.
  if constexpr (EPI == EPI_PARTIAL) {
    static_assert(sizeof(TO) == 4, "partial sums are fp32");
    if (vec_store == 1) {
      store_partial_lds<MB, NB>(acc, smem + wq * WTM * part_pitch<MB, NB>(), C, ldc, m0 + wm * WTM, n0 + wn * WTN,
                                M, N);
      return;
    }
  }
  if constexpr (sizeof(TO) == 2) {
    const bool v_part = EPI == EPI_QKV && n0 >= 2 * 1024;
    if (vec_store == 2 && !v_part) {
      store_tile_lds<EPI, MB, NB>(acc, smem + wq * WTM * epi_pitch<MB, NB>(), bias_l + wn * WTN, C, ldc,
                                  m0 + wm * WTM, n0 + wn * WTN, M, N);
      return;
    }
    if constexpr (VT_STAGED) {
      if (vt_staged) {
        store_vt_lds<MB, NB>(acc, smem + wq * 64 * vt_pitch<MB>(), bias_l + wn * WTN, static_cast<f16 *>(aux.vt),
                             m0 + wm * WTM, n0 + wn * WTN, M, vrun, aux.seq_pad);
        return;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
      store_block<EPI, TO>(acc[i][j], bias, C, ldc, m0 + wm * WTM + 32 * i + l32, n0 + wn * WTN + 32 * j + 4 * g, M, N,
                           vec_store, aux);
}

// DMA = 0 selects the register-staged main loop; DMA = 1 or 2 the fp16
// direct-to-LDS one with that many k-groups per workgroup.
template <int EPI, bool OUT_F32, typename T, int BM, int BN, int WGM, int WGN, int DMA, int NST>
__device__ __forceinline__ void gemm_body(const T *__restrict__ A, int lda, const T *__restrict__ W, int ldw,
                                          const float *__restrict__ bias, void *__restrict__ C, int ldc, int M, int N,
                                          int K, int vec_store, const GemmAux &aux) {
  typedef typename std::conditional<OUT_F32, float, T>::type TO;
  if constexpr (DMA)
    gemm_tile_dma<BM, BN, WGM, WGN, DMA, EPI, TO, NST>(A, lda, W, ldw, bias, static_cast<TO *>(C), ldc, M, N, K,
                                                     vec_store, aux);
  else
    gemm_tile<T, BM, BN, WGM, WGN, EPI, TO>(A, lda, W, ldw, bias, static_cast<TO *>(C), ldc, M, N, K, vec_store, aux);
}

// One kernel symbol per projection role and tile shape.
#define KMD_GEMM_ROLE(NAME, EPI, OUT_F32)                                                                   \
  template <typename T, int BM, int BN, int WGM, int WGN, int DMA, int MINB, int NST>                       \
  __global__ __launch_bounds__(64 * WGM * WGN * (DMA > 1 ? DMA : 1), MINB) void NAME(                      \
      const T *__restrict__ A, int lda, const T *__restrict__ W, int ldw, const float *__restrict__ bias,  \
      void *__restrict__ C, int ldc, int M, int N, int K, int vec_store, GemmAux aux) {                    \
    gemm_body<EPI, OUT_F32, T, BM, BN, WGM, WGN, DMA, NST>(A, lda, W, ldw, bias, C, ldc, M, N, K, vec_store,  \
                                                           aux);                                            \
  }
KMD_GEMM_ROLE(gemm_qkv, EPI_QKV, false)
KMD_GEMM_ROLE(gemm_out, EPI_BIAS, false)
KMD_GEMM_ROLE(gemm_ffn1_gelu, EPI_BIAS_GELU, false)
KMD_GEMM_ROLE(gemm_ffn2, EPI_BIAS, false)
KMD_GEMM_ROLE(gemm_in_proj, EPI_BIAS, true)
KMD_GEMM_ROLE(gemm_head, EPI_BIAS, true)
KMD_GEMM_ROLE(gemm_text, EPI_BIAS, false)
KMD_GEMM_ROLE(gemm_tmlp1_silu, EPI_BIAS_SILU, false)
KMD_GEMM_ROLE(gemm_tmlp2, EPI_BIAS, false)
#undef KMD_GEMM_ROLE

// Split-K (few output tiles): blockIdx.y = split takes k-tiles [split * klen,
// (split + 1) * klen) of the same tile grid and writes its fp32 partial sums
// to P[split][M][N]; splitk_reduce_kernel then adds the splits in index order
// (the result does not depend on which split finishes first), the bias and
// the role's epilogue.
template <int BM, int BN, int WGM, int WGN, int MINB, int NST>
__global__ __launch_bounds__(64 * WGM * WGN, MINB) void gemm_partial_kernel(const f16 *__restrict__ A, int lda,
                                                                          const f16 *__restrict__ W, int ldw,
                                                                          float *__restrict__ P, int M, int N,
                                                                          int klen, int vec) {
  const int split = blockIdx.y;
  gemm_tile_dma<BM, BN, WGM, WGN, 1, EPI_PARTIAL, float, NST>(A + (size_t)split * klen, lda,
                                                              W + (size_t)split * klen, ldw, nullptr,
                                                              P + (size_t)split * M * N, N, M, N, klen, vec,
                                                              GemmAux());
}

template <int EPI, typename TO>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ P, int splits,
                                                            const float *__restrict__ bias, TO *__restrict__ C,
                                                            int ldc, int M, int N, GemmAux aux) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t MN = (size_t)M * N;
  if (idx >= MN) return;
  const int m = (int)(idx / N), n = (int)(idx % N);
  // up to 8 splits' loads in flight at once; the sum stays in split order
  float v = 0.f;
  for (int s0 = 0; s0 < splits; s0 += 8) {
    float pv[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) pv[k] = s0 + k < splits ? P[(s0 + k) * MN + idx] : 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (s0 + k < splits) v += pv[k];
  }
  v += bias[n];
  if (EPI == EPI_BIAS_GELU) v = gelu_erf(v);
  if (EPI == EPI_BIAS_SILU) v = silu(v);
  if (EPI == EPI_QKV && n >= 2 * 1024) {
    const int ps = aux.pk.row_ps[m], p = ps >> 16, sq = ps & 0xffff;
    static_cast<TO *>(aux.vt)[((size_t)p * 1024 + (n - 2 * 1024)) * aux.seq_pad + sq] = from_f32<TO>(v);
    return;
  }
  C[(size_t)m * ldc + n] = from_f32<TO>(v);
}

template <typename T, int BM, int BN, int NT, typename K>
hipError_t launch_tiles(const char *name, K kernel, const T *A, int lda, const T *W, int ldw, const float *bias,
                        void *C, int ldc, int M, int N, int Kd, int vec, const GemmAux &aux, hipStream_t s) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int grid = ((tiles + NUM_XCD - 1) / NUM_XCD) * NUM_XCD;
  launch(name, kernel, dim3(grid), dim3(NT), s, A, lda, W, ldw, bias, C, ldc, M, N, Kd, vec, aux);
  return hipGetLastError();
}

}  // namespace

// Tile shapes, from measurements on MI355X at the denoiser's shapes (M =
// 2B(T+2) token rows; N, K from the layer). At small M the count of tiles
// against the 256 CUs decides: 4864 rows (16 clips x 150 frames) give 152
// tiles of 256 x 256 for N = 2048 (59 % of the CUs busy) but 496 tiles of
// 160 x 128 at two workgroups per CU.
//   QKV, M < 8192: 192 x 256, 8 wavefronts of 96 x 64 (at 32 clips of <= 180
//     frames about 252 tiles per chain, both chains 1.97 rounds of the CUs,
//     against 1.5 for 256 x 256: 0.295 -> 0.335 of peak per launch);
//   FFN1, M < 8192: 160 x 128, 4 wavefronts of 160 x 32, two workgroups per CU;
//   OUT / FFN2 (N = 1024), M < 8192: one workgroup of 4 wavefronts per CU
//     with four LDS stages (three k-tiles in flight): 160 x 128 while one
//     chain's tiles fit half of the CUs (at most 128: 2,432 rows, the two
//     chains then fill the chip once), else 128 x 128. Against 160 x 128
//     with two k-groups of 4 wavefronts on the two halves of K (one k-tile
//     in flight each): 16 x 150 OUT 15.0 -> 13.5 us, FFN2 25.2 -> 22.4 us,
//     the step -2 to -4%; 32 x <= 180 the step -1.5 to -2% (128 x 128; its
//     160 x 128 tiles would over-fill the chip, as 128 x 128 tiles do at 16
//     x 150: +1.7%);
//   layer GEMMs, 8192 <= M < 16384: 192 x 256, 8 wavefronts of 96 x 64;
//   layer GEMMs, M >= 16384: 256 x 256;
//   input projection, heads, text and timestep MLPs: 128 x 128, 4 wavefronts;
//   few tiles, no split-K: 128 x 128 with four LDS stages (FFN1, heads and
//     input projections: 64 x 64 with eight, see few_tile);
//   fp32 (the correctness setting): register-staged 128 x 128 tile.
enum TileCfg {
  TILE_256x256, TILE_192x256, TILE_160x128, TILE_128x128, TILE_128x128_S4, TILE_64x64_S8, TILE_64x128_S6,
  TILE_160x128_S4
};

// Few output tiles (a GEMM split-K does not take). The loop is then bound by
// load latency, not by the MFMAs: each workgroup walks all of K with a few
// k-tiles in flight. For FFN1, the heads and the input projections, 64 x 64
// tiles give four times the workgroups of 128 x 128 and eight LDS stages,
// seven k-tiles in flight, as long as they all fit one round of the CUs (one
// workgroup per CU: 129 KB of LDS). 1 clip (FFN1 304 x 2048 x 1024, 160
// tiles): 1.98 -> 1.88 ms per step, and 1% more with the heads and input
// projections; with 384 tiles (FFN1 of 4 takes of 90 frames) the second
// round made the pass 5% slower; there 64 x 128 tiles with six stages (192
// of them, five k-tiles in flight) gain 0.7% over 128 x 128. The QKV
// projection keeps 128 x 128: its staged V^T store needs 64-row sub-tiles,
// and at 64 x 64 it lost half of FFN1's gain.
TileCfg few_tile(GemmRole role, int M, int N) {
  const bool one_round = ((M + 63) / 64) * ((N + 63) / 64) <= 256;
  if ((role == ROLE_FFN1 || role == ROLE_HEAD || role == ROLE_IN) && one_round) return TILE_64x64_S8;
  if (role == ROLE_FFN1 && ((M + 63) / 64) * ((N + 127) / 128) <= 256) return TILE_64x128_S6;
  return TILE_128x128_S4;
}

TileCfg pick_tile(GemmRole role, int M, int N, int K) {
  if (role != ROLE_QKV && role != ROLE_OUT && role != ROLE_FFN1 && role != ROLE_FFN2) return TILE_128x128;
  if (M >= 16384) return TILE_256x256;
  if (M >= 8192) return TILE_192x256;
  if (role == ROLE_QKV) return TILE_192x256;
  // N = 1024: four-stage tiles, 160 rows while a chain's tiles fit half of
  // the CUs
  if (role == ROLE_OUT || role == ROLE_FFN2)
    return ((M + 159) / 160) * ((N + 127) / 128) <= 128 ? TILE_160x128_S4 : TILE_128x128_S4;
  return TILE_160x128;
}

// Split-K tiles are 128 x 128 (2 x 2 wavefronts of 64 x 64). A GEMM with at
// most 128 such tiles (1 to 4 sequences of ~150 tokens; a 1,024-wide product
// of up to ~2,000 rows) leaves CUs idle while each workgroup walks all of K;
// it is split instead into the largest divisor of its k-tile count that keeps
// at most 256 workgroups, at least 4 k-tiles per split, and the partial sums
// within aux.partial_cap floats. A split has few k-tiles and its weights come
// from HBM, so its workgroup (one per CU) has four LDS stages: three k-tiles
// in flight, one load round trip for a split of up to 4 k-tiles instead of
// one per k-tile. Below 4 k-tiles per split the partial sums cost more than
// the extra workgroups gain (304 x 1024 x 1024: 6.39 us at 4 splits, 6.44 us
// at 8, with twice the partial sums for the reduction to read).
constexpr int SPLITK_TILE = 128, SPLITK_MAX_TILES = 128, SPLITK_WGS = 256;
constexpr int SPLITK_NST = 4, SPLITK_MINB = 1;
constexpr int SPLITK_SOLO_MIN_KT = 32;  // k-tiles from which a split with its own reduction kernel pays

int splitk_splits(int M, int N, int K, const GemmAux &aux) {
  if (!aux.partial) return 1;
  const int tiles = ((M + SPLITK_TILE - 1) / SPLITK_TILE) * ((N + SPLITK_TILE - 1) / SPLITK_TILE);
  const int nk = K / 64;
  if (tiles > SPLITK_MAX_TILES || nk < 4) return 1;
  int best = 1;
  for (int sp = 2; sp <= nk / 4; ++sp)
    if (nk % sp == 0 && sp * tiles <= SPLITK_WGS && (size_t)sp * M * N <= aux.partial_cap) best = sp;
  return best;
}

template <int EPI, typename TO>
hipError_t splitk_run(const char *name, const f16 *A, int lda, const f16 *W, int ldw, const float *bias, void *C,
                      int ldc, int M, int N, int K, int splits, const GemmAux &aux, hipStream_t s) {
  const int tiles = ((M + SPLITK_TILE - 1) / SPLITK_TILE) * ((N + SPLITK_TILE - 1) / SPLITK_TILE);
  const int grid_x = ((tiles + NUM_XCD - 1) / NUM_XCD) * NUM_XCD;
  launch(name, gemm_partial_kernel<SPLITK_TILE, SPLITK_TILE, 2, 2, SPLITK_MINB, SPLITK_NST>, dim3(grid_x, splits), dim3(256), s, A, lda, W,
         ldw, aux.partial, M, N, K / splits, N % 4 == 0 ? 1 : 0);
  const size_t MN = (size_t)M * N;
  launch("splitk_reduce", splitk_reduce_kernel<EPI, TO>, dim3((unsigned)((MN + 255) / 256)), dim3(256), s,
         static_cast<const float *>(aux.partial), splits, bias, static_cast<TO *>(C), ldc, M, N, aux);
  return hipGetLastError();
}

hipError_t gemm_splitk(GemmRole role, const f16 *A, int lda, const f16 *W, int ldw, const float *bias, void *C,
                       int ldc, int M, int N, int K, int splits, const GemmAux &aux, hipStream_t s) {
  switch (role) {
    case ROLE_QKV: return splitk_run<EPI_QKV, f16>("gemm_qkv:splitk", A, lda, W, ldw, bias, C, ldc, M, N, K, splits, aux, s);
    case ROLE_OUT: return splitk_run<EPI_BIAS, f16>("gemm_out:splitk", A, lda, W, ldw, bias, C, ldc, M, N, K, splits, aux, s);
    case ROLE_FFN1:
      return splitk_run<EPI_BIAS_GELU, f16>("gemm_ffn1_gelu:splitk", A, lda, W, ldw, bias, C, ldc, M, N, K, splits, aux, s);
    case ROLE_FFN2: return splitk_run<EPI_BIAS, f16>("gemm_ffn2:splitk", A, lda, W, ldw, bias, C, ldc, M, N, K, splits, aux, s);
    case ROLE_IN: return splitk_run<EPI_BIAS, float>("gemm_in_proj:splitk", A, lda, W, ldw, bias, C, ldc, M, N, K, splits, aux, s);
    case ROLE_HEAD: return splitk_run<EPI_BIAS, float>("gemm_head:splitk", A, lda, W, ldw, bias, C, ldc, M, N, K, splits, aux, s);
    case ROLE_TXT: return splitk_run<EPI_BIAS, f16>("gemm_text:splitk", A, lda, W, ldw, bias, C, ldc, M, N, K, splits, aux, s);
    case ROLE_TMLP1:
      return splitk_run<EPI_BIAS_SILU, f16>("gemm_tmlp1_silu:splitk", A, lda, W, ldw, bias, C, ldc, M, N, K, splits, aux, s);
    case ROLE_TMLP2: return splitk_run<EPI_BIAS, f16>("gemm_tmlp2:splitk", A, lda, W, ldw, bias, C, ldc, M, N, K, splits, aux, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t gemm_partials(const char *name, const T *A, int lda, const T *W, int ldw, int M, int N, int K,
                         const GemmAux &aux, int *splits, hipStream_t s) {
  *splits = 1;
  if constexpr (sizeof(T) == 2) {
    if (M <= 0 || N <= 0 || K % 64 != 0 || lda % 8 || ldw % 8) return hipSuccess;
    const int sp = splitk_splits(M, N, K, aux);
    if (sp < 2) return hipSuccess;
    const int tiles = ((M + SPLITK_TILE - 1) / SPLITK_TILE) * ((N + SPLITK_TILE - 1) / SPLITK_TILE);
    const int grid_x = ((tiles + NUM_XCD - 1) / NUM_XCD) * NUM_XCD;
    launch(name, gemm_partial_kernel<SPLITK_TILE, SPLITK_TILE, 2, 2, SPLITK_MINB, SPLITK_NST>, dim3(grid_x, sp), dim3(256), s, A,
           lda, W, ldw, aux.partial, M, N, K / sp, N % 4 == 0 ? 1 : 0);
    *splits = sp;
    return hipGetLastError();
  }
  return hipSuccess;
}
template hipError_t gemm_partials<f16>(const char *, const f16 *, int, const f16 *, int, int, int, int,
                                       const GemmAux &, int *, hipStream_t);
template hipError_t gemm_partials<float>(const char *, const float *, int, const float *, int, int, int, int,
                                         const GemmAux &, int *, hipStream_t);

template <typename T>
hipError_t gemm(GemmRole role, const T *A, int lda, const T *W, int ldw, const float *bias, void *C, int ldc, int M,
                int N, int K, hipStream_t s, const GemmAux &aux) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K % gemm_k_tile<T>() != 0 || lda % (16 / (int)sizeof(T)) || ldw % (16 / (int)sizeof(T)))
    return hipErrorInvalidValue;
  // The QKV epilogue writes the V columns to aux.vt: it needs that buffer and a
  // whole number of sequences.
  // QKV rows are packed sequences that start on multiples of 8 rows
  if (role == ROLE_QKV && (aux.vt == nullptr || !aux.pk.row_ps || N != 3 * 1024 || M % 8 != 0))
    return hipErrorInvalidValue;
  bool few_tiles = false;
  if constexpr (sizeof(T) == 2) {
    // Here every split needs a reduction kernel of its own (the output and
    // FFN2 projections reduce inside the LayerNorm through gemm_partials
    // instead). Below SPLITK_SOLO_MIN_KT k-tiles one pass of the four-stage
    // loop is faster than the split plus that kernel (304 x 2048 x 1024:
    // 10.9 us against 7.2 + 4.7 us; 304 x 3072 x 1024: 11.1 against 8.6 + 5.7).
    const int splits = K / 64 >= SPLITK_SOLO_MIN_KT ? splitk_splits(M, N, K, aux) : 1;
    if (splits > 1) return gemm_splitk(role, A, lda, W, ldw, bias, C, ldc, M, N, K, splits, aux, s);
    // The QKV projection takes the few-tile path up to one round of the CUs
    // (8 sequences of 92 tokens: 144 tiles, against 36 of 256 x 256).
    const int tiles128 = ((M + SPLITK_TILE - 1) / SPLITK_TILE) * ((N + SPLITK_TILE - 1) / SPLITK_TILE);
    few_tiles = tiles128 <= (role == ROLE_QKV ? 2 * SPLITK_MAX_TILES : SPLITK_MAX_TILES);
  }
  const bool out_f32 = role == ROLE_IN || role == ROLE_HEAD;
  const size_t osize = out_f32 ? 4 : sizeof(T);
  // 2: 16-byte fp16 row chunks (LDS-staged epilogue), 1: 4-element stores, 0: scalar stores.
  const int vec = osize == 2 && ldc % 8 == 0 && N % 8 == 0 && reinterpret_cast<uintptr_t>(C) % 16 == 0 ? 2
                  : (ldc % 4 == 0) && (reinterpret_cast<uintptr_t>(C) % (4 * osize) == 0) ? 1
                                                                                          : 0;
  // few tiles: one workgroup per CU, each with four LDS stages (as the split-K
  // partial kernel), so its k-tiles stream three at a time
  const TileCfg cfg = few_tiles ? few_tile(role, M, N) : pick_tile(role, M, N, K);
#define KMD_GO_S(NAME, BM, BN, WGM, WGN, DMA, MINB, NST)                                                        \
  return launch_tiles<T, BM, BN, 64 * WGM * WGN * (DMA > 1 ? DMA : 1)>(                                         \
      #NAME, NAME<T, BM, BN, WGM, WGN, DMA, MINB, NST>, A, lda, W, ldw, bias, C, ldc, M, N, K, vec, aux, s)
#define KMD_GO(NAME, BM, BN, WGM, WGN, DMA, MINB) KMD_GO_S(NAME, BM, BN, WGM, WGN, DMA, MINB, 2)
#define KMD_LAYER_ROLE(R, NAME)                                     \
  case R:                                                           \
    if constexpr (sizeof(T) == 4) {                                 \
      KMD_GO(NAME, 128, 128, 2, 2, 0, 2);                           \
    } else {                                                        \
      switch (cfg) {                                                \
        case TILE_256x256: KMD_GO(NAME, 256, 256, 4, 2, 1, 1);      \
        case TILE_192x256: KMD_GO(NAME, 192, 256, 2, 4, 1, 1);      \
        case TILE_160x128: KMD_GO(NAME, 160, 128, 1, 4, 1, 2);      \
        case TILE_160x128_S4: KMD_GO_S(NAME, 160, 128, 1, 4, 1, 1, 4); \
        case TILE_128x128_S4: KMD_GO_S(NAME, 128, 128, 2, 2, 1, 1, 4); \
        case TILE_64x64_S8: KMD_GO_S(NAME, 64, 64, 2, 1, 1, 1, 8);  \
        case TILE_64x128_S6: KMD_GO_S(NAME, 64, 128, 1, 2, 1, 1, 6); \
        default: KMD_GO(NAME, 128, 128, 2, 2, 1, 2);                \
      }                                                             \
    }
#define KMD_SMALL_ROLE(R, NAME)                                     \
  case R:                                                           \
    if constexpr (sizeof(T) == 4) KMD_GO(NAME, 128, 128, 2, 2, 0, 2); \
    else if (cfg == TILE_128x128_S4) KMD_GO_S(NAME, 128, 128, 2, 2, 1, 1, 4); \
    else if (cfg == TILE_64x64_S8) KMD_GO_S(NAME, 64, 64, 2, 1, 1, 1, 8); \
    else KMD_GO(NAME, 128, 128, 2, 2, 1, 2);
  switch (role) {
    KMD_LAYER_ROLE(ROLE_QKV, gemm_qkv)
    KMD_LAYER_ROLE(ROLE_OUT, gemm_out)
    KMD_LAYER_ROLE(ROLE_FFN1, gemm_ffn1_gelu)
    KMD_LAYER_ROLE(ROLE_FFN2, gemm_ffn2)
    KMD_SMALL_ROLE(ROLE_IN, gemm_in_proj)
    KMD_SMALL_ROLE(ROLE_HEAD, gemm_head)
    KMD_SMALL_ROLE(ROLE_TXT, gemm_text)
    KMD_SMALL_ROLE(ROLE_TMLP1, gemm_tmlp1_silu)
    KMD_SMALL_ROLE(ROLE_TMLP2, gemm_tmlp2)
  }
#undef KMD_SMALL_ROLE
#undef KMD_LAYER_ROLE
#undef KMD_GO
#undef KMD_GO_S
  return hipErrorInvalidValue;
}

template hipError_t gemm<f16>(GemmRole, const f16 *, int, const f16 *, int, const float *, void *, int, int, int, int,
                              hipStream_t, const GemmAux &);
template hipError_t gemm<float>(GemmRole, const float *, int, const float *, int, const float *, void *, int, int, int,
                                int, hipStream_t, const GemmAux &);

}  // namespace kmd
