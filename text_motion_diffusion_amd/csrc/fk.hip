// Forward-kinematics decode of sampled motion into joint positions and global
// rotation matrices on the 30-joint skeleton (Kimodo WebGPU README: the FK
// decode after the denoising loop, "Model details" table: SOMA30, output joint
// positions and rotation matrices). Frame layout: root stream (x, y, z, c, s),
// then 30 joints x 9 features whose first 6 are the joint's local rotation in
// the 6D form of Zhou et al., "On the Continuity of Rotation Representations
// in Neural Networks" (CVPR 2019): two columns made orthonormal by
// Gram-Schmidt, the third their cross product. The root joint's global
// rotation is the heading yaw (x' = c x - s z, z' = s x + c z, the root
// conversion's convention) times its local rotation, at the root position;
// joint j has R_j = R_parent L_j and p_j = p_parent + R_parent o_j.
//
// gfx950 mapping: one half-wavefront (32 lanes) per frame, lane j = joint j
// (lanes 30, 31 idle), 8 frames per workgroup. The workgroup's input rows and
// outputs are contiguous, so they pass through LDS with 16-byte loads and
// stores that consecutive threads issue to consecutive addresses. Every lane
// builds its local rotation at once; the tree is then composed by pointer
// jumping in ceil(log2(depth + 1)) rounds of cross-lane permutes (4 for a
// depth-8 tree, against 8 rounds level by level). Bandwidth-bound: 0.74 KB of
// features read (whole 1.1 KB rows are fetched) and 1.44 KB written per frame.
#include "common.h"
#include "kernels.h"

namespace kmd {
namespace {

constexpr int NJ = 30, ROOT = 5, FEATS = 279, JF = 9;

__device__ __forceinline__ float inv_len(float x, float y, float z) {
  return 1.0f / fmaxf(sqrtf(x * x + y * y + z * z), 1e-8f);
}

constexpr int FPB = 8;  // frames per 256-thread workgroup, one per half-wavefront

// A workgroup's 8 frames are contiguous in x, pos and rot (8 x 1116, 8 x 360
// and 8 x 1080 bytes, all multiples of 16), so with vec set (16-byte aligned
// pointers, a whole block) they move as float4 through LDS; otherwise
// (ragged last block, unaligned pointers) element by element.
__global__ __launch_bounds__(256) void fk_kernel(const float *__restrict__ x, int n, FkSkeleton sk,
                                                 float *__restrict__ pos, float *__restrict__ rot, int vec) {
  __shared__ float4 s_in[FPB * FEATS / 4];
  __shared__ float4 s_pos[FPB * NJ * 3 / 4];
  __shared__ float4 s_rot[FPB * NJ * 9 / 4];
  float *si = reinterpret_cast<float *>(s_in), *sp = reinterpret_cast<float *>(s_pos),
        *sr = reinterpret_cast<float *>(s_rot);
  const int tid = threadIdx.x, lane = tid & 63, j = lane & 31, fl = tid >> 5;
  const int f0 = blockIdx.x * FPB, nf = min(FPB, n - f0);
  const bool full = vec && nf == FPB;
  if (full) {
    const float4 *src = reinterpret_cast<const float4 *>(x + (size_t)f0 * FEATS);
    for (int i = tid; i < FPB * FEATS / 4; i += 256) s_in[i] = src[i];
  } else {
    for (int i = tid; i < nf * FEATS; i += 256) si[i] = x[(size_t)f0 * FEATS + i];
  }
  __syncthreads();
  const bool valid = fl < nf, joint = j < NJ;
  const float *xf = si + fl * FEATS;
  float g[ROOT], a[6];
#pragma unroll
  for (int c = 0; c < ROOT; ++c) g[c] = valid ? xf[c] : 0.f;
#pragma unroll
  for (int c = 0; c < 6; ++c) a[c] = valid && joint ? xf[ROOT + JF * j + c] : 0.f;

  // local rotation L (row-major), columns b1, b2, b3
  float L[9];
  {
    const float s1 = inv_len(a[0], a[1], a[2]);
    const float b1[3] = {a[0] * s1, a[1] * s1, a[2] * s1};
    const float d = b1[0] * a[3] + b1[1] * a[4] + b1[2] * a[5];
    float u[3] = {a[3] - d * b1[0], a[4] - d * b1[1], a[5] - d * b1[2]};
    const float s2 = inv_len(u[0], u[1], u[2]);
    const float b2[3] = {u[0] * s2, u[1] * s2, u[2] * s2};
    const float b3[3] = {b1[1] * b2[2] - b1[2] * b2[1], b1[2] * b2[0] - b1[0] * b2[2], b1[0] * b2[1] - b1[1] * b2[0]};
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      L[3 * r] = b1[r];
      L[3 * r + 1] = b2[r];
      L[3 * r + 2] = b3[r];
    }
  }
  float R[9], p[3] = {0.f, 0.f, 0.f};
  if (j == 0) {
    // heading yaw H = [[hc, 0, -hs], [0, 1, 0], [hs, 0, hc]] times L
    const float hn = fmaxf(sqrtf(g[3] * g[3] + g[4] * g[4]), 1e-8f);
    const float hc = g[3] / hn, hs = g[4] / hn;
#pragma unroll
    for (int c = 0; c < 3; ++c) {
      R[c] = hc * L[c] - hs * L[6 + c];
      R[3 + c] = L[3 + c];
      R[6 + c] = hs * L[c] + hc * L[6 + c];
    }
    p[0] = g[0];
    p[1] = g[1];
    p[2] = g[2];
  } else {
#pragma unroll
    for (int k = 0; k < 9; ++k) R[k] = L[k];
  }
  // Pointer jumping (Wyllie's list ranking on the tree): every lane holds the
  // transform (R, p) of its joint relative to the frame of joint anc[r] (its
  // parent at first; the root's is already global). Each round composes it
  // with anc[r]'s transform, read from that lane, so after r rounds a lane
  // spans 2^r joints of its path to the root and ceil(log2(depth + 1))
  // rounds make every transform global. The ancestors of every round come
  // from the host. Only the first two columns of a rotation cross lanes: the
  // third is their cross product (both are orthonormal), rebuilt after the
  // exchange and at the end.
  const int jj = joint ? j : 0;
  int anc[FK_MAX_ROUNDS];
#pragma unroll
  for (int r = 0; r < FK_MAX_ROUNDS; ++r) anc[r] = joint ? sk.anc[r][jj] : -1;
  if (j > 0) {
    p[0] = sk.offset[jj][0];
    p[1] = sk.offset[jj][1];
    p[2] = sk.offset[jj][2];
  }
#pragma unroll
  for (int round = 0; round < FK_MAX_ROUNDS; ++round) {
    if (round >= sk.rounds) break;
    const int a = anc[round];
    const int srcl = (lane & 32) | (a >= 0 ? a : j);
    float Ra[9], pa[3];
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      Ra[3 * r] = __shfl(R[3 * r], srcl, 64);
      Ra[3 * r + 1] = __shfl(R[3 * r + 1], srcl, 64);
      pa[r] = __shfl(p[r], srcl, 64);
    }
    // third column = first x second
    Ra[2] = Ra[3] * Ra[7] - Ra[6] * Ra[4];
    Ra[5] = Ra[6] * Ra[1] - Ra[0] * Ra[7];
    Ra[8] = Ra[0] * Ra[4] - Ra[3] * Ra[1];
    if (a >= 0) {
      float Rn[6], pn[3];
#pragma unroll
      for (int r = 0; r < 3; ++r) {
#pragma unroll
        for (int c = 0; c < 2; ++c) Rn[2 * r + c] = Ra[3 * r] * R[c] + Ra[3 * r + 1] * R[3 + c] + Ra[3 * r + 2] * R[6 + c];
        pn[r] = pa[r] + Ra[3 * r] * p[0] + Ra[3 * r + 1] * p[1] + Ra[3 * r + 2] * p[2];
      }
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        R[3 * r] = Rn[2 * r];
        R[3 * r + 1] = Rn[2 * r + 1];
        p[r] = pn[r];
      }
      R[2] = R[3] * R[7] - R[6] * R[4];
      R[5] = R[6] * R[1] - R[0] * R[7];
      R[8] = R[0] * R[4] - R[3] * R[1];
    }
  }
  if (valid && joint) {
#pragma unroll
    for (int k = 0; k < 3; ++k) sp[(fl * NJ + j) * 3 + k] = p[k];
#pragma unroll
    for (int k = 0; k < 9; ++k) sr[(fl * NJ + j) * 9 + k] = R[k];
  }
  __syncthreads();
  if (full) {
    float4 *pd = reinterpret_cast<float4 *>(pos + (size_t)f0 * NJ * 3);
    for (int i = tid; i < FPB * NJ * 3 / 4; i += 256) pd[i] = s_pos[i];
    if (rot) {
      float4 *rd = reinterpret_cast<float4 *>(rot + (size_t)f0 * NJ * 9);
      for (int i = tid; i < FPB * NJ * 9 / 4; i += 256) rd[i] = s_rot[i];
    }
  } else {
    for (int i = tid; i < nf * NJ * 3; i += 256) pos[(size_t)f0 * NJ * 3 + i] = sp[i];
    if (rot)
      for (int i = tid; i < nf * NJ * 9; i += 256) rot[(size_t)f0 * NJ * 9 + i] = sr[i];
  }
}

}  // namespace

hipError_t fk_decode(const float *x, int n, const FkSkeleton &sk, float *pos, float *rot, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const uintptr_t bits = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(pos) |
                         reinterpret_cast<uintptr_t>(rot);
  const int vec = (bits & 15) == 0;
  launch("fk", fk_kernel, dim3((unsigned)((n + FPB - 1) / FPB)), dim3(256), s, x, n, sk, pos, rot, vec);
  return hipGetLastError();
}

}  // namespace kmd
