// Exact attention over the uncompressed recent window, one 128-token tile
// per workgroup of 4 waves (32 tokens per wave), gfx950.
//
// LowRAM review (agihunt.info), keys paragraph: only the older part of the
// context is compressed; the most recent tokens keep their exact keys and
// values, and every step attends them in full beside the rebuilt chunks.
// A tile ends as one partial softmax state (m, l, o) per query head of its
// KV head, in the same slot format as the selected-chunk tiles, so the merge
// treats both alike.  The 4-wave attention kernel runs these tiles in its
// own grid, and the landmark-score kernel runs them as extra workgroups of
// its grid (the window needs neither the scores nor the selection).
#pragma once
#include "common.h"
#include "internal.h"

namespace lowram {

// Softmax state of one wave's 16 NT tokens for query head j = col: the logits
// z[t][j] sit in rows t = 16 nt + 4 grp + e of zacc[nt].  Returns the wave's
// max and sum and the unnormalised weights as NT / 2 MFMA operands; in
// operand q, k slot 8 grp + e' is token 32 q + 4 grp + e' (e' < 4) or
// 32 q + 16 + 4 grp + e' - 4.
template <int NT>
__device__ __forceinline__ void wave_softmax(const f32x4 (&zacc)[NT], int nvalid, float scale_log2, int grp,
                                             float& m, float& lsum, bf16x8 (&pa)[NT / 2]) {
  float p[NT][4];
  m = -__builtin_huge_valf();
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * nt + 4 * grp + e;
      p[nt][e] = t < nvalid ? zacc[nt][e] * scale_log2 : -__builtin_huge_valf();
      m = fmaxf(m, p[nt][e]);
    }
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  const float msafe = m == -__builtin_huge_valf() ? 0.f : m;
  lsum = 0.f;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[nt][e] = __builtin_amdgcn_exp2f(p[nt][e] - msafe);
      lsum += p[nt][e];
    }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
#pragma unroll
  for (int q = 0; q < NT / 2; ++q)
    pa[q] = pack8(f32x4{p[2 * q][0], p[2 * q][1], p[2 * q][2], p[2 * q][3]},
                  f32x4{p[2 * q + 1][0], p[2 * q + 1][1], p[2 * q + 1][2], p[2 * q + 1][3]});
}

// One wave's tokens [w0, w0 + 32) of the window (those at or past `window`
// are masked; their loads are clamped into it).  qh: the KV head's g query
// rows; kw, vw: its window keys (post-RoPE) and values, [window][d] bf16.
// Ends with the wave's softmax state of query head j = col (m, l) and
// o^T[d][j] in rows d = 16 nd + 4 grp + e of oacc[nd].
//   QK  z[t][j] = K[t][d] x q[j][d]   (K rows as the A operand, 16-byte loads)
//   PV  o[d][j] = V^T[d][t] x p[t][j] (V^T gathered as the A operand)
__device__ __forceinline__ void window_wave(const uint16_t* qh, const uint16_t* kw, const uint16_t* vw, int w0,
                                            int window, int g, float scale_log2, int grp, int col,
                                            f32x4 (&oacc)[8], float& wm, float& wl) {
  const int nvalid = max(0, min(kAttTokWave, window - w0));
  bf16x8 qn[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qn[s] = col < g ? load_bf16x8(qh + col * kHeadDim + 32 * s + 8 * grp) : zero_bf16x8();
  f32x4 zacc[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int t = min(w0 + 16 * nt + col, window - 1);
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) z = mfma16(load_bf16x8(kw + (size_t)t * kHeadDim + 32 * s + 8 * grp), qn[s], z);
    zacc[nt] = z;
  }
  // V^T[d][t] as the A operand: dimension d = 16 nd + col, token slots
  bf16x8 vt[8];
#pragma unroll
  for (int nd = 0; nd < 8; ++nd) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = min(w0 + 16 * (e >> 2) + 4 * grp + (e & 3), window - 1);
      vt[nd][e] = __builtin_bit_cast(__bf16, vw[(size_t)t * kHeadDim + 16 * nd + col]);
    }
  }
  bf16x8 pa[1];
  wave_softmax<2>(zacc, nvalid, scale_log2, grp, wm, wl, pa);
#pragma unroll
  for (int nd = 0; nd < 8; ++nd) oacc[nd] = mfma16(vt[nd], pa[0], f32x4{0.f, 0.f, 0.f, 0.f});
}

// The 4 waves' states (as window_wave leaves them) combined into one partial
// per query head j < g, written to part[j * kPartStride + {0: m, 1: l,
// 2 + d: o}].  mo: 4 * 16 * 128 floats (32 KiB) of LDS, ml: 2 * 4 * 16 floats of LDS; both
// are overwritten, after a barrier, so the caller may have used that memory.
__device__ __forceinline__ void write_partial4(float* mo, float* ml, const f32x4 (&oacc)[8], float wm, float wl,
                                               float* part, int g, int tid, int wave, int grp, int col) {
  __syncthreads();
#pragma unroll
  for (int nd = 0; nd < 8; ++nd)
    *reinterpret_cast<f32x4*>(&mo[(wave * 16 + col) * kHeadDim + 16 * nd + 4 * grp]) = oacc[nd];
  if (grp == 0) {
    ml[wave * 16 + col] = wm;
    ml[kAttWaves * 16 + wave * 16 + col] = wl;
  }
  __syncthreads();
  for (int idx = tid; idx < g * kHeadDim; idx += kAttWaves * 64) {
    const int j = idx / kHeadDim, d = idx % kHeadDim;
    float M = -__builtin_huge_valf();
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) M = fmaxf(M, ml[w * 16 + j]);
    float lt = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) {
      const float mw = ml[w * 16 + j];
      const float sc = mw == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      lt += ml[kAttWaves * 16 + w * 16 + j] * sc;
      o += mo[(w * 16 + j) * kHeadDim + d] * sc;
    }
    if (d == 0) {
      part[j * kPartStride] = M;
      part[j * kPartStride + 1] = lt;
    }
    part[j * kPartStride + 2 + d] = o;
  }
}

}  // namespace lowram
