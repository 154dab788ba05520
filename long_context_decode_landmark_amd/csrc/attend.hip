// Fused selective reconstruction + GQA split-K flash-decode attention, gfx950.
//
// For the top-k chunks of one (sequence, KV head) this rebuilds the tokens'
// keys and values and attends over them, never writing a rebuilt key or
// value to HBM:
//   K_pre = C[t] . B_blk        cross-layer low-rank keys (LowRAM review,
//                               key paragraph; explainer "Low-rank keys")
//   K_post = RoPE(K_pre, t)     RoPE re-applied at the token position (keys
//                               are stored with RoPE undone)
//   V = W2 gelu(W1 K_pre + b1) + b2 + R[t]
//                               amortised values + residual of the worst
//                               tokens (review, value paragraph; explainer
//                               "Amortised values", "Residuals")
//   partial softmax state (m, l, o) of the GQA query heads over the tokens
// The exact recent window is attended by extra workgroups of the same grid.
//
// Layout of the work.  A workgroup is 8 waves; each wave owns 32 tokens
// (4 chunks) and runs every stage on them with v_mfma_f32_16x16x32_bf16.
// Tokens are the MFMA N dimension throughout, so each stage's accumulator
// layout is the next stage's operand layout (up to a fixed permutation of
// the contraction index, applied to the other operand instead):
//   recon   D[d][t]  = basis^T[d][r] (LDS)   x C[t][r] (global -> VGPR)
//   RoPE    lane-local: pair (i, i+64) sits in m-tiles mt and mt+4
//   QK      D[t][j]  = K_post[t][d] (VGPR, hi+lo bf16) x q[j][d]
//   MLP1    D[h][t]  = W1[h][d] (LDS)        x K_pre[t][d] (VGPR)
//   MLP2    D[t][d]  = hid[t][h] (VGPR)      x W2[d][h] (LDS)
//   PV      D[j][d]  = p[j][t] (VGPR)        x V[t][d] (VGPR, hi+lo bf16)
// The shared operands (basis block, then W1/W2) are staged in LDS once per
// workgroup and read by all 8 waves.
#include "common.h"
#include "internal.h"

namespace lowram {

// Sigmoid-form GELU: Phi(x) = sigmoid(logit Phi(x)) with logit Phi(x) fitted
// by the odd polynomial x * P(x^2), P of degree 4 (weighted least squares of
// the GELU error over |x| <= 5, x^2 clamped at 25 inside P so the sigmoid
// saturates correctly beyond).  This is the sigmoid/tanh approximation form
// of Hendrycks & Gimpel's GELU paper with a refitted polynomial; its maximum
// absolute deviation from the exact erf form is 3.1e-6 on the real line.
constexpr float kGeluP0 = 1.595655155f;
constexpr float kGeluP1 = 0.07293980766f;
constexpr float kGeluP2 = -0.0002509101281f;
constexpr float kGeluP3 = -6.094355622e-05f;
constexpr float kGeluP4 = 2.225823705e-06f;

__device__ __forceinline__ float gelu_fast(float x) {
  const float u = fminf(x * x, 25.0f);
  const float p = fmaf(fmaf(fmaf(fmaf(kGeluP4, u, kGeluP3), u, kGeluP2), u, kGeluP1), u, kGeluP0);
  const float t = __builtin_amdgcn_exp2f(-kLog2e * x * p);
  return x * __builtin_amdgcn_rcpf(1.0f + t);
}

// 2*pi split for the Cody-Waite reduction of large RoPE angles in fp64.
constexpr double kTwoPiHi = 6.283185307179586;
constexpr double kTwoPiLo = 2.4492935982947064e-16;
constexpr double kInvTwoPi = 0.15915494309189535;

__device__ __forceinline__ float2 rot_of(double angle) {
  const double k = rint(angle * kInvTwoPi);
  double r = fma(-k, kTwoPiHi, angle);
  r = fma(-k, kTwoPiLo, r);
  float s, c;
  sincosf(static_cast<float>(r), &s, &c);
  return make_float2(c, s);
}

template <int RANK>
struct AttLds {
  static constexpr int BS = RANK + 8;         // basis^T row stride (elements)
  static constexpr int W1S = kHeadDim + 8;    // W1 row stride
  static constexpr int W2S = kHidden + 8;     // W2 row stride
  static constexpr int W1_BYTES = kHidden * W1S * 2;
  static constexpr int W_BYTES = W1_BYTES + kHeadDim * W2S * 2;
  static constexpr int B_BYTES = kHeadDim * BS * 2;
  static constexpr int M_BYTES = (kAttWaves * 16 * kHeadDim + 2 * kAttWaves * 16) * 4;
  static constexpr int U_BYTES = (W_BYTES > B_BYTES ? (W_BYTES > M_BYTES ? W_BYTES : M_BYTES)
                                                   : (B_BYTES > M_BYTES ? B_BYTES : M_BYTES));
  alignas(16) unsigned char u[U_BYTES];
  float2 rope_off[kChunk][64];
  float2 rope_base[kAttChunksWG][64];
  float b1f[kHidden];
  float b2f[kHeadDim];
};

// Column permutation of W1 (over d) and W2 (over h) inside each block of 32:
// the MFMA slot 8*G + e of a k-step holds index 4*G + e (e < 4) or
// 16 + 4*G + (e - 4) (e >= 4), which is how the previous stage's accumulator
// rows sit in the lane.  Source 4-element group og -> slot group:
__device__ __forceinline__ int perm_group(int og) { return og < 4 ? 2 * og : 2 * (og - 4) + 1; }

// Stage a [rows][cols] bf16 matrix (global, dense) into LDS rows of stride
// `ld`, permuting 4-element groups inside every 32-column block.
__device__ __forceinline__ void stage_permuted(uint16_t* dst, int ld, const uint16_t* src,
                                               int rows, int cols, int tid) {
  const int per_row = cols / 8;  // 16-byte pieces per row
  for (int i = tid; i < rows * per_row; i += kAttWaves * 64) {
    const int r = i / per_row, p = i % per_row;
    const u32x4 v = *reinterpret_cast<const u32x4*>(src + (size_t)r * cols + 8 * p);
    const int blk = p >> 2, og0 = (p & 3) * 2;
    uint16_t* row = dst + r * ld + 32 * blk;
    *reinterpret_cast<u32x2*>(row + 4 * perm_group(og0)) = u32x2{v[0], v[1]};
    *reinterpret_cast<u32x2*>(row + 4 * perm_group(og0 + 1)) = u32x2{v[2], v[3]};
  }
}

// int4 x 8 (one 32-bit word, element e in bits 4e..4e+3) times scale -> bf16x8
__device__ __forceinline__ bf16x8 dequant8(uint32_t w, float scale) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int code = static_cast<int>(w << (28 - 4 * e)) >> 28;
    r[e] = (__bf16)(static_cast<float>(code) * scale);
  }
  return r;
}

template <int RANK, bool CI4, bool RI4>
__global__ __launch_bounds__(kAttWaves * 64) void attend_kernel(const AttendArgs a) {
  __shared__ AttLds<RANK> L;
  using Lds = AttLds<RANK>;
  constexpr int NKS = RANK / 32;   // k-steps of the reconstruction
  constexpr int NKB = RANK / 128;  // int4 k-blocks (4 k-steps, 16 B per lane)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, col = lane & 15;
  const int logical = xcd_logical_block(blockIdx.x, a.padded_total);
  if (logical >= a.total) return;
  const int bh = logical / a.n_split, split = logical % a.n_split;
  const int b = bh / a.hkv, h = bh % a.hkv;
  const int g = a.g;
  const size_t head = (size_t)b * a.hkv + h;
  const uint16_t* qh = a.q + ((size_t)b * a.hq + (size_t)h * g) * kHeadDim;

  f32x4 zacc[2];
  bf16x8 vb_hi[8], vb_lo[8];
  int nvalid;

  if (split < a.n_sel_tiles) {
    // ===================================================== selected chunks
    const int chunk0 = split * kAttChunksWG;
    const int nch = min(kAttChunksWG, a.k_eff - chunk0);
    const int32_t* selh = a.sel + head * (size_t)a.k_eff;
    nvalid = max(0, min(kAttTokWave, (nch - 4 * wave) * kChunk));
    // chunk id of selection slot i of this workgroup (clamped into the prefix)
    auto chunk_of = [&](int i) { return min(max(selh[chunk0 + min(i, nch - 1)], 0), a.n_chunks - 1); };
    int tok[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) tok[nt] = chunk_of(4 * wave + 2 * nt + (col >> 3)) * kChunk + (col & 7);

    // ---- issue the coefficient gather first (HBM), then stage LDS
    bf16x8 cv[CI4 ? 1 : NKS][2];
    u32x4 cq[CI4 ? NKB : 1][2];
    float csc[CI4 ? NKB : 1][2];
    if constexpr (!CI4) {
      const uint16_t* cb = static_cast<const uint16_t*>(a.coeff) + (size_t)b * a.prefix * RANK;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          cv[ks][nt] = load_bf16x8(cb + (size_t)tok[nt] * RANK + 32 * ks + 8 * grp);
    } else {
      const uint8_t* cb = static_cast<const uint8_t*>(a.coeff) + (size_t)b * a.prefix * (RANK / 2);
      const uint16_t* sb = a.coeff_scale + (size_t)b * a.prefix * (RANK / 32);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          cq[kb][nt] = *reinterpret_cast<const u32x4*>(cb + (size_t)tok[nt] * (RANK / 2) + 64 * kb + 16 * grp);
          csc[kb][nt] = f16_to_f32(sb[(size_t)tok[nt] * (RANK / 32) + 4 * kb + grp]);
        }
    }

    uint16_t* basisT = reinterpret_cast<uint16_t*>(L.u);
    {
      const uint16_t* src = a.basis + head * (size_t)kHeadDim * RANK;
      constexpr int per_row = RANK / 8;
      for (int i = tid; i < kHeadDim * per_row; i += kAttWaves * 64) {
        const int r = i / per_row, p = i % per_row;
        *reinterpret_cast<u32x4*>(basisT + r * Lds::BS + 8 * p) =
            *reinterpret_cast<const u32x4*>(src + (size_t)r * RANK + 8 * p);
      }
    }
    {  // RoPE rotations: base angle of every chunk start, offsets 0..7
      const int cs = tid >> 4, p0 = (tid & 15) * 4;
      const double pos = (double)chunk_of(cs) * kChunk;
#pragma unroll
      for (int p = p0; p < p0 + 4; ++p) L.rope_base[cs][p] = rot_of(pos * a.inv_freq[p]);
      const int i = tid >> 6, p = tid & 63;
      L.rope_off[i][p] = rot_of((double)i * a.inv_freq[p]);
    }
    __syncthreads();

    // ---- reconstruction: acc[nt][mt] = K_pre^T rows d = 16 mt + 4 grp + e
    f32x4 acc[2][8];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      bf16x8 bop[2];
      int r0;
      if constexpr (!CI4) {
        bop[0] = cv[ks][0];
        bop[1] = cv[ks][1];
        r0 = 32 * ks + 8 * grp;
      } else {
        const int kb = ks >> 2, kw = ks & 3;
        bop[0] = dequant8(cq[kb][0][kw], csc[kb][0]);
        bop[1] = dequant8(cq[kb][1][kw], csc[kb][1]);
        r0 = 128 * kb + 32 * grp + 8 * kw;
      }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const bf16x8 aop = load_bf16x8(basisT + (16 * mt + col) * Lds::BS + r0);
        acc[0][mt] = mfma16(aop, bop[0], acc[0][mt]);
        acc[1][mt] = mfma16(aop, bop[1], acc[1][mt]);
      }
    }
    const size_t row0 = head * (size_t)a.k_eff * kChunk + (size_t)(chunk0 + 4 * wave) * kChunk;
    if (a.kpre_out) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        if (16 * nt + col < nvalid)
#pragma unroll
          for (int mt = 0; mt < 8; ++mt)
            *reinterpret_cast<f32x4*>(a.kpre_out + (row0 + 16 * nt + col) * kHeadDim + 16 * mt + 4 * grp) = acc[nt][mt];
    }

    // ---- K_pre as the MLP1 operand (bf16), then RoPE in place
    bf16x8 kpre_b[2][4];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int s = 0; s < 4; ++s) kpre_b[nt][s] = pack8(acc[nt][2 * s], acc[nt][2 * s + 1]);

#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int cs = 4 * wave + 2 * nt + (col >> 3), i = col & 7;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int p = 16 * mt + 4 * grp + e;
          const float2 bs = L.rope_base[cs][p], of = L.rope_off[i][p];
          const float c = bs.x * of.x - bs.y * of.y;
          const float s = bs.y * of.x + bs.x * of.y;
          const float x1 = acc[nt][mt][e], x2 = acc[nt][mt + 4][e];
          acc[nt][mt][e] = x1 * c - x2 * s;
          acc[nt][mt + 4][e] = x2 * c + x1 * s;
        }
      }
    }
    if (a.kpost_out) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        if (16 * nt + col < nvalid)
#pragma unroll
          for (int mt = 0; mt < 8; ++mt)
            *reinterpret_cast<f32x4*>(a.kpost_out + (row0 + 16 * nt + col) * kHeadDim + 16 * mt + 4 * grp) = acc[nt][mt];
    }

    // ---- QK: z[t][j], K_post split hi + lo so the logits keep fp32 accuracy
    {
      bf16x8 qp[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        qp[s] = col < g ? load_bf16x4x2(qh + col * kHeadDim + 32 * s + 4 * grp,
                                        qh + col * kHeadDim + 32 * s + 16 + 4 * grp)
                        : zero_bf16x8();
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 hi = pack8(acc[nt][2 * s], acc[nt][2 * s + 1]);
          const bf16x8 lo = pack8_lo(acc[nt][2 * s], acc[nt][2 * s + 1], hi);
          z = mfma16(hi, qp[s], z);
          z = mfma16(lo, qp[s], z);
        }
        zacc[nt] = z;
      }
    }

    // ---- swap the LDS contents: basis out, W1 / W2 / biases in
    __syncthreads();
    uint16_t* w1s = reinterpret_cast<uint16_t*>(L.u);
    uint16_t* w2s = reinterpret_cast<uint16_t*>(L.u + Lds::W1_BYTES);
    stage_permuted(w1s, Lds::W1S, a.w1 + head * (size_t)kHidden * kHeadDim, kHidden, kHeadDim, tid);
    stage_permuted(w2s, Lds::W2S, a.w2 + head * (size_t)kHeadDim * kHidden, kHeadDim, kHidden, tid);
    if (tid < kHidden) L.b1f[tid] = bf16_to_f32(a.b1[head * kHidden + tid]);
    if (tid < kHeadDim) L.b2f[tid] = bf16_to_f32(a.b2[head * kHeadDim + tid]);
    __syncthreads();

    // ---- value MLP, 32 hidden units at a time; hid never leaves the VGPRs
    f32x4 vacc[2][8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) vacc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
    for (int hc = 0; hc < kHidden / 32; ++hc) {
      f32x4 hacc[2][2];
#pragma unroll
      for (int hm = 0; hm < 2; ++hm)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) hacc[hm][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
#pragma unroll
        for (int hm = 0; hm < 2; ++hm) {
          const bf16x8 aop = load_bf16x8(w1s + (32 * hc + 16 * hm + col) * Lds::W1S + 32 * s + 8 * grp);
          hacc[hm][0] = mfma16(aop, kpre_b[0][s], hacc[hm][0]);
          hacc[hm][1] = mfma16(aop, kpre_b[1][s], hacc[hm][1]);
        }
      }
#pragma unroll
      for (int hm = 0; hm < 2; ++hm)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float bias = L.b1f[32 * hc + 16 * hm + 4 * grp + e];
          hacc[hm][0][e] = gelu_fast(hacc[hm][0][e] + bias);
          hacc[hm][1][e] = gelu_fast(hacc[hm][1][e] + bias);
        }
      const bf16x8 ha0 = pack8(hacc[0][0], hacc[1][0]);
      const bf16x8 ha1 = pack8(hacc[0][1], hacc[1][1]);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const bf16x8 bop = load_bf16x8(w2s + (16 * nt + col) * Lds::W2S + 32 * hc + 8 * grp);
        vacc[0][nt] = mfma16(ha0, bop, vacc[0][nt]);
        vacc[1][nt] = mfma16(ha1, bop, vacc[1][nt]);
      }
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const float bias = L.b2f[16 * nt + col];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) vacc[mt][nt][e] += bias;
    }

    // ---- residual scatter-add: lane t (< 32) finds token t's stored row
    {
      int rn = -1;
      if (lane < nvalid) {
        const int cid = chunk_of(4 * wave + (lane >> 3));
        const int token = cid * kChunk + (lane & 7);
        const int32_t* off = a.res_off + head * (size_t)(a.n_chunks + 1);
        const int32_t* ridx = a.res_idx + head * (size_t)a.n_resid;
        const int o1 = min(off[cid + 1], a.n_resid);
        for (int i = max(off[cid], 0); i < o1; ++i)
          if (ridx[i] == token) rn = i;
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int nn = __shfl(rn, 16 * mt + 4 * grp + e);
          if (nn >= 0) {
            const size_t rrow = head * (size_t)a.n_resid + nn;
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) {
              const int d = 16 * nt + col;
              float r;
              if constexpr (!RI4) {
                r = bf16_to_f32(static_cast<const uint16_t*>(a.res_val)[rrow * kHeadDim + d]);
              } else {
                const uint32_t byte = static_cast<const uint8_t*>(a.res_val)[rrow * (kHeadDim / 2) + (d >> 1)];
                const int code = static_cast<int>(((byte >> (4 * (d & 1))) & 0xFu) ^ 8u) - 8;
                r = static_cast<float>(code) * f16_to_f32(a.res_scale[rrow * (kHeadDim / 32) + (d >> 5)]);
              }
              vacc[mt][nt][e] += r;
            }
          }
        }
    }
    if (a.vhat_out) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 16 * mt + 4 * grp + e;
          if (t < nvalid)
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) a.vhat_out[(row0 + t) * kHeadDim + 16 * nt + col] = vacc[mt][nt][e];
        }
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      vb_hi[nt] = pack8(vacc[0][nt], vacc[1][nt]);
      vb_lo[nt] = pack8_lo(vacc[0][nt], vacc[1][nt], vb_hi[nt]);
    }
  } else {
    // ========================================================= exact window
    const int w0 = (split - a.n_sel_tiles) * kAttTokWG + wave * kAttTokWave;
    nvalid = max(0, min(kAttTokWave, a.window - w0));
    const uint16_t* kw = a.win_k + head * (size_t)a.window * kHeadDim;
    const uint16_t* vw = a.win_v + head * (size_t)a.window * kHeadDim;
    bf16x8 qn[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      qn[s] = col < g ? load_bf16x8(qh + col * kHeadDim + 32 * s + 8 * grp) : zero_bf16x8();
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int t = min(w0 + 16 * nt + col, a.window - 1);
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) z = mfma16(load_bf16x8(kw + (size_t)t * kHeadDim + 32 * s + 8 * grp), qn[s], z);
      zacc[nt] = z;
    }
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = min(w0 + 16 * (e >> 2) + 4 * grp + (e & 3), a.window - 1);
        v[e] = __builtin_bit_cast(__bf16, vw[(size_t)t * kHeadDim + 16 * nt + col]);
      }
      vb_hi[nt] = v;
      vb_lo[nt] = zero_bf16x8();
    }
  }

  // ============================================= softmax + PV (both roles)
  float p[2][4];
  float m = -__builtin_huge_valf();
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * nt + 4 * grp + e;
      p[nt][e] = t < nvalid ? zacc[nt][e] * a.scale_log2 : -__builtin_huge_valf();
      m = fmaxf(m, p[nt][e]);
    }
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  const float msafe = m == -__builtin_huge_valf() ? 0.f : m;
  float lsum = 0.f;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[nt][e] = __builtin_amdgcn_exp2f(p[nt][e] - msafe);
      lsum += p[nt][e];
    }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  const bf16x8 pa = pack8(f32x4{p[0][0], p[0][1], p[0][2], p[0][3]},
                          f32x4{p[1][0], p[1][1], p[1][2], p[1][3]});
  f32x4 oacc[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) {
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
    o = mfma16(pa, vb_hi[nt], o);
    o = mfma16(pa, vb_lo[nt], o);
    oacc[nt] = o;
  }

  // ======================================== merge the 8 waves, write partial
  __syncthreads();
  float* mo = reinterpret_cast<float*>(L.u);
  float* ml = mo + kAttWaves * 16 * kHeadDim;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
#pragma unroll
    for (int e = 0; e < 4; ++e) mo[(wave * 16 + 4 * grp + e) * kHeadDim + 16 * nt + col] = oacc[nt][e];
  if (grp == 0) {
    ml[wave * 16 + col] = m;
    ml[kAttWaves * 16 + wave * 16 + col] = lsum;
  }
  __syncthreads();
  float* part = a.part + ((head * a.n_split + split) * (size_t)g) * kPartStride;
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

template <int RANK>
static hipError_t launch_rank(const AttendArgs& a, bool ci4, bool ri4, hipStream_t st) {
  const dim3 grid(a.padded_total), block(kAttWaves * 64);
  if (!ci4 && !ri4) hipLaunchKernelGGL((attend_kernel<RANK, false, false>), grid, block, 0, st, a);
  else if (ci4 && ri4) hipLaunchKernelGGL((attend_kernel<RANK, true, true>), grid, block, 0, st, a);
  else if (ci4) hipLaunchKernelGGL((attend_kernel<RANK, true, false>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((attend_kernel<RANK, false, true>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attend(const AttendArgs& a, int rank, bool ci4, bool ri4, hipStream_t st) {
  if (a.total == 0) return hipSuccess;
  switch (rank) {
    case 128: return launch_rank<128>(a, ci4, ri4, st);
    case 256: return launch_rank<256>(a, ci4, ri4, st);
    case 512: return launch_rank<512>(a, ci4, ri4, st);
    default: break;
  }
  // rank 64: the int4 path needs rank % 128 == 0 and is not instantiated here
  if (ci4) return hipErrorInvalidValue;
  const dim3 grid(a.padded_total), block(kAttWaves * 64);
  if (ri4) hipLaunchKernelGGL((attend_kernel<64, false, true>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((attend_kernel<64, false, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split merge: log-sum-exp combination of the per-workgroup partial states
// (m in log2 units, l, o) of each query head, written as bf16.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void merge_kernel(const float* __restrict__ part,
                                                    uint16_t* __restrict__ out, int hkv, int g,
                                                    int n_split) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const size_t head = (size_t)b * hkv + h;
  for (int j = 0; j < g; ++j) {
    const float* p = part + (head * n_split * (size_t)g + j) * kPartStride;
    const size_t st = (size_t)g * kPartStride;
    float M = -__builtin_huge_valf();
    for (int s = 0; s < n_split; ++s) M = fmaxf(M, p[s * st]);
    float lt = 0.f, o = 0.f;
    for (int s = 0; s < n_split; ++s) {
      const float ms = p[s * st];
      const float sc = ms == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(ms - M);
      lt += p[s * st + 1] * sc;
      o += p[s * st + 2 + d] * sc;
    }
    const __bf16 r = (__bf16)(o / lt);
    out[(head * g + j) * kHeadDim + d] = __builtin_bit_cast(uint16_t, r);
  }
}

hipError_t launch_merge(const float* part, uint16_t* out, int nb, int hkv, int g, int n_split,
                        hipStream_t st) {
  hipLaunchKernelGGL(merge_kernel, dim3(hkv, nb), dim3(kHeadDim), 0, st, part, out, hkv, g, n_split);
  return hipGetLastError();
}

}  // namespace lowram
