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
// The exact recent window is attended by extra workgroups of the same grid;
// a separate merge kernel combines the partial states of each head.
//
// Layout of the work.  A workgroup is 4 waves; each wave owns 32 tokens
// (4 chunks) and runs every stage on them with v_mfma_f32_16x16x32_bf16.
// Tokens are the MFMA N dimension throughout, so each stage's accumulator
// layout is the next stage's operand layout (up to a fixed permutation of
// the contraction index, applied to the other operand instead):
//   recon   D[d][t]  = basis^T[d][r] (LDS)   x C[t][r] (global -> VGPR)
//   RoPE    lane-local: pair (i, i+64) sits in m-tiles mt and mt+4
//   QK      D[t][j]  = K_post[t][d] (VGPR, bf16)  x q[j][d]
//   MLP1    D[h][t]  = W1[h][d] (LDS)        x K_pre[t][d] (VGPR)
//   MLP2    D[t][d]  = hid[t][h] (VGPR)      x W2[d][h] (LDS)
//   PV      D[j][d]  = p[j][t] (VGPR)        x V[t][d] (VGPR, bf16)
// The operands shared by the 4 waves pass through one 64 KiB LDS buffer in
// four stages (basis r < 256, basis r >= 256, W1, W2), so a workgroup needs
// under 80 KiB and two workgroups share a CU: one stages or waits on the
// coefficient gather while the other runs MFMA.
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

constexpr int kBuf = 65536;  // bytes of the staged operand buffer

struct AttLds {
  alignas(16) unsigned char buf[kBuf];
  float2 rope_off[kChunk][64];
  float2 rope_base[kAttChunksWG][64];
  float b1f[kHidden];
  float b2f[kHeadDim];
};

// Staged matrices keep dense rows of NP 16-byte pieces; piece p of row r
// sits at p ^ (r & mask) with mask = 15 (7 for 8-piece rows), so the 16
// rows one MFMA operand read touches fall on different LDS banks.
template <int NP>
__device__ __forceinline__ constexpr int swz(int row, int piece) {
  return piece ^ (row & (NP >= 16 ? 15 : 7));
}

// Column permutation of W1 (over d) and W2 (over h) inside each block of 32:
// the MFMA slot 8*G + e of a k-step holds index 4*G + e (e < 4) or
// 16 + 4*G + (e - 4) (e >= 4), which is how the previous stage's accumulator
// rows sit in the lane.  Source 4-element group og -> slot group:
__device__ __forceinline__ constexpr int perm_group(int og) { return og < 4 ? 2 * og : 2 * (og - 4) + 1; }

// Stage columns [c0, c0 + 8*NP) of the matrix behind `src` (row stride LD
// elements) into dst (ROWS rows of NP pieces).  Thread t copies piece t % NP
// of rows t / NP + u * (256 / NP): a buffer load (one lane offset, the pass
// as SGPR offset) and an LDS store at a lane base plus an immediate.
template <int ROWS, int NP, int LD>
__device__ __forceinline__ void stage_plain(unsigned char* dst, __amdgpu_buffer_rsrc_t src, int c0, int tid) {
  constexpr int RSTEP = kAttWaves * 64 / NP;
  const int r0 = tid / NP, p = tid % NP;
  const uint32_t goff = (uint32_t)(r0 * LD + c0 + 8 * p) * 2;
#pragma unroll
  for (int u = 0; u < ROWS / RSTEP; ++u) {
    const int r = r0 + u * RSTEP;
    const u32x4 v = buffer_ld16(src, goff, u * RSTEP * LD * 2);
    *reinterpret_cast<u32x4*>(dst + (r * NP + swz<NP>(r, p)) * 16) = v;
  }
}

// As stage_plain for 16-piece rows, with the 4-element group permutation
// inside every 32-column block (W1 over d, W2 over h).
template <int ROWS, int LD>
__device__ __forceinline__ void stage_perm16(unsigned char* dst, __amdgpu_buffer_rsrc_t src, int c0, int tid) {
  constexpr int NP = 16, RSTEP = kAttWaves * 64 / NP;  // 16 rows per pass keep r & 15
  const int r0 = tid / NP, p = tid % NP;
  const int blk = p >> 2, og0 = (p & 3) * 2;
  const int sg0 = perm_group(og0), sg1 = perm_group(og0 + 1);
  const int o0 = (r0 * NP + ((4 * blk + (sg0 >> 1)) ^ r0)) * 16 + 8 * (sg0 & 1);
  const int o1 = (r0 * NP + ((4 * blk + (sg1 >> 1)) ^ r0)) * 16 + 8 * (sg1 & 1);
  const uint32_t goff = (uint32_t)(r0 * LD + c0 + 8 * p) * 2;
#pragma unroll
  for (int u = 0; u < ROWS / RSTEP; ++u) {
    const u32x4 v = buffer_ld16(src, goff, u * RSTEP * LD * 2);
    *reinterpret_cast<u32x2*>(dst + o0 + u * RSTEP * NP * 16) = u32x2{v[0], v[1]};
    *reinterpret_cast<u32x2*>(dst + o1 + u * RSTEP * NP * 16) = u32x2{v[2], v[3]};
  }
}

__device__ __forceinline__ bf16x8 lds16(const unsigned char* base, int off) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + off));
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
__global__ __launch_bounds__(kAttWaves * 64, 2) void attend_kernel(const AttendArgs a) {
  __shared__ AttLds L;
  constexpr int NKS = RANK / 32;         // k-steps of the reconstruction
  constexpr int NKB = RANK / 128;        // int4 k-blocks (4 k-steps, 16 B per lane)
  constexpr int RB = RANK < 256 ? RANK : 256;  // basis columns per staged half
  constexpr int NHALF = RANK / RB;
  constexpr int KS_HALF = RB / 32;
  constexpr int NPB = RB / 8;                  // 16-byte pieces per staged basis row
  constexpr int W2OFF = (kHidden / 2) * kHeadDim * 2;  // byte offset of the W2 half in buf

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, col = lane & 15;
  const int logical = xcd_logical_block(blockIdx.x, a.padded_total);
  if (logical >= a.total) return;
  const int bh = logical / a.n_split, split = logical % a.n_split;
  const int b = bh / a.hkv, h = bh % a.hkv;
  const int g = a.g;
  const size_t head = (size_t)b * a.hkv + h;
  const uint16_t* qh = a.q + ((size_t)b * a.hq + (size_t)h * g) * kHeadDim;
  unsigned char* buf = L.buf;

  f32x4 zacc[2];
  bf16x8 vb[8];
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

    // Per-lane byte offsets of the swizzled operand reads.  A read of row
    // 16*m + col, piece 4*k + grp lands at piece (4*k + grp) ^ (col & mask)
    // = 4*(k ^ (col >> 2)) + (grp ^ (col & 3)) of that row (mask 15); the
    // int4 basis read of piece 4*grp + k lands at 4*(grp ^ (col >> 2)) +
    // (k ^ (col & 3)).  Row and 16-piece-block terms are immediates.
    const int chi = col >> 2, clo = col & 3;
    const int chib = NPB >= 16 ? chi : (chi & 1);
    auto pbw = [&](int k) { return col * 256 + 16 * (4 * (k ^ chi) + (grp ^ clo)); };
    auto pbb = [&](int k) { return col * (NPB * 16) + 16 * (4 * (k ^ chib) + (grp ^ clo)); };
    auto pbi = [&](int k) { return col * (NPB * 16) + 16 * (4 * (grp ^ chib) + (k ^ clo)); };

    // ---- the coefficient gather goes out first (HBM), one basis half at a
    //      time: half hb+1 is in flight while half hb is multiplied
    bf16x8 cv[CI4 ? 1 : NKS][2];
    u32x4 cq[CI4 ? NKB : 1][2];
    float csc[CI4 ? NKB : 1][2];
    auto gather_half = [&](int hb) {
      if constexpr (!CI4) {
        const uint16_t* cb = static_cast<const uint16_t*>(a.coeff) + (size_t)b * a.prefix * RANK;
#pragma unroll
        for (int kl = 0; kl < KS_HALF; ++kl)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const int ks = hb * KS_HALF + kl;
            cv[ks][nt] = load_bf16x8(cb + (size_t)tok[nt] * RANK + 32 * ks + 8 * grp);
          }
      } else {
        const uint8_t* cb = static_cast<const uint8_t*>(a.coeff) + (size_t)b * a.prefix * (RANK / 2);
        const uint16_t* sb = a.coeff_scale + (size_t)b * a.prefix * (RANK / 32);
#pragma unroll
        for (int kl = 0; kl < NKB / NHALF; ++kl)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) {
            const int kb = hb * (NKB / NHALF) + kl;
            cq[kb][nt] = *reinterpret_cast<const u32x4*>(cb + (size_t)tok[nt] * (RANK / 2) + 64 * kb + 16 * grp);
            csc[kb][nt] = f16_to_f32(sb[(size_t)tok[nt] * (RANK / 32) + 4 * kb + grp]);
          }
      }
    };
    gather_half(0);
    // ---- residual descriptor of token `lane` (< 32)'s chunk: one load,
    //      consumed only after the MLP
    uint32_t rdesc = 0;
    if (lane < nvalid) rdesc = a.res_desc[head * (size_t)a.n_chunks + chunk_of(4 * wave + (lane >> 3))];

    const __amdgpu_buffer_rsrc_t basis = buffer_rsrc(a.basis + head * (size_t)kHeadDim * RANK, kHeadDim * RANK * 2);
    stage_plain<kHeadDim, NPB, RANK>(buf, basis, 0, tid);
    __syncthreads();

    // ---- reconstruction: acc[nt][mt] = K_pre^T rows d = 16 mt + 4 grp + e
    f32x4 acc[2][8];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hb = 0; hb < NHALF; ++hb) {
      if (hb > 0) {
        __syncthreads();
        stage_plain<kHeadDim, NPB, RANK>(buf, basis, RB * hb, tid);
        __syncthreads();
      }
      if (hb + 1 < NHALF) gather_half(hb + 1);
#pragma unroll
      for (int kl = 0; kl < KS_HALF; ++kl) {
        const int ks = hb * KS_HALF + kl;
        bf16x8 bop[2];
        int off;
        if constexpr (!CI4) {
          bop[0] = cv[ks][0];
          bop[1] = cv[ks][1];
          off = pbb(kl & 3) + 256 * (kl >> 2);  // piece 4*kl + grp of the half
        } else {
          const int kb = ks >> 2, kw = ks & 3;
          bop[0] = dequant8(cq[kb][0][kw], csc[kb][0]);
          bop[1] = dequant8(cq[kb][1][kw], csc[kb][1]);
          off = pbi(kw) + 256 * (kb & 1);       // piece 16*(kb&1) + 4*grp + kw
        }
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
          const bf16x8 aop = lds16(buf, off + mt * 16 * NPB * 16);
          acc[0][mt] = mfma16(aop, bop[0], acc[0][mt]);
          acc[1][mt] = mfma16(aop, bop[1], acc[1][mt]);
        }
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

    // ---- K_pre as the MLP1 operand (bf16)
    bf16x8 kpre_b[2][4];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int s = 0; s < 4; ++s) kpre_b[nt][s] = pack8(acc[nt][2 * s], acc[nt][2 * s + 1]);

    // ---- RoPE rotations of this workgroup's tokens: base angle of every
    //      chunk start (fp64-reduced) and the offsets 0..7 inside a chunk.
    //      The basis is no longer read: W1 / biases go to LDS meanwhile.
    {
      const int cs = tid >> 4, p0 = (tid & 15) * 4;
      const double pos = (double)chunk_of(cs) * kChunk;
#pragma unroll
      for (int p = p0; p < p0 + 4; ++p) L.rope_base[cs][p] = rot_of(pos * a.inv_freq[p]);
      const int i = tid >> 5, q0 = (tid & 31) * 2;
#pragma unroll
      for (int p = q0; p < q0 + 2; ++p) L.rope_off[i][p] = rot_of((double)i * a.inv_freq[p]);
    }
    __syncthreads();
    const __amdgpu_buffer_rsrc_t w1h = buffer_rsrc(a.w1 + head * (size_t)kHidden * kHeadDim, kHidden * kHeadDim * 2);
    const __amdgpu_buffer_rsrc_t w2h = buffer_rsrc(a.w2 + head * (size_t)kHeadDim * kHidden, kHeadDim * kHidden * 2);
    stage_perm16<kHidden / 2, kHeadDim>(buf, w1h, 0, tid);             // W1 rows h < 128
    stage_perm16<kHeadDim, kHidden>(buf + W2OFF, w2h, 0, tid);         // W2 columns h < 128
    L.b1f[tid] = bf16_to_f32(a.b1[head * kHidden + tid]);
    if (tid < kHeadDim) L.b2f[tid] = bf16_to_f32(a.b2[head * kHeadDim + tid]);

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

    // ---- QK: z[t][j] with K_post rounded to bf16 (2^-9 relative per entry)
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
        for (int s = 0; s < 4; ++s) z = mfma16(pack8(acc[nt][2 * s], acc[nt][2 * s + 1]), qp[s], z);
        zacc[nt] = z;
      }
    }

    // ---- value MLP, 32 hidden units at a time: MLP1 chunk (b1 as the
    //      accumulator's initial value) -> GELU -> bf16 -> MLP2 accumulate.
    //      Hidden units [0, 128) use the W1/W2 halves staged above, then the
    //      buffer is refilled with the halves of units [128, 256).
    __syncthreads();
    f32x4 vacc[2][8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const float bias = L.b2f[16 * nt + col];
      vacc[0][nt] = f32x4{bias, bias, bias, bias};
      vacc[1][nt] = vacc[0][nt];
    }
#pragma unroll
    for (int hp = 0; hp < 2; ++hp) {
      if (hp > 0) {
        __syncthreads();
        stage_perm16<kHidden / 2, kHeadDim>(buf, w1h, (kHidden / 2) * kHeadDim, tid);
        stage_perm16<kHeadDim, kHidden>(buf + W2OFF, w2h, kHidden / 2, tid);
        __syncthreads();
      }
#pragma unroll 1
      for (int hl = 0; hl < 4; ++hl) {
        const int hc = 4 * hp + hl;
        f32x4 hacc[2][2];
#pragma unroll
        for (int hm = 0; hm < 2; ++hm) {
          const f32x4 bias = *reinterpret_cast<const f32x4*>(&L.b1f[32 * hc + 16 * hm + 4 * grp]);
          hacc[hm][0] = bias;
          hacc[hm][1] = bias;
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
          for (int hm = 0; hm < 2; ++hm) {
            const bf16x8 aop = lds16(buf, pbw(s) + (32 * hl + 16 * hm) * 256);
            hacc[hm][0] = mfma16(aop, kpre_b[0][s], hacc[hm][0]);
            hacc[hm][1] = mfma16(aop, kpre_b[1][s], hacc[hm][1]);
          }
        }
#pragma unroll
        for (int hm = 0; hm < 2; ++hm)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int e = 0; e < 4; ++e) hacc[hm][nt][e] = gelu_fast(hacc[hm][nt][e]);
        const bf16x8 ha0 = pack8(hacc[0][0], hacc[1][0]);
        const bf16x8 ha1 = pack8(hacc[0][1], hacc[1][1]);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
          const bf16x8 bop = lds16(buf, W2OFF + pbw(hl) + 16 * nt * 256);
          vacc[0][nt] = mfma16(ha0, bop, vacc[0][nt]);
          vacc[1][nt] = mfma16(ha1, bop, vacc[1][nt]);
        }
      }
    }

    // ---- residual scatter-add: token `lane` has a stored row iff its bit is
    //      set; the row is the chunk's first row plus the set bits below it
    int rn = -1;
    {
      const int i = lane & 7;
      if ((rdesc >> i) & 1u) {
        rn = (int)(rdesc >> 8) + __popc(rdesc & ((1u << i) - 1u) & 0xFFu);
        rn = min(rn, a.n_resid - 1);
      }
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
      vb[nt] = pack8(vacc[0][nt], vacc[1][nt]);
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
      vb[nt] = v;
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
    o = mfma16(pa, vb[nt], o);
    oacc[nt] = o;
  }

  // ======================================== merge the 4 waves, write partial
  __syncthreads();
  float* mo = reinterpret_cast<float*>(L.buf);
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
  float* part = a.part + (head * (size_t)a.n_split + split) * g * kPartStride;
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
// Split merge: one workgroup per (sequence, KV head).  The per-split weights
// w[s][j] = exp2(m_sj - M_j) / L_j go to LDS first, then every thread sums
// its (j, d) outputs over the splits with independent loads.
// ---------------------------------------------------------------------------
constexpr int kMergeThreads = 512;
constexpr int kMergeMaxSplit = 1024;

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const float* __restrict__ part,
                                                              uint16_t* __restrict__ out, int hkv,
                                                              int g, int n_split) {
  __shared__ float wgt[kMergeMaxSplit * 4];
  __shared__ float inv_l[16];
  const int tid = threadIdx.x;
  const size_t head = (size_t)blockIdx.y * hkv + blockIdx.x;
  const float* ph = part + head * (size_t)n_split * g * kPartStride;
  const size_t st = (size_t)g * kPartStride;
  uint16_t* oh = out + head * (size_t)g * kHeadDim;
  const int ns = n_split;  // n_split * min(g, 16) <= 4096 is checked at launch
  for (int j0 = 0; j0 < g; j0 += 16) {
    const int gj = min(16, g - j0);
    // M_j: one wave per query head
    const int wave = tid >> 6, lane = tid & 63;
    for (int j = wave; j < gj; j += kMergeThreads / 64) {
      float m = -__builtin_huge_valf();
      for (int s = lane; s < ns; s += 64) m = fmaxf(m, ph[s * st + (j0 + j) * kPartStride]);
      for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
      float l = 0.f;
      for (int s = lane; s < ns; s += 64) {
        const float ms = ph[s * st + (j0 + j) * kPartStride];
        const float w = ms == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(ms - m);
        wgt[s * gj + j] = w;
        l += w * ph[s * st + (j0 + j) * kPartStride + 1];
      }
      for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
      if (lane == 0) inv_l[j] = 1.f / l;
    }
    __syncthreads();
    for (int idx = tid; idx < gj * kHeadDim; idx += kMergeThreads) {
      const int j = idx / kHeadDim, d = idx % kHeadDim;
      const float* p = ph + (j0 + j) * kPartStride + 2 + d;
      float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
      int s = 0;
      for (; s + 4 <= ns; s += 4) {
        const float a0 = p[s * st], a1 = p[(s + 1) * st], a2 = p[(s + 2) * st], a3 = p[(s + 3) * st];
        o0 += a0 * wgt[s * gj + j];
        o1 += a1 * wgt[(s + 1) * gj + j];
        o2 += a2 * wgt[(s + 2) * gj + j];
        o3 += a3 * wgt[(s + 3) * gj + j];
      }
      for (; s < ns; ++s) o0 += p[s * st] * wgt[s * gj + j];
      const __bf16 r = (__bf16)(((o0 + o1) + (o2 + o3)) * inv_l[j]);
      oh[(j0 + j) * kHeadDim + d] = __builtin_bit_cast(uint16_t, r);
    }
    __syncthreads();
  }
}

hipError_t launch_merge(const float* part, uint16_t* out, int nb, int hkv, int g, int n_split,
                        hipStream_t st) {
  if ((long long)n_split * (g < 16 ? g : 16) > kMergeMaxSplit * 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(merge_kernel, dim3(hkv, nb), dim3(kMergeThreads), 0, st, part, out, hkv, g, n_split);
  return hipGetLastError();
}

}  // namespace lowram
