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
// is the next stage's operand without any data movement:
//   recon   D[d][t]  = basis^T[d][r] (LDS)   x C[t][r] (global -> VGPR)
//   RoPE    lane-local: pair (i, i+64) sits in m-tiles mt and mt+4
//   QK      D[t][j]  = K_post[t][d] (VGPR, bf16)  x q[j][d]
//   MLP1    D[h][t]  = W1[h][d] (LDS)        x K_pre[t][d] (VGPR)
//   MLP2    D[t][d]  = hid[t][h] (VGPR)      x W2[d][h] (LDS)
//   PV      D[j][d]  = p[j][t] (VGPR)        x V[t][d] (VGPR, bf16)
// An accumulator tile holds rows 4*(lane/16) + e (e < 4) of each 16-row
// m-tile, while the next product's operand wants 8 consecutive k per lane.
// Staging the basis (and W1) rows in the order pi(16 m + 4 g + e) =
// 32 (m / 2) + 8 g + 4 (m % 2) + e makes the two m-tiles 2s and 2s + 1 of
// a lane hold exactly k = 32 s + 8 g .. 32 s + 8 g + 7, in natural order.
//
// Pipeline.  The shared operands (basis in r-slices of 64, then W1/W2 in
// slices of 32 hidden units) stream through two 16 KiB LDS buffers, one
// stage per step, 16 steps at rank 512.  Every load is an ordinary vector
// load: a stage is loaded into registers two steps before it is needed and
// written to LDS at the end of the previous step, and each wave's
// coefficient gather runs three steps ahead.  Loads are issued in the order
// they are consumed, so the in-order vmcnt waits never hold a step on data
// it does not need.  The selected tokens' residual rows go to LDS as one
// dense tile (zero rows where a token has none) after the last stage.
#include "attend_ops.h"
#include "common.h"
#include "internal.h"
#include "window.h"

namespace lowram {

struct AttLds {
  // stage ring; then the residual tile (one row of kResRow per token); then the wave merge
  alignas(16) unsigned char buf[2 * kStage > 8 * kAttChunksWG * kResRow ? 2 * kStage : 8 * kAttChunksWG * kResRow];
  float2 rope_off[kChunk][65];  // padded: the 8 offsets of one frequency fall on distinct banks
  float2 rope_base[kAttChunksWG][64];
  float b1f[kHidden];
  float b2f[kHeadDim];
  float ml[2 * kAttWaves * 16];
  uint32_t rdesc[kAttChunksWG];
  alignas(16) uint16_t qs[16][kHeadDim];  // this KV head's query rows
};

// Workgroups per CU the register budget is sized for, and how many stages
// ahead each wave's coefficient gather runs (compile-time tunables).
#ifndef LOWRAM_ATT_WG_PER_CU
#define LOWRAM_ATT_WG_PER_CU (kAttSelNT >= 4 ? 1 : 2)
#endif
#ifndef LOWRAM_ATT_GATHER_AHEAD
#define LOWRAM_ATT_GATHER_AHEAD 2
#endif
#ifndef LOWRAM_ATT_STAGE_AHEAD
#define LOWRAM_ATT_STAGE_AHEAD 2
#endif

// STAGES: also write the rebuilt keys and the per-token values (for stage
// parity checks).  The per-token values need the value MLP's second layer
// per token, which the output path never forms (see the value section).
template <int RANK, bool CI4, bool RI4, bool STAGES>
__global__ __launch_bounds__(kAttWaves * 64, LOWRAM_ATT_WG_PER_CU) void attend_kernel(const AttendArgs a) {
  __shared__ AttLds L;
  constexpr int NR = RANK / 64;          // basis stages (64 columns of r each)
  constexpr int NM = kHidden / 32;       // MLP stages (32 hidden units each)
  constexpr int NS = NR + NM;
  constexpr int LG = LOWRAM_ATT_GATHER_AHEAD;
  constexpr int SL = LOWRAM_ATT_STAGE_AHEAD;  // stage s + SL is loaded at the top of step s
  constexpr int NT = kAttSelNT;               // 16-token tiles per wave (selected chunks)
  constexpr int TOKW = 16 * NT;               // tokens per wave
  constexpr int CPW = TOKW / kChunk;          // chunks per wave

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, col = lane & 15;
  const int logical = xcd_logical_block(blockIdx.x, a.padded_total);
  if (logical >= a.total) return;
  // this launch covers splits [split_base, split_base + n_split_launch) of every head
  const int bh = logical / a.n_split_launch, split = a.split_base + logical % a.n_split_launch;
  const int b = bh / a.hkv, h = bh % a.hkv;
  const int g = a.g;
  const size_t head = (size_t)b * a.hkv + h;
  // cache arrays: per sequence, or one context shared by every query (stride 0)
  const int cseq = b * a.cache_bmul;
  const size_t chead = (size_t)cseq * a.hkv + h;
  const uint16_t* qh = a.q + ((size_t)b * a.hq + (size_t)h * g) * kHeadDim;
  unsigned char* buf = L.buf;

  // every role ends with this wave's softmax state of query head j = col and
  // o^T[d][j] in rows d = 16 nd + 4 grp + e of oacc[nd]
  f32x4 oacc[8];
  float wm, wl;

  if (split < a.n_sel_tiles) {
    // ===================================================== selected chunks
    const int chunk0 = split * kAttChunksWG;
    const int nch = min(kAttChunksWG, a.k_eff - chunk0);
    const int32_t* selh = a.sel + head * (size_t)a.k_eff;
    const int nvalid = max(0, min(TOKW, (nch - CPW * wave) * kChunk));
    // chunk id of selection slot i of this workgroup (clamped into the prefix)
    auto chunk_of = [&](int i) { return min(max(selh[chunk0 + min(i, nch - 1)], 0), a.n_chunks - 1); };
    // ---- operand stream: stage s < NR is basis columns [64 s, 64 s + 64)
    //      (128 rows in pi order, two rows per 256-byte line); stage NR + c
    //      is W1 rows [32 c, 32 c + 32) (pi order, 8 KiB) then W2 columns
    //      [32 c, 32 c + 32) (natural, four rows per line, 8 KiB).  Pieces
    //      are XOR-swizzled inside each 256-byte line by the line index.
    const __amdgpu_buffer_rsrc_t bas = buffer_rsrc(a.basis + chead * (size_t)kHeadDim * RANK, kHeadDim * RANK * 2);
    const __amdgpu_buffer_rsrc_t w1r = buffer_rsrc(a.w1 + chead * (size_t)kHidden * kHeadDim, kHidden * kHeadDim * 2);
    const __amdgpu_buffer_rsrc_t w2r = buffer_rsrc(a.w2 + chead * (size_t)kHeadDim * kHidden, kHeadDim * kHidden * 2);
    // basis: load u covers rows 32 u + r0 (r0 = tid / 8), piece tid % 8
    const int r0 = tid >> 3, pb = tid & 7;
    const uint32_t bas_goff = (uint32_t)((row_perm32(r0) * RANK + 8 * pb) * 2);
    const int bas_loff = (r0 >> 1) * 256 + ((((r0 & 1) << 3) | pb) ^ ((r0 >> 1) & 15)) * 16;
    // W1: load u < 2 covers pi rows 16 u + tid / 16, piece tid % 16
    const int w1row = tid >> 4, w1p = tid & 15;
    const uint32_t w1_goff = (uint32_t)(((8 * ((w1row >> 2) & 3) + (w1row & 3)) * kHeadDim + 8 * w1p) * 2);
    const int w1_loff = w1row * 256 + (w1p ^ (w1row & 15)) * 16;
    // W2: load u in {2, 3} covers rows 64 (u - 2) + tid / 4, piece tid % 4
    const uint32_t w2_goff = (uint32_t)(((tid >> 2) * kHidden + 8 * (tid & 3)) * 2);
    const int w2_loff = 8192 + (tid >> 4) * 256 + ((tid & 15) ^ ((tid >> 4) & 15)) * 16;

    auto stage_load = [&](int s, u32x4 (&r)[kStageLd]) {
      if (s < NR) {
#pragma unroll
        for (int u = 0; u < kStageLd; ++u) r[u] = buffer_ld16(bas, bas_goff, (32 * u * RANK + 64 * s) * 2);
      } else {
        const int c = s - NR;
#pragma unroll
        for (int u = 0; u < 2; ++u) r[u] = buffer_ld16(w1r, w1_goff, (32 * c + 4 * u) * kHeadDim * 2);
#pragma unroll
        for (int u = 2; u < 4; ++u) r[u] = buffer_ld16(w2r, w2_goff, ((u - 2) * 64 * kHidden + 32 * c) * 2);
      }
    };
    auto stage_store = [&](int s, const u32x4 (&r)[kStageLd]) {
      unsigned char* dst = L.buf + (s & 1) * kStage;
      if (s < NR) {
#pragma unroll
        for (int u = 0; u < kStageLd; ++u) *reinterpret_cast<u32x4*>(dst + bas_loff + 4096 * u) = r[u];
      } else {
#pragma unroll
        for (int u = 0; u < 2; ++u) *reinterpret_cast<u32x4*>(dst + w1_loff + 4096 * u) = r[u];
#pragma unroll
        for (int u = 2; u < 4; ++u) *reinterpret_cast<u32x4*>(dst + w2_loff + 4096 * (u - 2)) = r[u];
      }
    };

    int tok[NT];  // this lane's token rows (set in the prologue)

    // ---- coefficient gather of stage s (< NR): k-steps 2 s, 2 s + 1
    bf16x8 cv[CI4 ? 1 : NR][2][NT];
    u32x2 cq[CI4 ? NR : 1][NT];
    float csc[CI4 ? NR : 1][NT];
    auto gather = [&](int s) {
      if constexpr (!CI4) {
        const uint16_t* cb = static_cast<const uint16_t*>(a.coeff) + (size_t)cseq * a.prefix_cap * RANK;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            cv[s][ks][nt] = load_bf16x8(cb + (size_t)tok[nt] * RANK + 64 * s + 32 * ks + 8 * grp);
      } else {
        // 16 codes r = 64 s + 16 grp .. + 15 and their group scale
        const uint8_t* cb = static_cast<const uint8_t*>(a.coeff) + (size_t)cseq * a.prefix_cap * (RANK / 2);
        const uint16_t* sb = a.coeff_scale + (size_t)cseq * a.prefix_cap * (RANK / 32);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          cq[s][nt] = *reinterpret_cast<const u32x2*>(cb + (size_t)tok[nt] * (RANK / 2) + 32 * s + 8 * grp);
          csc[s][nt] = f16_to_f32(sb[(size_t)tok[nt] * (RANK / 32) + 2 * s + (grp >> 1)]);
        }
      }
    };

    // ---- prologue.  One memory round trip before the stream starts: the
    //      first stages, biases, queries, RoPE frequencies and this
    //      workgroup's chunk ids are loaded together and waited for at once;
    //      then the gathers (which need the chunk ids) and the residual
    //      descriptors go out.
    u32x4 sreg[NS + SL][kStageLd];
#pragma unroll
    for (int s = 0; s < SL && s < NS; ++s) stage_load(s, sreg[s]);
    // b1 in the order the value section reads it: unit 32 c + row_perm32(p) at 32 c + p
    const uint16_t b1v = a.b1[chead * kHidden + (tid & ~31) + row_perm32(tid & 31)];
    const uint16_t b2v = tid < kHeadDim ? a.b2[chead * kHeadDim + tid] : 0;
    const u32x4 qv = tid < 16 * g ? *reinterpret_cast<const u32x4*>(qh + 8 * tid) : u32x4{0u, 0u, 0u, 0u};
    constexpr int PPT = kAttChunksWG / 4;  // RoPE base entries per thread (chunks x 64 / 256)
    const int rp0 = (tid % (64 / PPT)) * PPT, rq0 = (tid & 31) * 2;
    double fb[PPT], fo[2];
#pragma unroll
    for (int p = 0; p < PPT; ++p) fb[p] = a.inv_freq[rp0 + p];
#pragma unroll
    for (int p = 0; p < 2; ++p) fo[p] = a.inv_freq[rq0 + p];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) tok[nt] = chunk_of(CPW * wave + 2 * nt + (col >> 3)) * kChunk + (col & 7);
    const int rope_chunk = chunk_of(tid / (64 / PPT));  // chunk whose RoPE base row this thread fills
    const int rd_chunk = chunk_of(tid & (kAttChunksWG - 1));
    asm volatile("" ::"v"(b1v), "v"(b2v), "v"(qv), "v"(rope_chunk), "v"(rd_chunk), "v"(fo[0]), "v"(fo[1])
                 : "memory");
#pragma unroll
    for (int p = 0; p < PPT; ++p) asm volatile("" ::"v"(fb[p]) : "memory");
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) asm volatile("" ::"v"(tok[nt]) : "memory");
    uint32_t rd = 0;
    if (tid < kAttChunksWG) rd = a.res_desc[chead * (size_t)(a.prefix_cap / kChunk) + rd_chunk];
#pragma unroll
    for (int s = 0; s < LG && s < NR; ++s) gather(s);
    __builtin_amdgcn_sched_barrier(0);

    // RoPE rotations of this workgroup's tokens (VALU work while the loads
    // fly): base angle of every chunk start, reduced in fp64, and the
    // offsets 0..7 inside a chunk
    {
      const int cs = tid / (64 / PPT);
      const double pos = (double)rope_chunk * kChunk;
#pragma unroll
      for (int p = 0; p < PPT; ++p) L.rope_base[cs][rp0 + p] = rot_of(pos * fb[p]);
      const int i = tid >> 5;
#pragma unroll
      for (int p = 0; p < 2; ++p) L.rope_off[i][rq0 + p] = rot_of((double)i * fo[p]);
    }
    L.b1f[tid] = bf16_to_f32(b1v);
    if (tid < kHeadDim) L.b2f[tid] = bf16_to_f32(b2v);
    if (tid < 16 * g) *reinterpret_cast<u32x4*>(&L.qs[tid >> 4][8 * (tid & 15)]) = qv;
    stage_store(0, sreg[0]);
    __syncthreads();

    // ---- per-lane LDS read offsets
    // recon A (basis), k-step ks of a stage, m-tile parity q: row 16 mt + col
    // is line 8 mt + col/2, half col%2; the lane's piece is 4 ks + grp (bf16)
    // or 2 grp + ks (int4: the lane holds r = 16 grp + 8 ks + e of the slice)
    int ra[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int p = CI4 ? 2 * grp + ks : 4 * ks + grp;
        ra[ks][q] = (col >> 1) * 256 + ((((col & 1) ^ q) << 3) | (p ^ (col >> 1))) * 16;
      }
    // W1 position row 16 hn + col, piece 4 ks + grp; W2 row 16 nd + col,
    // piece grp (line 4 nd + col/4)
    int rw1[4], rw2[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) rw1[s] = col * 256 + ((4 * s + grp) ^ col) * 16;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      rw2[q] = 8192 + (col >> 2) * 256 + ((((col & 3) ^ q) << 2) | (grp ^ (col >> 2))) * 16;

    f32x4 acc[NT][8];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 kpre_b[NT][4];
    bf16x8 pa[NT / 2];                      // softmax weights (B operand, token slots)
    f32x4 vacc[STAGES ? NT : 1][8];         // per-token values (stage output only)
    constexpr int RL = RI4 ? kAttChunksWG / 8 : kAttChunksWG / 2;  // residual pieces per thread
    u32x4 rres[RI4 ? RL + 1 : RL];

    const size_t row0 = head * (size_t)a.k_eff * kChunk + (size_t)(chunk0 + CPW * wave) * kChunk;
    // residual row of workgroup token tl (< 128), or -1
    auto resid_row = [&](int tl) -> int {
      const uint32_t dsc = L.rdesc[tl >> 3];
      const int i = tl & 7;
      if (!((dsc >> i) & 1u)) return -1;
      return (int)(dsc >> 8) + __popc(dsc & ((1u << i) - 1u) & 0xFFu);
    };

#pragma unroll
    for (int s = 0; s < NS; ++s) {
      // loads for later stages: the stage SL ahead, the gather LG ahead,
      // and (two stages before the end) the residual tile
      if (s + SL < NS) stage_load(s + SL, sreg[s + SL]);
      if (s + LG < NR) gather(s + LG);
      if (s == NS - 2) {
        if constexpr (!RI4) {
          // 128 tokens x 16 pieces; a token without a residual reads past
          // the end of the buffer, which returns zeros
          const uint32_t nbytes = (uint32_t)a.n_resid * kHeadDim * 2;
          const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(
              static_cast<const uint16_t*>(a.res_val) + chead * (size_t)a.n_resid * kHeadDim, nbytes);
#pragma unroll
          for (int u = 0; u < RL; ++u) {
            const int tl = 16 * u + (tid >> 4);
            const int rn = resid_row(tl);
            rres[u] = buffer_ld16(rv, rn >= 0 ? (uint32_t)rn * 256 + (tid & 15) * 16 : nbytes, 0);
          }
        } else {
          // int4 rows: 64 bytes of codes (4 pieces) + 8 bytes of scales
          const uint32_t nbytes = (uint32_t)a.n_resid * (kHeadDim / 2);
          const uint32_t sbytes = (uint32_t)a.n_resid * (kHeadDim / 32) * 2;
          const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(
              static_cast<const uint8_t*>(a.res_val) + chead * (size_t)a.n_resid * (kHeadDim / 2), nbytes);
          const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(
              a.res_scale + chead * (size_t)a.n_resid * (kHeadDim / 32), sbytes);
#pragma unroll
          for (int u = 0; u < RL; ++u) {
            const int tl = 64 * u + (tid >> 2);
            const int rn = resid_row(tl);
            rres[u] = buffer_ld16(rv, rn >= 0 ? (uint32_t)rn * 64 + (tid & 3) * 16 : nbytes, 0);
          }
          {
            // scales: 8 bytes per token, threads 2 t and 2 t + 1 (and 2 t + 256...) share token t
            const int tl = tid >> 1;
            const int rn = resid_row(tl);
            const u32x2 sc = __builtin_amdgcn_raw_buffer_load_b64(rs, rn >= 0 ? (uint32_t)rn * 8 : sbytes, 0, 0);
            u32x2 sc2 = {0u, 0u};
            if constexpr (kAttChunksWG * 8 > 128) {
              const int rn2 = resid_row(tl + 128);
              sc2 = __builtin_amdgcn_raw_buffer_load_b64(rs, rn2 >= 0 ? (uint32_t)rn2 * 8 : sbytes, 0, 0);
            }
            rres[RL] = u32x4{sc[0], sc[1], sc2[0], sc2[1]};
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the loads above at the top of the step

      const unsigned char* sb = L.buf + (s & 1) * kStage;
      if (s < NR) {
        // ---------------- reconstruction, basis columns [64 s, 64 s + 64)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8 bop[NT];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            if constexpr (!CI4) bop[nt] = cv[s][ks][nt];
            else bop[nt] = dequant8(cq[s][nt][ks], csc[s][nt]);
          }
#pragma unroll
          for (int mt = 0; mt < 8; ++mt) {
            const bf16x8 aop = lds16(sb, ra[ks][mt & 1] + 2048 * mt);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) acc[nt][mt] = mfma16(aop, bop[nt], acc[nt][mt]);
          }
        }
        if (s == NR - 1) {
          // -------- K_pre done: acc[nt][mt][e] = K_pre[t][d], t = 16 nt + col,
          //          d = 32 (mt / 2) + 8 grp + 4 (mt % 2) + e
          if constexpr (STAGES) {
            if (a.kpre_out) {
#pragma unroll
              for (int nt = 0; nt < NT; ++nt)
                if (16 * nt + col < nvalid)
#pragma unroll
                  for (int mt = 0; mt < 8; ++mt)
                    *reinterpret_cast<f32x4*>(a.kpre_out + (row0 + 16 * nt + col) * kHeadDim + 32 * (mt >> 1) +
                                              8 * grp + 4 * (mt & 1)) = acc[nt][mt];
            }
          }
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) kpre_b[nt][ks] = pack8(acc[nt][2 * ks], acc[nt][2 * ks + 1]);
          // RoPE: pair (d, d + 64) = m-tiles (mt, mt + 4) of the same lane
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const int cs = CPW * wave + 2 * nt + (col >> 3), i = col & 7;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int p = 32 * (mt >> 1) + 8 * grp + 4 * (mt & 1) + e;
                const float2 bs = L.rope_base[cs][p], of = L.rope_off[i][p];
                const float c = bs.x * of.x - bs.y * of.y;
                const float sn = bs.y * of.x + bs.x * of.y;
                const float x1 = acc[nt][mt][e], x2 = acc[nt][mt + 4][e];
                acc[nt][mt][e] = x1 * c - x2 * sn;
                acc[nt][mt + 4][e] = x2 * c + x1 * sn;
              }
            }
          }
          if constexpr (STAGES) {
            if (a.kpost_out) {
#pragma unroll
              for (int nt = 0; nt < NT; ++nt)
                if (16 * nt + col < nvalid)
#pragma unroll
                  for (int mt = 0; mt < 8; ++mt)
                    *reinterpret_cast<f32x4*>(a.kpost_out + (row0 + 16 * nt + col) * kHeadDim + 32 * (mt >> 1) +
                                              8 * grp + 4 * (mt & 1)) = acc[nt][mt];
            }
          }
          // QK with K_post rounded to bf16 (2^-9 relative per entry), then
          // this wave's softmax weights: the value section needs them
          f32x4 zacc[NT];
          {
            bf16x8 qp[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
              qp[ks] = col < g ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(&L.qs[col][32 * ks + 8 * grp]))
                               : zero_bf16x8();
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int ks = 0; ks < 4; ++ks) z = mfma16(pack8(acc[nt][2 * ks], acc[nt][2 * ks + 1]), qp[ks], z);
              zacc[nt] = z;
            }
          }
          wave_softmax<NT>(zacc, nvalid, a.scale_log2, grp, wm, wl, pa);
#pragma unroll
          for (int nd = 0; nd < 8; ++nd) oacc[nd] = f32x4{0.f, 0.f, 0.f, 0.f};
          if constexpr (STAGES) {
#pragma unroll
            for (int nd = 0; nd < 8; ++nd) {
              const float bias = L.b2f[16 * nd + col];
#pragma unroll
              for (int tt = 0; tt < NT; ++tt) vacc[tt][nd] = f32x4{bias, bias, bias, bias};
            }
          }
        }
      } else {
        // ---------------- values, hidden units [32 c, 32 c + 32).  With p the
        // softmax weights, sum_t p_t V_t = W2 (sum_t p_t gelu(W1 K_t + b1))
        // + b2 sum_t p_t + sum_t p_t R_t: the hidden activations are
        // contracted over this wave's tokens first, so W2 is applied to
        // one row per query head instead of one per token.
        //   MLP1  D[t][h] = K_pre[t][d] x W1^T[d][h]   (b1 initial value)
        //   PH    D[h][j] = gelu(hid)^T[h][t] x p^T[t][j]
        //   OUT   D[d][j] += W2[d][h] x PH[h][j]
        const int c = s - NR;
        f32x4 hacc[NT][2];  // [token tile][hidden tile]
#pragma unroll
        for (int hn = 0; hn < 2; ++hn) {
          const float bias = L.b1f[32 * c + 16 * hn + col];
#pragma unroll
          for (int tt = 0; tt < NT; ++tt) hacc[tt][hn] = f32x4{bias, bias, bias, bias};
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
          for (int hn = 0; hn < 2; ++hn) {
            const bf16x8 bop = lds16(sb, rw1[ks] + 4096 * hn);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) hacc[tt][hn] = mfma16(kpre_b[tt][ks], bop, hacc[tt][hn]);
          }
        }
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
          for (int hn = 0; hn < 2; ++hn)
#pragma unroll
            for (int e = 0; e < 4; ++e) hacc[tt][hn][e] = gelu_fast(hacc[tt][hn][e]);
        f32x4 pht[2];
#pragma unroll
        for (int hn = 0; hn < 2; ++hn) {
          pht[hn] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int q = 0; q < NT / 2; ++q)
            pht[hn] = mfma16(pack8(hacc[2 * q][hn], hacc[2 * q + 1][hn]), pa[q], pht[hn]);
        }
        const bf16x8 hb = pack8(pht[0], pht[1]);
#pragma unroll
        for (int nd = 0; nd < 8; ++nd) oacc[nd] = mfma16(lds16(sb, rw2[nd & 3] + 1024 * nd), hb, oacc[nd]);

        if constexpr (STAGES) {
          // per-token values for the stage output: MLP1 again as D[h][t]
          // (W1 as the A operand), GELU, then D[t][d] = hid x W2^T
          f32x4 hq[2][NT];  // [hidden tile][token tile]
#pragma unroll
          for (int hm = 0; hm < 2; ++hm) {
            const f32x4 bias = *reinterpret_cast<const f32x4*>(&L.b1f[32 * c + 16 * hm + 4 * grp]);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) hq[hm][nt] = bias;
          }
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int hm = 0; hm < 2; ++hm) {
              const bf16x8 aop = lds16(sb, rw1[ks] + 4096 * hm);
#pragma unroll
              for (int nt = 0; nt < NT; ++nt) hq[hm][nt] = mfma16(aop, kpre_b[nt][ks], hq[hm][nt]);
            }
#pragma unroll
          for (int hm = 0; hm < 2; ++hm)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int e = 0; e < 4; ++e) hq[hm][nt][e] = gelu_fast(hq[hm][nt][e]);
#pragma unroll
          for (int nd = 0; nd < 8; ++nd) {
            const bf16x8 bop = lds16(sb, rw2[nd & 3] + 1024 * nd);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) vacc[nt][nd] = mfma16(pack8(hq[0][nt], hq[1][nt]), bop, vacc[nt][nd]);
          }
        }
      }
      if (s == 0 && tid < kAttChunksWG) L.rdesc[tid] = rd;  // first read at step NS - 2
      if (s + 1 < NS) {
        stage_store(s + 1, sreg[s + 1]);  // into the buffer step s - 1 read
        __syncthreads();
      }
    }

    // ---- residual tile -> LDS (rows of kResRow / kResRow4 bytes)
    __syncthreads();
    if constexpr (!RI4) {
#pragma unroll
      for (int u = 0; u < RL; ++u) {
        const int tl = 16 * u + (tid >> 4);
        *reinterpret_cast<u32x4*>(buf + tl * kResRow + (tid & 15) * 16) = rres[u];
      }
    } else {
#pragma unroll
      for (int u = 0; u < RL; ++u) {
        const int tl = 64 * u + (tid >> 2);
        *reinterpret_cast<u32x4*>(buf + tl * kResRow4 + (tid & 3) * 16) = rres[u];
      }
      if ((tid & 1) == 0) {
        *reinterpret_cast<u32x2*>(buf + (tid >> 1) * kResRow4 + 64) = u32x2{rres[RL][0], rres[RL][1]};
        if constexpr (kAttChunksWG * 8 > 128)
          *reinterpret_cast<u32x2*>(buf + ((tid >> 1) + 128) * kResRow4 + 64) = u32x2{rres[RL][2], rres[RL][3]};
      }
    }
    __syncthreads();
    // residual of wave token t (< 32) at dimension d, as a float
    auto resid_at = [&](int t, int d) -> float {
      const int tl = TOKW * wave + t;
      if constexpr (!RI4) {
        return bf16_to_f32(*reinterpret_cast<const uint16_t*>(buf + tl * kResRow + d * 2));
      } else {
        const uint32_t byte = buf[tl * kResRow4 + (d >> 1)];
        const int code = static_cast<int>(((byte >> (4 * (d & 1))) & 0xFu) ^ 8u) - 8;
        const uint16_t sc = *reinterpret_cast<const uint16_t*>(buf + tl * kResRow4 + 64 + (d >> 5) * 2);
        return static_cast<float>(code) * f16_to_f32(sc);
      }
    };
    // OUT += R^T[d][t] x p^T[t][j] (token slots as in the softmax operand)
    // and b2[d] * sum_t p_t
#pragma unroll
    for (int nd = 0; nd < 8; ++nd) {
#pragma unroll
      for (int q = 0; q < NT / 2; ++q) {
        bf16x8 rop;
        if constexpr (!RI4) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int tl = TOKW * wave + 32 * q + (e < 4 ? 4 * grp + e : 16 + 4 * grp + e - 4);
            rop[e] = *reinterpret_cast<const __bf16*>(buf + tl * kResRow + (16 * nd + col) * 2);
          }
        } else {
          f32x4 lo, hi;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            lo[e] = resid_at(32 * q + 4 * grp + e, 16 * nd + col);
            hi[e] = resid_at(32 * q + 16 + 4 * grp + e, 16 * nd + col);
          }
          rop = pack8(lo, hi);
        }
        oacc[nd] = mfma16(rop, pa[q], oacc[nd]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) oacc[nd][e] = fmaf(L.b2f[16 * nd + 4 * grp + e], wl, oacc[nd][e]);
    }
    if constexpr (STAGES) {
      if (a.vhat_out) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int t = 16 * tt + 4 * grp + e;
            if (t < nvalid)
#pragma unroll
              for (int nd = 0; nd < 8; ++nd)
                a.vhat_out[(row0 + t) * kHeadDim + 16 * nd + col] = vacc[tt][nd][e] + resid_at(t, 16 * nd + col);
          }
      }
    }
  } else {
    // ========================================================= exact window
    const int w0 = (split - a.n_sel_tiles) * kAttTokWG + wave * kAttTokWave;
    window_wave(qh, a.win_k + chead * (size_t)a.window_cap * kHeadDim,
                a.win_v + chead * (size_t)a.window_cap * kHeadDim, w0, a.window, g, a.scale_log2, grp, col, oacc,
                wm, wl);
  }

  // ======================================== merge the 4 waves, write partial
  write_partial4(reinterpret_cast<float*>(buf), L.ml, oacc, wm, wl,
                 a.part + (head * (size_t)a.n_split + split) * g * kPartStride, g, tid, wave, grp, col);
}

template <int RANK, bool STAGES>
static hipError_t launch_rank(const AttendArgs& a, bool ci4, bool ri4, hipStream_t st) {
  const dim3 grid(a.padded_total), block(kAttWaves * 64);
  if (!ci4 && !ri4) hipLaunchKernelGGL((attend_kernel<RANK, false, false, STAGES>), grid, block, 0, st, a);
  else if (ci4 && ri4) hipLaunchKernelGGL((attend_kernel<RANK, true, true, STAGES>), grid, block, 0, st, a);
  else if (ci4) hipLaunchKernelGGL((attend_kernel<RANK, true, false, STAGES>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((attend_kernel<RANK, false, true, STAGES>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <bool STAGES>
static hipError_t launch_attend_t(const AttendArgs& a, int rank, bool ci4, bool ri4, hipStream_t st) {
  switch (rank) {
    case 128: return launch_rank<128, STAGES>(a, ci4, ri4, st);
    case 256: return launch_rank<256, STAGES>(a, ci4, ri4, st);
    case 512: return launch_rank<512, STAGES>(a, ci4, ri4, st);
    default: break;
  }
  // rank 64: the int4 path needs rank % 128 == 0 and is not instantiated here
  if (ci4) return hipErrorInvalidValue;
  const dim3 grid(a.padded_total), block(kAttWaves * 64);
  if (ri4) hipLaunchKernelGGL((attend_kernel<64, false, true, STAGES>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((attend_kernel<64, false, false, STAGES>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attend(const AttendArgs& a, int rank, bool ci4, bool ri4, hipStream_t st) {
  if (a.total == 0) return hipSuccess;
  if (a.kpre_out || a.kpost_out || a.vhat_out) return launch_attend_t<true>(a, rank, ci4, ri4, st);
  return launch_attend_t<false>(a, rank, ci4, ri4, st);
}

// ---------------------------------------------------------------------------
// Split merge: one workgroup per (sequence, KV head, query head j), 512
// threads = 128 output dims d x 4 split groups.  Every load that does not
// depend on the weights goes out first, together: each thread's o values
// (splits sg, sg + 4, ... in batches of kMergeBatch), its W2 row piece, its PH
// values, and for wave 0 the (m, l) of the first 128 splits.  Wave 0 then
// forms the weights w_s = exp2(m_s - M) / L in LDS (M = max_s m_s,
// L = sum_s exp2(m_s - M) l_s) from registers; the 4 split groups' sums meet
// in LDS.
// The producer/consumer kernel's slots come in groups of 4 (one group of
// tiles, slot w = consumer w); beside each slot's o (its residual share and
// b2 l), a group has one PH row, sum_t p_t gelu(W1 K_pre + b1) over its
// tokens, relative to the largest of its slots' maxima, and the value MLP's
// second layer is applied here, once:
//   out = (sum_s w_s o_s + W2 (sum_groups W_g PH_g)) / L,  W_g = max of the group's w_s.
// The 512 threads first form the weighted sum of the PH rows (256 units x 2
// halves of the groups), then thread (d, sg) adds W2[d][64 sg .. 64 sg + 63]
// . that sum.
// ---------------------------------------------------------------------------
constexpr int kMergeThreads = 512;
constexpr int kMergeBatch = 16;
constexpr int kMergePhBatch = 8;  // PH groups a thread has in flight (per half)

__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const float* __restrict__ part,
                                                              uint16_t* __restrict__ out, int hkv,
                                                              int g, int n_split, MergePH phm, int n_blocks) {
  __shared__ float wgt[kMergeMaxSplits];
  __shared__ float red[3][kHeadDim];
  __shared__ float phc[2][kHidden];
  __shared__ float inv_l;
  const int tid = threadIdx.x, d = tid & (kHeadDim - 1), sg = tid >> 7;
  // one workgroup per (sequence, KV head, query head j), j fastest; the
  // workgroups of one (sequence, KV head) go to one XCD, so that the head's
  // W2 rows are fetched into that XCD's L2 once and shared
  const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
  if (lb >= n_blocks) return;
  const int j = lb % g, hb = lb / g;
  const int bq = hb / hkv, hq = hb - bq * hkv;
  const size_t head = (size_t)hb;
  const size_t st = (size_t)g * kPartStride;  // between splits
  const float* pj = part + head * (size_t)n_split * st + (size_t)j * kPartStride;
  const int ns = n_split;
  const int nph = phm.n_ph_used;
  // this thread's first batch of o values (indices clamped into the list,
  // so that the loads are unconditional and all in flight together; the
  // extra ones are not summed)
  float ov[kMergeBatch];
#pragma unroll
  for (int k = 0; k < kMergeBatch; ++k) ov[k] = pj[min(sg + 4 * k, ns - 1) * st + 2 + d];
  // W2 row d, units [64 sg, 64 sg + 64), of this head, and this thread's PH
  // values: unit u = tid % 256 of the groups of parity tid / 256 (PH row of
  // group gx = slot 4 gx)
  bf16x8 w2v[8];
  const int u = tid & (kHidden - 1), half = tid >> 8;
  const int ngrp = nph / 4;
  const size_t phs = (size_t)g * kHidden;  // between slots
  const float* pp = phm.ph + head * (size_t)phm.ph_stride * phs + (size_t)j * kHidden + u;
  float hv[kMergePhBatch];
  if (nph > 0) {
    const size_t chead = (size_t)bq * phm.cache_bmul * hkv + hq;
    const uint16_t* w2row = phm.w2 + (chead * kHeadDim + d) * kHidden + 64 * sg;
#pragma unroll
    for (int k = 0; k < 8; ++k) w2v[k] = load_bf16x8(w2row + 8 * k);
#pragma unroll
    for (int k = 0; k < kMergePhBatch; ++k) hv[k] = pp[4 * min(half + 2 * k, ngrp - 1) * phs];
  }
  if (tid < 64) {
    // (m, l) of splits tid and tid + 64 in registers; any beyond 128 are read in a loop
    float mv[2], lv[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int sp = min(tid + 64 * r, ns - 1);
      mv[r] = pj[sp * st];
      lv[r] = pj[sp * st + 1];
    }
    float m = -__builtin_huge_valf();
#pragma unroll
    for (int r = 0; r < 2; ++r) m = tid + 64 * r < ns ? fmaxf(m, mv[r]) : m;
    for (int sp = tid + 128; sp < ns; sp += 64) m = fmaxf(m, pj[sp * st]);
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    float l = 0.f;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int sp = tid + 64 * r;
      if (sp < ns) {
        const float w = mv[r] == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(mv[r] - m);
        wgt[sp] = w;
        l += w * lv[r];
      }
    }
    for (int sp = tid + 128; sp < ns; sp += 64) {
      const float ms = pj[sp * st];
      const float w = ms == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(ms - m);
      wgt[sp] = w;
      l += w * pj[sp * st + 1];
    }
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
    if (tid == 0) inv_l = 1.f / l;
  }
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int k = 0; k < kMergeBatch; ++k) {
    const int sp = sg + 4 * k;
    acc += sp < ns ? ov[k] * wgt[min(sp, ns - 1)] : 0.f;
  }
  for (int base = 4 * kMergeBatch; base < ns; base += 4 * kMergeBatch) {
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) ov[k] = pj[min(base + sg + 4 * k, ns - 1) * st + 2 + d];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const int sp = base + sg + 4 * k;
      acc += sp < ns ? ov[k] * wgt[min(sp, ns - 1)] : 0.f;
    }
  }
  if (nph > 0) {
    // sum_g W_g PH_g over this thread's groups (the first batch already loaded)
    auto group_weight = [&](int gx) {
      return fmaxf(fmaxf(wgt[4 * gx], wgt[4 * gx + 1]), fmaxf(wgt[4 * gx + 2], wgt[4 * gx + 3]));
    };
    float hs = 0.f;
#pragma unroll
    for (int k = 0; k < kMergePhBatch; ++k) {
      const int gx = half + 2 * k;
      hs += gx < ngrp ? hv[k] * group_weight(min(gx, ngrp - 1)) : 0.f;
    }
    for (int base = half + 2 * kMergePhBatch; base < ngrp; base += 2 * kMergePhBatch) {
#pragma unroll
      for (int k = 0; k < kMergePhBatch; ++k) hv[k] = pp[4 * min(base + 2 * k, ngrp - 1) * phs];
#pragma unroll
      for (int k = 0; k < kMergePhBatch; ++k) {
        const int gx = base + 2 * k;
        hs += gx < ngrp ? hv[k] * group_weight(min(gx, ngrp - 1)) : 0.f;
      }
    }
    phc[half][u] = hs;
    __syncthreads();
    float w2acc = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int uu = 64 * sg + 8 * k + e;
        w2acc = fmaf((float)w2v[k][e], phc[0][uu] + phc[1][uu], w2acc);
      }
    acc += w2acc;
  }
  if (sg > 0) red[sg - 1][d] = acc;
  __syncthreads();
  if (sg == 0) {
    const float o = ((acc + red[0][d]) + (red[1][d] + red[2][d])) * inv_l;
    out[(head * g + j) * kHeadDim + d] = __builtin_bit_cast(uint16_t, (__bf16)o);
  }
}

hipError_t launch_merge(const float* part, uint16_t* out, int nb, int hkv, int g, int n_split,
                        hipStream_t st, const MergePH& phm) {
  if (n_split > kMergeMaxSplits || n_split < 1) return hipErrorInvalidValue;
  if (phm.n_ph_used > 0 && (!phm.ph || !phm.w2 || phm.n_ph_used > n_split || phm.ph_stride < phm.n_ph_used ||
                            phm.n_ph_used % 4))
    return hipErrorInvalidValue;
  const long long n_blocks = (long long)g * hkv * nb;
  if (n_blocks <= 0) return hipSuccess;
  if (n_blocks > ((long long)0xFFFFFFFF / kMergeThreads & ~7LL)) return hipErrorInvalidValue;  // work-items in 32 bits
  const int padded = (int)((n_blocks + 7) & ~7LL);  // a multiple of the 8 XCDs
  hipLaunchKernelGGL(merge_kernel, dim3(padded), dim3(kMergeThreads), 0, st, part, out, hkv, g, n_split, phm,
                     (int)n_blocks);
  return hipGetLastError();
}

}  // namespace lowram
