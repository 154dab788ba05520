// Producer/consumer form of the fused selective-reconstruction attention over
// the selected chunks (gfx950).  It computes what the selected-chunk branch of
// the 4-wave kernel in attend.hip computes, with the same operand layouts and
// the same algebra of the value section (LowRAM review, key and value
// paragraphs; explainer "How the method works"):
//   K_pre = C[t] . B_blk, K_post = RoPE(K_pre, t), z = q . K_post,
//   sum_t p_t V_t = W2 (sum_t p_t gelu(W1 K_pre + b1)) + b2 sum_t p_t + sum_t p_t R_t.
// What changes is which wave does what, and when.
//
// In the 4-wave kernel every wave runs the MFMA-only reconstruction and then
// the VALU-heavy value section of its own tokens, so the two co-resident
// workgroups of a CU keep the matrix cores and the vector ALUs busy in turn
// rather than together.  Here one workgroup of 8 waves holds a CU (about
// 158 KiB of LDS) for the whole launch.  The 128-token tiles of every
// (sequence, KV head) are cut into groups of tpw consecutive tiles; the grid
// has one workgroup per CU (W of them), and workgroup w takes groups
// w, w + W, w + 2 W, ... one after another inside one pipeline, so the
// pipeline fills and drains once per CU, and at any time the neighbouring
// workgroups of an XCD work on the groups of the same few heads (their
// basis and W1/W2 stay in that XCD's L2).  Waves 0-3 are producers and
// waves 4-7 consumers; producer w and consumer w + 4 own the same 32 tokens
// (slot w) of every tile.  Time runs in tile-steps of 8 steps with a
// workgroup barrier after each step:
//   producer, tile-step i      rebuild K_pre of tile i from the basis stream
//                              (one r-slice of 64 per step); after the last
//                              slice hand K_pre to the consumer through LDS,
//                              then RoPE, QK and the running softmax, and
//                              hand over the weights p
//   consumer, tile-step i + 1  the value MLP of tile i from the W1/W2 stream
//                              (32 hidden units per step), then the tile's
//                              residual rows
// so on every SIMD the reconstruction of one tile runs beside the value
// section of the one before.  Producer and consumer run separate loops with
// the same number of barriers; the role is a scalar (wave-uniform) branch.
// Everything that depends on the head (basis, W1/W2, biases, queries,
// selection list, descriptors) is looked up per tile, and the loads issued
// for the next tile use the next tile's head.
//
// Running softmax.  A producer keeps (m, l) per query head of its slot over
// the tiles of the current group.  For a new tile it takes
// m' = max(m, max_t z_t), sends the consumer p_t = exp2(z_t - m') and
// alpha = exp2(m - m'), and sets l = l alpha + sum_t p_t; a group starts from
// m = -inf, so its first alpha is 0 and clears the consumer's accumulator.
// The consumer scales its output accumulator by alpha before adding the
// tile.  When a group ends, each consumer writes its slot's partial
// (m, l, o + b2 l) per query head to partial slot 4 gx + slot of the head
// (gx = the group's index in the head); the merge kernel combines them with
// the window's.
#include "attend_ops.h"
#include "common.h"
#include "internal.h"

namespace lowram {

constexpr int kPipeSlots = kPipeSplitsPerGroup;  // producer/consumer pairs (one partial slot each)
constexpr int kPipeThreads = 2 * kPipeSlots * 64;
constexpr int kPipeSteps = kHidden / 32;      // value stages = steps per tile-step
constexpr int kHandSlot = 9216;               // per slot: K_pre operands (8 KiB), then p (1 KiB)
constexpr int kHandP = 8192;
static_assert(kAttSelNT == 2 && kAttChunksWG == 16, "tiles of 128 tokens, 32 per slot");

struct PipeLds {
  alignas(16) unsigned char bring[2][kStage];                   // basis stages (producers)
  alignas(16) unsigned char mring[2][kStage];                   // W1/W2 stages (consumers)
  alignas(16) unsigned char hand[2][kPipeSlots][kHandSlot];     // by tile parity; consumer residual rows too
  // RoPE rotations as fp16 (cos, sin) tables, frequency-contiguous: by the
  // offset 0..7 inside a chunk, and to each chunk start (per producer, its 4 chunks)
  alignas(16) _Float16 rope_oc[kChunk][64];
  alignas(16) _Float16 rope_os[kChunk][64];
  alignas(16) _Float16 rope_bc[kPipeSlots][4][64];
  alignas(16) _Float16 rope_bs[kPipeSlots][4][64];
  // the queries of the current tile's head as fp16: row j < g (zeros above),
  // 16-byte piece p of the row at piece p ^ j
  alignas(16) _Float16 qh[16][kHeadDim];
  // per tile parity: b1 of unit 32 c + row_perm32(p) at 32 c + p, x4 (an MFMA
  // C operand), and b2 (read when a group's partial is written)
  f32x4 b1q[2][kHidden];
  float b2f[2][kHeadDim];
  double invf[64];                       // RoPE frequencies (read where needed: no registers held)
  // per query head after each tile, by tile parity: the accumulator rescale
  // alpha and the running (m, l)
  f32x4 sm[2][kPipeSlots][16];
  uint32_t rdesc[2][kPipeSlots][4];     // residual descriptors of each slot's 4 chunks, by tile parity
};
static_assert(sizeof(PipeLds) <= 160 * 1024, "one workgroup per CU");

// One tile's softmax weights of a slot, relative to the running max, as an
// fp16 MFMA operand.  z[t][j] sits in rows t = 16 nt + 4 grp + e of zacc[nt]
// (column j = lane % 16).
__device__ __forceinline__ void pipe_softmax(const f32x4 (&zacc)[2], int nvalid, float scale_log2, int grp,
                                             float& mrun, float& lrun, float& alpha, f16x8& pa) {
  float p[2][4];
  float m = -__builtin_huge_valf();
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * nt + 4 * grp + e;
      p[nt][e] = t < nvalid ? zacc[nt][e] * scale_log2 : -__builtin_huge_valf();
      m = fmaxf(m, p[nt][e]);
    }
  m = fmaxf(m, __shfl_xor(m, 16));
  m = fmaxf(m, __shfl_xor(m, 32));
  const float mnew = fmaxf(mrun, m);
  const float msafe = mnew == -__builtin_huge_valf() ? 0.f : mnew;
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
  alpha = mrun == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(mrun - mnew);
  lrun = lrun * alpha + lsum;
  mrun = mnew;
  pa = pack8h(f32x4{p[0][0], p[0][1], p[0][2], p[0][3]}, f32x4{p[1][0], p[1][1], p[1][2], p[1][3]});
}

// x as a value the compiler cannot trace to its definition: addresses built
// from it are formed where they are used instead of being hoisted out of the
// tile loop and held (or spilled) for its whole length
__device__ __forceinline__ int fresh(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Position in a workgroup's tile sequence: tile lt of the head of group g,
// with what the group fixes (derived once per group, so that the per-tile
// scalar work stays small): head bh = g / n_grp = sequence * hkv + KV head,
// group gx = g % n_grp of the head, the group's end tile, and the cache
// sequence and cache head (per sequence, or the shared context) it reads.
struct PipeCur {
  int g, lt, bh, gx, gend, cseq, chead;
};
__device__ __forceinline__ PipeCur pipe_first(const AttendArgs& a, int g) {
  PipeCur c;
  c.g = g;
  c.bh = fdiv(g, a.grp_div);
  c.gx = g - c.bh * a.pipe_grp;
  c.lt = c.gx * a.pipe_tpw;
  c.gend = min(c.lt + a.pipe_tpw, a.pipe_tiles);
  const int b = fdiv(c.bh, a.hkv_div);
  c.cseq = b * a.cache_bmul;
  c.chead = c.cseq * a.hkv + (c.bh - b * a.hkv);
  return c;
}
// the tile after c in this workgroup's sequence (groups g, g + W, ...); past
// the last one, c itself, so that look-ahead loads stay in bounds
__device__ __forceinline__ PipeCur pipe_next(const AttendArgs& a, PipeCur c) {
  if (c.lt + 1 < c.gend) {
    ++c.lt;
    return c;
  }
  return c.g + a.pipe_wgs < a.pipe_groups ? pipe_first(a, c.g + a.pipe_wgs) : c;
}

template <int RANK, bool CI4, bool RI4>
__global__ __launch_bounds__(kPipeThreads, 1) void attend_pipe_kernel(const AttendArgs a) {
  __shared__ PipeLds L;
  constexpr int NR = RANK / 64;                 // basis stages per tile
  constexpr int NS = kPipeSteps;                // steps per tile-step
  static_assert(NR >= 1 && NR <= NS, "rank 64 .. 512");
  constexpr int SL = NR < 2 ? NR : 2;           // basis stage registers run SL stages ahead
  constexpr int LG = NR - 1 < 2 ? NR - 1 : 2;   // coefficient gathers run LG stages ahead (0: same step)
  constexpr int NT = 2;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: the role branch is uniform
  const int grp = lane >> 4, col = lane & 15;
  const bool producer = wave < kPipeSlots;
  const int slot = wave & (kPipeSlots - 1), rt = tid & 255;
  const int wg = xcd_logical_block(blockIdx.x, a.pipe_padded);
  if (wg >= a.pipe_wgs) return;
  const int g = a.g;
  // this workgroup's tiles: groups wg, wg + W, ... in turn
  int ntiles = 0;
  for (int gg = wg; gg < a.pipe_groups; gg += a.pipe_wgs)
    ntiles += min(a.pipe_tpw, a.pipe_tiles - (gg - fdiv(gg, a.grp_div) * a.pipe_grp) * a.pipe_tpw);
  auto clamp_chunk = [&](int c) { return min(max(c, 0), a.n_chunks - 1); };
  // raw chunk id at position p of the selection rows of tile lt of head bh
  // (clamped into the list)
  auto sel_at = [&](int bh, int lt, int p) {
    return a.sel[(size_t)bh * a.k_eff + min(lt * kAttChunksWG + p, a.k_eff - 1)];
  };
  // valid tokens of this slot in tile lt
  auto slot_valid = [&](int lt) {
    const int nch = min(kAttChunksWG, a.k_eff - lt * kAttChunksWG);
    return max(0, min(32, (nch - 4 * slot) * kChunk));
  };

  // tables
  if (tid < 64) L.invf[tid] = a.inv_freq[tid];
  if (tid < 256) {
    // offset tables: two consecutive frequencies per thread, as fp16 pairs
    const int io = tid >> 5, p = 2 * (tid & 31);
    const float2 r0 = rot_of((double)io * a.inv_freq[p]), r1 = rot_of((double)io * a.inv_freq[p + 1]);
    reinterpret_cast<h2*>(&L.rope_oc[io][p])[0] = __builtin_convertvector(f32x2{r0.x, r1.x}, h2);
    reinterpret_cast<h2*>(&L.rope_os[io][p])[0] = __builtin_convertvector(f32x2{r0.y, r1.y}, h2);
  }

  if (producer) {
    // ===================================================================== producer
    // basis stage s = columns [64 s, 64 s + 64), 128 rows in pi order, two rows per
    // 256-byte line, 16-byte pieces XOR-swizzled by the line index
    // The basis of one cache head through a descriptor carried across tiles:
    // it moves to the next tile's head at the step whose stage loads start
    // reading the next tile (step NR - SL), so every load keeps constant offsets.
    auto bas_of = [&](int chead) {
      return buffer_rsrc(a.basis + (size_t)chead * kHeadDim * RANK, kHeadDim * RANK * 2);
    };
    const int r0 = rt >> 3, pb = rt & 7;
    const uint32_t bas_goff = (uint32_t)((row_perm32(r0) * RANK + 8 * pb) * 2);
    const int bas_loff = (r0 >> 1) * 256 + ((((r0 & 1) << 3) | pb) ^ ((r0 >> 1) & 15)) * 16;
    auto stage_load = [&](__amdgpu_buffer_rsrc_t bas, int s, u32x4 (&r)[kStageLd]) {
#pragma unroll
      for (int u = 0; u < kStageLd; ++u) r[u] = buffer_ld16(bas, bas_goff, (32 * u * RANK + 64 * s) * 2);
    };
    auto stage_store = [&](int buf, const u32x4 (&r)[kStageLd]) {
      unsigned char* dst = L.bring[buf];
#pragma unroll
      for (int u = 0; u < kStageLd; ++u) *reinterpret_cast<u32x4*>(dst + bas_loff + 4096 * u) = r[u];
    };
    // this lane's gather rows of tile lt of head bh: token 16 nt + col of the slot
    auto tokens_of = [&](int bh, int lt, int (&tk)[NT]) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        tk[nt] = clamp_chunk(sel_at(bh, lt, 4 * slot + 2 * nt + (col >> 3))) * kChunk + (col & 7);
    };
    bf16x8 cv[CI4 ? 1 : NR][2][NT];
    u32x2 cq[CI4 ? NR : 1][NT];
    float csc[CI4 ? NR : 1][NT];
    // coefficient rows tk of cache sequence cseq, stage s
    auto gather = [&](int s, const int (&tk)[NT], int cseq) {
      if constexpr (!CI4) {
        const uint16_t* cb = static_cast<const uint16_t*>(a.coeff) + (size_t)cseq * a.prefix_cap * RANK;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            cv[s][ks][nt] = load_bf16x8(cb + (size_t)tk[nt] * RANK + 64 * s + 32 * ks + 8 * grp);
      } else {
        const uint8_t* cb = static_cast<const uint8_t*>(a.coeff) + (size_t)cseq * a.prefix_cap * (RANK / 2);
        const uint16_t* sb = a.coeff_scale + (size_t)cseq * a.prefix_cap * (RANK / 32);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          cq[s][nt] = *reinterpret_cast<const u32x2*>(cb + (size_t)tk[nt] * (RANK / 2) + 32 * s + 8 * grp);
          csc[s][nt] = f16_to_f32(sb[(size_t)tk[nt] * (RANK / 32) + 2 * s + (grp >> 1)]);
        }
      }
    };
    // recon A operand offsets (see attend.hip): k-step ks, m-tile parity q
    int ra[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int p = CI4 ? 2 * grp + ks : 4 * ks + grp;
        ra[ks][q] = (col >> 1) * 256 + ((((col & 1) ^ q) << 3) | (p ^ (col >> 1))) * 16;
      }

    // ---- prologue
    u32x4 sreg[NR][kStageLd];
    int tokA[NT], tokB[NT];
    // this tile, the next and the one after (look-ahead loads)
    PipeCur tc = pipe_first(a, wg);
    PipeCur tn = pipe_next(a, tc);
    PipeCur tnn = pipe_next(a, tn);
    const int bh0 = tc.bh;
    tokens_of(bh0, tc.lt, tokA);
    // raw chunk ids of the next tile (gather rows, rotation-table row): issued a
    // tile ahead, carried through the loop and clamped at step 1, so that neither
    // the compiler nor the in-order load counter ties them to a wait right away
    int selN[NT], rcN;
    auto load_next_ids = [&](const PipeCur& t) {
      const int bh = t.bh;
      const int ln = fresh(lane);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) selN[nt] = sel_at(bh, t.lt, 4 * slot + 2 * nt + ((ln & 15) >> 3));
      rcN = sel_at(bh, t.lt, 4 * slot + (ln >> 4));
    };
    load_next_ids(tn);
    // The queries of a tile's head go to LDS as fp16 before its tail (step 0
    // of its tile-step; rank 64: the last step of the tile-step before), from
    // 16 bytes per thread loaded at the previous tail.
    constexpr int kQStep = NR >= 2 ? 0 : NS - 1;
    bf16x8 qld;
    auto load_q = [&](int bh) {
      const int r = fresh(rt), j = r >> 4;
      const bf16x8 v = load_bf16x8(a.q + ((size_t)bh * g + min(j, g - 1)) * kHeadDim + 8 * (r & 15));
      qld = j < g ? v : zero_bf16x8();
    };
    auto store_q = [&]() {
      const int r = fresh(rt), j = r >> 4;
      f16x8 h;
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = (_Float16)(float)qld[e];
      *reinterpret_cast<f16x8*>(&L.qh[j][8 * ((r & 15) ^ j)]) = h;
    };
    load_q(bh0);
    if constexpr (NR == 1) store_q();  // the first tail is at step 0
    // this wave's rotation table row: chunk lane / 16, frequencies 4 (lane % 16) + k,
    // written as fp16 pairs, the access type the RoPE reads use
    auto store_rot = [&](float2 r0, float2 r1, float2 r2, float2 r3) {
      const h2 c01 = __builtin_convertvector(f32x2{r0.x, r1.x}, h2), c23 = __builtin_convertvector(f32x2{r2.x, r3.x}, h2);
      const h2 s01 = __builtin_convertvector(f32x2{r0.y, r1.y}, h2), s23 = __builtin_convertvector(f32x2{r2.y, r3.y}, h2);
      // [slot][lane / 16][4 (lane % 16)] = slot base + 4 lane
      const int ln = fresh(lane);
      h2* pc = reinterpret_cast<h2*>(&L.rope_bc[slot][0][0] + 4 * ln);
      h2* ps = reinterpret_cast<h2*>(&L.rope_bs[slot][0][0] + 4 * ln);
      pc[0] = c01;
      pc[1] = c23;
      ps[0] = s01;
      ps[1] = s23;
    };
    float2 rot_next[4];  // rotations to the chunk starts: tile 0 here, later the next tile's
    __amdgpu_buffer_rsrc_t bas = bas_of(tc.chead);
#pragma unroll
    for (int s = 0; s < SL; ++s) stage_load(bas, s, sreg[s]);
#pragma unroll
    for (int s = 0; s < LG; ++s) gather(s, tokA, tc.cseq);
    {
      const double pos = (double)clamp_chunk(sel_at(bh0, tc.lt, 4 * slot + (lane >> 4))) * kChunk;
#pragma unroll
      for (int k = 0; k < 4; ++k) rot_next[k] = rot_of(pos * a.inv_freq[(lane & 15) * 4 + k]);
      store_rot(rot_next[0], rot_next[1], rot_next[2], rot_next[3]);
    }
    stage_store(0, sreg[0]);
    float mrun = -__builtin_huge_valf(), lrun = 0.f;
    __syncthreads();

    f32x4 acc[NT][8];
    const size_t desc_rows = (size_t)(a.prefix_cap / kChunk);
    for (int i = 0; i < ntiles; ++i) {
      const int bh_n = tn.bh, chead_c = tc.chead, cseq_c = tc.cseq, cseq_n = tn.cseq;
      const bool grp_end = tc.lt + 1 == tc.gend;  // the group ends with this tile
      int rc_next = 0;   // the next tile's rotation-table chunk (clamped)
      uint32_t rdv = 0;
      uint16_t b1raw = 0, b2raw = 0;  // this tile's biases, to LDS at the last step
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (s == kQStep) store_q();  // rank >= 128: this tile's; rank 64: the next tile's
        if (s == NS - 1) {
          // this tile's biases for its consumer tile-step (b2: for its
          // partial), ahead of the tail so that they are not held through it
          // (indexed as slot base + lane, the lane offsets the other writes use)
          const float v = bf16_to_f32(b1raw);
          const int ln = fresh(lane);
          (&L.b1q[i & 1][slot * 64])[ln] = f32x4{v, v, v, v};
          if (slot < kHeadDim / 64) (&L.b2f[i & 1][slot * 64])[ln] = bf16_to_f32(b2raw);
        }
        if (s < NR) {
          if (s == 0) {
            // residual descriptors of this tile's 4 chunks (lane k < 4: chunk k),
            // handed to the consumer with K_pre; token 0 of chunk k sits in
            // tokA[k / 2] of lane 8 (k % 2)
            const int c0 = __shfl(tokA[0], 8 * (lane & 1)), c1 = __shfl(tokA[1], 8 * (lane & 1));
            if (lane < 4) rdv = a.res_desc[(size_t)chead_c * desc_rows + ((lane & 2) ? c1 : c0) / kChunk];
            const int r = fresh(rt);
            b1raw = a.b1[(size_t)chead_c * kHidden + (r & ~31) + row_perm32(r & 31)];
            b2raw = a.b2[(size_t)chead_c * kHeadDim + (r & (kHeadDim - 1))];
          }
          if (s == (NR > 1 ? 1 : 0)) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) tokB[nt] = clamp_chunk(selN[nt]) * kChunk + (col & 7);
            rc_next = clamp_chunk(rcN);
          }
          if constexpr (LG == 0) gather(s, tokA, cseq_c);  // rank 64: the stage's own rows
          __builtin_amdgcn_sched_barrier(0);

          if (s == 0) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int mt = 0; mt < 8; ++mt) acc[nt][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
          // all 16 basis operands of the stage are read first, so that the
          // matrix core is not left waiting on one LDS round trip per pair
          const unsigned char* sb = L.bring[(i * NR + s) & 1];
          bf16x8 aop[2][8];
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) aop[ks][mt] = lds16(sb, ra[ks][mt & 1] + 2048 * mt);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            bf16x8 bop[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              if constexpr (!CI4) bop[nt] = cv[s][ks][nt];
              else bop[nt] = dequant8(cq[s][nt][ks], csc[s][nt]);
            }
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
#pragma unroll
              for (int nt = 0; nt < NT; ++nt) acc[nt][mt] = mfma16(aop[ks][mt], bop[nt], acc[nt][mt]);
          }
          // fp64 angle reductions for the next tile, one per step from step 1 on,
          // off the tail of the last stage
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            if (s == (NR > 1 ? (1 + k < NR - 1 ? 1 + k : NR - 1) : 0)) {
              rot_next[k] = rot_of((double)rc_next * kChunk * L.invf[(lane & 15) * 4 + k]);
              // keep the work in this step (the compiler would otherwise sink it into the tail)
              asm volatile("" : "+v"(rot_next[k].x), "+v"(rot_next[k].y));
            }
          }

          if (s == NR - 1) {
            // ---- K_pre done: acc[nt][mt][e] = K_pre[t][d], t = 16 nt + col,
            //      d = 32 (mt / 2) + 8 grp + 4 (mt % 2) + e.  Hand the bf16
            //      operands to the consumer in its register layout.
            unsigned char* hb = L.hand[i & 1][slot];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int ks = 0; ks < 4; ++ks)
                *reinterpret_cast<u32x4*>(hb + (nt * 4 + ks) * 1024 + lane * 16) =
                    __builtin_bit_cast(u32x4, pack8(acc[nt][2 * ks], acc[nt][2 * ks + 1]));
            // RoPE on packed fp16 pairs of consecutive frequencies: pair (d, d + 64)
            // = m-tiles (mt, mt + 4) of the same lane; the rotation is the chunk
            // start's composed with the offset's.  K_post stays fp16 (relative
            // error ~3 2^-11, below the 2^-9 of a bf16 operand) and feeds an fp16
            // QK.  One 16-token half at a time, so that only half of K_post is
            // held at once.
            const int cl = fresh(lane) & 15;
            f16x8 qp[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
              qp[ks] = *reinterpret_cast<const f16x8*>(&L.qh[cl][8 * ((4 * ks + grp) ^ cl)]);
            f32x4 zacc[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
              const int cs = 2 * nt + (cl >> 3);
              h2 kp[8][2];  // K_post of this half, [mt][e pair]
#pragma unroll
              for (int mt = 0; mt < 4; ++mt) {
                const int p0 = 32 * (mt >> 1) + 8 * grp + 4 * (mt & 1);
                const h2* oc = reinterpret_cast<const h2*>(&L.rope_oc[cl & 7][p0]);
                const h2* os = reinterpret_cast<const h2*>(&L.rope_os[cl & 7][p0]);
                const h2* bc = reinterpret_cast<const h2*>(&L.rope_bc[slot][cs][p0]);
                const h2* bs = reinterpret_cast<const h2*>(&L.rope_bs[slot][cs][p0]);
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                  const h2 o_c = oc[q], o_s = os[q], b_c = bc[q], b_s = bs[q];
                  const h2 c = __builtin_elementwise_fma(b_c, o_c, -(b_s * o_s));
                  const h2 sn = __builtin_elementwise_fma(b_s, o_c, b_c * o_s);
                  const h2 x1 = __builtin_convertvector(f32x2{acc[nt][mt][2 * q], acc[nt][mt][2 * q + 1]}, h2);
                  const h2 x2 = __builtin_convertvector(f32x2{acc[nt][mt + 4][2 * q], acc[nt][mt + 4][2 * q + 1]}, h2);
                  kp[mt][q] = __builtin_elementwise_fma(x1, c, -(x2 * sn));
                  kp[mt + 4][q] = __builtin_elementwise_fma(x2, c, x1 * sn);
                }
              }
              // QK of this half (fp16 operands)
              f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int ks = 0; ks < 4; ++ks) {
                const f16x8 kop = __builtin_shufflevector(
                    __builtin_shufflevector(kp[2 * ks][0], kp[2 * ks][1], 0, 1, 2, 3),
                    __builtin_shufflevector(kp[2 * ks + 1][0], kp[2 * ks + 1][1], 0, 1, 2, 3),
                    0, 1, 2, 3, 4, 5, 6, 7);
                z = mfma16h(kop, qp[ks], z);
              }
              zacc[nt] = z;
            }
            // the running softmax
            float alpha;
            f16x8 pa;
            pipe_softmax(zacc, slot_valid(tc.lt), a.scale_log2, grp, mrun, lrun, alpha, pa);
            *reinterpret_cast<u32x4*>(hb + kHandP + lane * 16) = __builtin_bit_cast(u32x4, pa);
            {
              const int ln = fresh(lane);
              if (lane < 16) (&L.sm[i & 1][slot][0])[ln] = f32x4{alpha, mrun, lrun, 0.f};
              if (lane < 4) (&L.rdesc[i & 1][slot][0])[ln] = rdv;
            }
            // a new group starts from nothing (its first alpha is 0)
            if (grp_end) {
              mrun = -__builtin_huge_valf();
              lrun = 0.f;
            }
            // this wave's rotation table for the next tile
            store_rot(rot_next[0], rot_next[1], rot_next[2], rot_next[3]);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) tokA[nt] = tokB[nt];
            load_next_ids(tnn);
            load_q(bh_n);
          }
          // Loads for later stages, issued after this step's products so that
          // a full memory pipeline stalls nothing the step needs.  (Past the
          // last tile they repeat the last tile: harmless, and they keep the
          // code branch-free.)
          __builtin_amdgcn_sched_barrier(0);
          if (s == NR - SL) bas = bas_of(tn.chead);  // from here on the loads are the next tile's
          if constexpr (SL > 0) stage_load(bas, (s + SL) % NR, sreg[(s + SL) % NR]);
          if constexpr (LG > 0) {
            if (s + LG < NR) gather(s + LG, tokA, cseq_c);
            else gather(s + LG - NR, tokB, cseq_n);
          }
          // next basis stage into the buffer the previous step read
          stage_store((i * NR + s + 1) & 1, sreg[(s + 1) % NR]);
        }
        __syncthreads();
      }
      tc = tn;
      tn = tnn;
      tnn = pipe_next(a, tnn);
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) __syncthreads();  // the consumers' last tile
  } else {
    // ===================================================================== consumer
    // Software-pipelined by one value stage: step c runs GELU, PH and OUT of
    // stage c - 1 (VALU work that overlaps the producer's reconstruction
    // MFMAs and this wave's own next products) and then MLP1 of stage c.
    // The last stage of a tile finishes at step 0 of the next tile-step (or
    // after the loop).  Accordingly the W1 half of stage c is stored at the
    // end of step c - 1 and read at step c, the W2 half stored at the end of
    // step c and read at step c + 1, each half in a ring of two buffers.
    // W1 and W2 of one cache head through descriptors carried across tiles,
    // moved to the next tile's head at the steps whose loads start reading it
    // (W1: step NS - 2, W2: step NS - 1)
    auto w1_of = [&](int chead) { return buffer_rsrc(a.w1 + (size_t)chead * kHidden * kHeadDim, kHidden * kHeadDim * 2); };
    auto w2_of = [&](int chead) { return buffer_rsrc(a.w2 + (size_t)chead * kHeadDim * kHidden, kHeadDim * kHidden * 2); };
    // stage c: W1 rows [32 c, 32 c + 32) in pi order (8 KiB at offset 0 of a
    // ring buffer), W2 columns [32 c, 32 c + 32) (natural, four rows per
    // 256-byte line, 8 KiB at offset 8192)
    const int w1row = rt >> 4, w1p = rt & 15;
    const uint32_t w1_goff = (uint32_t)(((8 * ((w1row >> 2) & 3) + (w1row & 3)) * kHeadDim + 8 * w1p) * 2);
    const int w1_loff = w1row * 256 + (w1p ^ (w1row & 15)) * 16;
    const uint32_t w2_goff = (uint32_t)(((rt >> 2) * kHidden + 8 * (rt & 3)) * 2);
    const int w2_loff = 8192 + (rt >> 4) * 256 + ((rt & 15) ^ ((rt >> 4) & 15)) * 16;
    auto w1_load = [&](__amdgpu_buffer_rsrc_t w1r, int c, u32x4 (&r)[2]) {
#pragma unroll
      for (int u = 0; u < 2; ++u) r[u] = buffer_ld16(w1r, w1_goff, (32 * c + 4 * u) * kHeadDim * 2);
    };
    auto w2_load = [&](__amdgpu_buffer_rsrc_t w2r, int c, u32x4 (&r)[2]) {
#pragma unroll
      for (int u = 0; u < 2; ++u) r[u] = buffer_ld16(w2r, w2_goff, (u * 64 * kHidden + 32 * c) * 2);
    };
    auto w1_store = [&](int buf, const u32x4 (&r)[2]) {
#pragma unroll
      for (int u = 0; u < 2; ++u) *reinterpret_cast<u32x4*>(L.mring[buf] + w1_loff + 4096 * u) = r[u];
    };
    auto w2_store = [&](int buf, const u32x4 (&r)[2]) {
#pragma unroll
      for (int u = 0; u < 2; ++u) *reinterpret_cast<u32x4*>(L.mring[buf] + w2_loff + 4096 * u) = r[u];
    };
    // W1 position row 16 hn + col, piece 4 ks + grp; W2 row 16 nd + col, piece grp
    int rw1[4], rw2[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) rw1[s] = col * 256 + ((4 * s + grp) ^ col) * 16;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      rw2[q] = 8192 + (col >> 2) * 256 + ((((col & 3) ^ q) << 2) | (grp ^ (col >> 2))) * 16;

    u32x4 w1reg[NS][2], w2reg[NS][2];
    __amdgpu_buffer_rsrc_t w1r, w2r;
    {
      const int chead0 = pipe_first(a, wg).chead;
      w1r = w1_of(chead0);
      w2r = w2_of(chead0);
      w1_load(w1r, 0, w1reg[0]);
      w1_load(w1r, 1, w1reg[1]);
      w2_load(w2r, 0, w2reg[0]);
    }
    w1_store(0, w1reg[0]);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < NS; ++s) __syncthreads();  // the producers' first tile

    f32x4 oacc[8];
#pragma unroll
    for (int nd = 0; nd < 8; ++nd) oacc[nd] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 hacc[2][NT][2];  // MLP1 of stage c in hacc[c & 1] (before GELU)
    f16x8 pa;              // softmax weights of the current tile (fp16: the PH product)
    // GELU, PH and OUT of stage cs (MLP1 result in hacc[cs & 1], W2 operands
    // already read), softmax weights pw:
    //   PH  D[h][j] = gelu(hid)^T[h][t] x p^T[t][j];  OUT D[d][j] += W2[d][h] x PH[h][j]
    auto finish_stage = [&](int cs, const bf16x8 (&w2op)[8], const f16x8& pw) {
      const f32x4 lo[2] = {hacc[cs & 1][0][0], hacc[cs & 1][0][1]};
      const f32x4 hi[2] = {hacc[cs & 1][1][0], hacc[cs & 1][1][1]};
      f16x8 gl[2];
      gelu16_h(lo, hi, gl);
      f32x4 pht[2];
#pragma unroll
      for (int hn = 0; hn < 2; ++hn) pht[hn] = mfma16h(gl[hn], pw, f32x4{0.f, 0.f, 0.f, 0.f});
      const bf16x8 hbv = pack8(pht[0], pht[1]);
#pragma unroll
      for (int nd = 0; nd < 8; ++nd) oacc[nd] = mfma16(w2op[nd], hbv, oacc[nd]);
    };
    auto read_w2 = [&](int cs, bf16x8 (&w2op)[8]) {
      const unsigned char* sb = L.mring[cs & 1];
#pragma unroll
      for (int nd = 0; nd < 8; ++nd) w2op[nd] = lds16(sb, rw2[nd & 3] + 1024 * nd);
    };
    // group grp_id's partial: slot 4 gx + slot of its head bh; (m, l) from the
    // producer, b2 of the head from LDS (parity par)
    auto write_part = [&](const PipeCur& t, float m, float l, int par) {
      if (col >= g) return;
      float* pp = a.part + (((size_t)t.bh * a.n_split + kPipeSlots * t.gx + slot) * g + col) * kPartStride;
      if (grp == 0) {
        pp[0] = m;
        pp[1] = l;
      }
#pragma unroll
      for (int nd = 0; nd < 8; ++nd)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d = 16 * nd + 4 * grp + e;
          pp[2 + d] = fmaf(L.b2f[par][d], l, oacc[nd][e]);
        }
    };
    constexpr int RL = RI4 ? 2 : 8;  // 16-byte residual pieces per lane
    float m_cur = 0.f, l_cur = 0.f;    // the producer's (m, l) after the tile being consumed
    PipeCur tc = pipe_first(a, wg), tp = tc;  // this tile and the one before
    PipeCur tn = pipe_next(a, tc);
    for (int i = 0; i < ntiles; ++i) {
      const int chead_c = tc.chead;
      // the previous tile ended its group
      const bool prev_end = i > 0 && tp.lt + 1 == tp.gend;
      unsigned char* hb = L.hand[i & 1][slot];
      bf16x8 kpre_b[NT][4];
      bf16x8 pab;  // the softmax weights in bf16 (the residual product)
      u32x4 rres[RL];
      u32x2 rsc = {0u, 0u};
#pragma unroll
      for (int c = 0; c < NS; ++c) {
        // ---- LDS operands first: MLP1 of stage c, OUT of stage c - 1, and at a
        //      tile start the handoff (at the very first step the W2 read is unused)
        bf16x8 w1op[4][2];
        f32x4 b1v[2];
        {
          const unsigned char* sb = L.mring[c & 1];
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int hn = 0; hn < 2; ++hn) w1op[ks][hn] = lds16(sb, rw1[ks] + 4096 * hn);
#pragma unroll
          for (int hn = 0; hn < 2; ++hn) b1v[hn] = L.b1q[i & 1][32 * c + 16 * hn + col];
        }
        bf16x8 w2op[8];  // W2 operands of the previous stage
        read_w2((c + NS - 1) % NS, w2op);
        f16x8 pnew;
        float alpha = 1.f;
        float m_prev = 0.f, l_prev = 0.f;
        if (c == 0) {
          m_prev = m_cur;
          l_prev = l_cur;
          const f32x4 sm = L.sm[i & 1][slot][col];
          m_cur = sm[1];
          l_cur = sm[2];
          alpha = sm[0];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
              kpre_b[nt][ks] = lds16(hb, (nt * 4 + ks) * 1024 + lane * 16);
          pnew = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(hb + kHandP + lane * 16));
        }
        __builtin_amdgcn_sched_barrier(0);
        // ---- MLP1 of stage c: D[t][h] = K_pre[t][d] x W1^T[d][h] (b1 initial value),
        //      hidden units [32 c, 32 c + 32); its matrix work runs under the GELU below
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int hn = 0; hn < 2; ++hn)
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
              hacc[c & 1][tt][hn] = mfma16(kpre_b[tt][ks], w1op[ks][hn], ks == 0 ? b1v[hn] : hacc[c & 1][tt][hn]);
        // ---- the previous stage: GELU, PH, OUT (at a tile start: the previous
        //      tile's last stage with that tile's weights, then the rescale)
        if (c > 0 || i > 0) finish_stage((c + NS - 1) % NS, w2op, pa);
        if (c == 0) {
          if (prev_end) write_part(tp, m_prev, l_prev, (i - 1) & 1);
          pa = pnew;
#pragma unroll
          for (int e = 0; e < 8; ++e) pab[e] = (__bf16)(float)pa[e];
#pragma unroll
          for (int nd = 0; nd < 8; ++nd) oacc[nd] *= alpha;
        }

        if (c == NS - 1) {
          // ---- residuals: rows -> this slot's handoff region (read at step 0,
          //      not written again before the tile after next), then
          //      OUT += R^T[d][t] x p^T[t][j]
          if constexpr (!RI4) {
#pragma unroll
            for (int u = 0; u < RL; ++u)
              *reinterpret_cast<u32x4*>(hb + (4 * u + (lane >> 4)) * kResRow + (lane & 15) * 16) = rres[u];
            // the reads below take the bytes just written under another type
            asm volatile("" ::: "memory");
#pragma unroll
            for (int nd = 0; nd < 8; ++nd) {
              bf16x8 rop;
#pragma unroll
              for (int e = 0; e < 8; ++e) {
                const int t = e < 4 ? 4 * grp + e : 16 + 4 * grp + e - 4;
                rop[e] = *reinterpret_cast<const __bf16*>(hb + t * kResRow + (16 * nd + col) * 2);
              }
              oacc[nd] = mfma16(rop, pab, oacc[nd]);
            }
          } else {
#pragma unroll
            for (int u = 0; u < RL; ++u)
              *reinterpret_cast<u32x4*>(hb + (16 * u + (lane >> 2)) * kResRow4 + (lane & 3) * 16) = rres[u];
            if (lane < 32) *reinterpret_cast<u32x2*>(hb + lane * kResRow4 + 64) = rsc;
            asm volatile("" ::: "memory");  // the reads below take these bytes under other types
            auto resid_at = [&](int t, int d) -> float {
              const uint32_t byte = hb[t * kResRow4 + (d >> 1)];
              const int code = static_cast<int>(((byte >> (4 * (d & 1))) & 0xFu) ^ 8u) - 8;
              const uint16_t sc = *reinterpret_cast<const uint16_t*>(hb + t * kResRow4 + 64 + (d >> 5) * 2);
              return static_cast<float>(code) * f16_to_f32(sc);
            };
#pragma unroll
            for (int nd = 0; nd < 8; ++nd) {
              f32x4 lo, hi;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                lo[e] = resid_at(4 * grp + e, 16 * nd + col);
                hi[e] = resid_at(16 + 4 * grp + e, 16 * nd + col);
              }
              oacc[nd] = mfma16(pack8(lo, hi), pab, oacc[nd]);
            }
          }
        }
        // Loads for later steps after this step's work (see the producer):
        // the same weights every tile, W1 two stages ahead and W2 one, and
        // the tile's residual rows for step NS - 1
        __builtin_amdgcn_sched_barrier(0);
        if (c == NS - 2) w1r = w1_of(tn.chead);  // from here on the loads are the next tile's
        if (c == NS - 1) w2r = w2_of(tn.chead);
        w1_load(w1r, (c + 2) % NS, w1reg[(c + 2) % NS]);
        w2_load(w2r, (c + 1) % NS, w2reg[(c + 1) % NS]);
        if (c >= 2 && c <= 5) {
          // this slot's residual rows, spread over steps 2-5 (zeros where a
          // token has none: reads past the end of the buffer return 0);
          // descriptors from the producer
          auto row_of = [&](uint32_t dsc, int t) -> int {
            const int bit = t & 7;
            if (!((dsc >> bit) & 1u)) return -1;
            return (int)(dsc >> 8) + __popc(dsc & ((1u << bit) - 1u) & 0xFFu);
          };
          if constexpr (!RI4) {
            const uint32_t nbytes = (uint32_t)a.n_resid * kHeadDim * 2;
            const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(
                static_cast<const uint16_t*>(a.res_val) + (size_t)chead_c * a.n_resid * kHeadDim, nbytes);
#pragma unroll
            for (int u = 2 * (c - 2); u < 2 * (c - 1); ++u) {
              const int t = 4 * u + (lane >> 4);
              const int rn = row_of(L.rdesc[i & 1][slot][u >> 1], t);
              rres[u] = buffer_ld16(rv, rn >= 0 ? (uint32_t)rn * 256 + (lane & 15) * 16 : nbytes, 0);
            }
          } else {
            const uint32_t nbytes = (uint32_t)a.n_resid * (kHeadDim / 2);
            const uint32_t sbytes = (uint32_t)a.n_resid * (kHeadDim / 32) * 2;
            const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(
                static_cast<const uint8_t*>(a.res_val) + (size_t)chead_c * a.n_resid * (kHeadDim / 2), nbytes);
            const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(
                a.res_scale + (size_t)chead_c * a.n_resid * (kHeadDim / 32), sbytes);
            if (c - 1 <= RL) {
              const int u = c - 2;
              const int t = 16 * u + (lane >> 2);
              const int rn = row_of(L.rdesc[i & 1][slot][2 * u + (lane >> 5)], t);
              rres[u] = buffer_ld16(rv, rn >= 0 ? (uint32_t)rn * 64 + (lane & 3) * 16 : nbytes, 0);
            } else if (c == RL + 2) {
              const int t = lane & 31;
              const int rn = row_of(L.rdesc[i & 1][slot][t >> 3], t);
              rsc = __builtin_amdgcn_raw_buffer_load_b64(rs, rn >= 0 ? (uint32_t)rn * 8 : sbytes, 0, 0);
            }
          }
        }
        // W1 of stage c + 1 into the buffer step c - 1 read; W2 of stage c
        // into the buffer step c - 1 read (stage c - 2)
        w1_store((c + 1) & 1, w1reg[(c + 1) % NS]);
        w2_store(c & 1, w2reg[c]);
        __syncthreads();
      }
      tp = tc;
      tc = tn;
      tn = pipe_next(a, tn);
    }
    {
      // the last tile's last stage (its W2 buffer is not written again), and
      // the partial of the last group
      bf16x8 w2op[8];
      read_w2(NS - 1, w2op);
      finish_stage(NS - 1, w2op, pa);
      write_part(tp, m_cur, l_cur, (ntiles - 1) & 1);
    }
  }
}

void plan_pipe(int heads, int n_tiles, int n_cu, int* n_wg, int* tpw, int* n_grp) {
  // Groups of t tiles (t >= 2 where a head has 2 tiles), dealt round-robin to
  // W = min(n_cu, groups) workgroups; a workgroup's pipeline holds at most
  // ceil(groups / W) x t tiles.  Take the t with the fewest, the largest on
  // ties (fewer partial slots).
  *n_wg = *tpw = *n_grp = 0;
  if (heads <= 0 || n_tiles <= 0 || n_cu <= 0) return;
  long long best = -1;
  int bt = 1;
  for (int t = n_tiles < 2 ? 1 : 2; t <= n_tiles; ++t) {
    const long long groups = (long long)heads * ((n_tiles + t - 1) / t);
    const long long w = groups < n_cu ? groups : n_cu;
    const long long cost = (groups + w - 1) / w * t;
    if (best < 0 || cost <= best) {
      best = cost;
      bt = t;
    }
  }
  *tpw = bt;
  *n_grp = (n_tiles + bt - 1) / bt;
  const long long groups = (long long)heads * *n_grp;
  *n_wg = (int)(groups < n_cu ? groups : n_cu);
}

template <int RANK>
static hipError_t launch_pipe_rank(const AttendArgs& a, bool ci4, bool ri4, hipStream_t st) {
  const dim3 grid(a.pipe_padded), block(kPipeThreads);
  if (!ci4 && !ri4) hipLaunchKernelGGL((attend_pipe_kernel<RANK, false, false>), grid, block, 0, st, a);
  else if (ci4 && ri4) hipLaunchKernelGGL((attend_pipe_kernel<RANK, true, true>), grid, block, 0, st, a);
  else if (ci4) hipLaunchKernelGGL((attend_pipe_kernel<RANK, true, false>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((attend_pipe_kernel<RANK, false, true>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attend_pipe(const AttendArgs& a, int rank, bool ci4, bool ri4, hipStream_t st) {
  if (a.pipe_wgs == 0) return hipSuccess;
  switch (rank) {
    case 128: return launch_pipe_rank<128>(a, ci4, ri4, st);
    case 256: return launch_pipe_rank<256>(a, ci4, ri4, st);
    case 512: return launch_pipe_rank<512>(a, ci4, ri4, st);
    default: break;
  }
  // rank 64: the int4 coefficient path needs rank % 128 == 0
  if (ci4) return hipErrorInvalidValue;
  const dim3 grid(a.pipe_padded), block(kPipeThreads);
  if (ri4) hipLaunchKernelGGL((attend_pipe_kernel<64, false, true>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((attend_pipe_kernel<64, false, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace lowram
