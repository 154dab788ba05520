// Producer/consumer form of the fused selective-reconstruction attention over
// the selected chunks (gfx950).  It computes what the selected-chunk branch of
// the 4-wave kernel in attend.hip computes, with the same operand layouts and
// the same algebra of the value section (LowRAM review, key and value
// paragraphs; explainer "How the method works"):
//   K_pre = C[t] . B_blk, K_post = RoPE(K_pre, t), z = q . K_post,
//   sum_t p_t V_t = W2 (sum_t p_t gelu(W1 K_pre + b1)) + b2 sum_t p_t + sum_t p_t R_t.
// What changes is which wave does what, and when, and where W2 is applied:
// W2 is linear, so this kernel stops at PH = sum_t p_t gelu(W1 K_pre + b1)
// (per slot and group of tiles, beside the output-space record of the
// residuals and b2), and the merge kernel applies W2 once per (sequence, KV
// head) to the softmax-weighted sum of the groups' PH.
//
// In the 4-wave kernel every wave runs the MFMA-only reconstruction and then
// the VALU-heavy value section of its own tokens, so the two co-resident
// workgroups of a CU keep the matrix cores and the vector ALUs busy in turn
// rather than together.  Here one workgroup of 8 waves holds a CU (about
// 160 KiB of LDS) for the whole launch.  The 128-token tiles of every
// (sequence, KV head) are cut into groups of tpw consecutive tiles; the grid
// has one workgroup per CU (W of them), and workgroup w takes groups
// w, w + W, w + 2 W, ... one after another inside one pipeline, so the
// pipeline fills and drains once per CU, and at any time the neighbouring
// workgroups of an XCD work on the groups of the same few heads (their
// basis and W1 stay in that XCD's L2).  Waves 0-3 are producers and waves
// 4-7 consumers; producer w owns the 32 tokens of slot w of every tile, and
// consumer w hidden units 64 w .. 64 w + 63 of all of them plus slot w's
// residual rows.  Per tile:
//   producer, tile i       rebuild K_pre of tile i from the basis stream (one
//                          r-slice of 64 per step, rank / 64 steps); after the
//                          last slice hand K_pre to the consumers through LDS,
//                          then RoPE, QK and the running softmax, and hand over
//                          the weights p
//   consumer, tile i - 1   the first MLP layer, GELU and PH of the tile the
//                          producers handed over last, one 16-token piece per
//                          step (8 steps, its W1 rows in registers); then slot
//                          w's residual rows
// so on every SIMD the reconstruction of one tile runs beside the value
// section of the one before.  The role is a scalar (wave-uniform) branch, and
// the waves meet through counters in LDS (pipe_post / pipe_wait), never at a
// workgroup barrier: the producers among themselves over the basis ring (a
// stage is read once all four have stored their quarter of it), the
// consumers when a tile has been handed over, and the producers, before they
// overwrite a hand-off buffer, when the consumers have released the tile
// that used it two tiles earlier.  The producers thus run up to about half a
// step apart, and the two roles at most two tiles apart.  Every count is
// exact: no wave can post ahead of the count another wave is waiting for (a
// producer cannot store stage G + 2 before all have stored G + 1, nor hand
// over tile i + 2 before all have handed over tile i, hence the per-parity
// hand-off counts; a consumer cannot release tile i + 1 before all have
// released tile i).
// Everything that depends on the head (basis, W1, biases, queries,
// selection list, descriptors) is looked up per tile, and the loads issued
// for the next tile use the next tile's head.
//
// Running softmax.  A producer keeps (m, l) per query head of its slot over
// the tiles of the current group.  For a new tile it takes
// m' = max(m, max_t z_t), sends the consumer p_t = exp2(z_t - m') and
// alpha = exp2(m - m'), and sets l = l alpha + sum_t p_t; a group starts from
// m = -inf, so its first alpha is 0 and clears the consumer's accumulator.
// The consumers put the four slots' weights on one scale per tile (the
// largest slot maximum) for PH, and keep slot w's own scale for its residual
// share R.  When a group ends, consumer w writes slot w's output-space
// partial (m, l, R + b2 l) per query head to slot 4 gx + w of the head (gx =
// the group's index in the head) and its quarter of the group's PH (256
// hidden units, relative to the largest slot maximum) to PH row 4 gx; the
// merge kernel combines them with the window's.
#include "attend_ops.h"
#include "common.h"
#include "internal.h"

namespace lowram {

constexpr int kPipeSlots = kPipeSplitsPerGroup;  // producer/consumer pairs (one partial slot each)
constexpr int kPipeThreads = 2 * kPipeSlots * 64;
constexpr int kPipeSteps = kHidden / 32;      // value stages = steps per tile
constexpr int kHandSlot = 9216;               // per slot: K_pre operands (8 KiB), then p (1 KiB)
constexpr int kHandP = 8192;
static_assert(kAttSelNT == 2 && kAttChunksWG == 16, "tiles of 128 tokens, 32 per slot");

struct PipeLds {
  alignas(16) unsigned char bring[2][kStage];                   // basis stages (producers)
  alignas(16) unsigned char hand[2][kPipeSlots][kHandSlot];     // K_pre operands and weights, by tile parity
  alignas(16) unsigned char rrow[kPipeSlots][32 * kResRow];     // each slot's residual rows (consumer w: slot w)
  // RoPE rotations as fp16 (cos, sin) tables, frequency-contiguous: by the
  // offset 0..7 inside a chunk, and to each chunk start (per producer, its 4 chunks)
  alignas(16) _Float16 rope_oc[kChunk][64];
  alignas(16) _Float16 rope_os[kChunk][64];
  alignas(16) _Float16 rope_bc[kPipeSlots][4][64];
  alignas(16) _Float16 rope_bs[kPipeSlots][4][64];
  // the queries of each tile's head as fp16, three tiles in turn (tile i in
  // buffer i % 3): row j < g (zeros above), 16-byte piece p of the row at
  // piece p ^ j
  alignas(16) _Float16 qh[3][16][kHeadDim];
  // b2 of each tile's head, by tile parity (read when a group's partial is written)
  float b2f[2][kHeadDim];
  double invf[64];                       // RoPE frequencies (read where needed: no registers held)
  // per query head after each tile, by tile parity: the accumulator rescale
  // alpha and the running (m, l)
  f32x4 sm[2][kPipeSlots][16];
  uint32_t rdesc[2][kPipeSlots][4];     // residual descriptors of each slot's 4 chunks, by tile parity
  // role synchronisation (counts only grow): basis stage quarters stored to
  // the ring, tiles handed to the consumers (by tile parity), tiles the
  // consumers have released
  unsigned sync_stored, sync_handed[2], sync_released;
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
  m = pair_max32(pair_max16(m));
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
  lsum = pair_add32(pair_add16(lsum));
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

// The two roles meet through counters in LDS instead of workgroup barriers.
// pipe_post: lane 0 adds 1 after every earlier LDS access of the wave has
// completed (release).  pipe_wait: the wave spins until the count reaches
// target (acquire); the spin is bounded (about 4 ms, several hundred times a
// tile's time), so a count that never arrived would end the wait, not hang the
// kernel.
__device__ __forceinline__ void pipe_post(unsigned* c, int lane) {
  if (lane == 0) __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void pipe_wait(unsigned* c, unsigned target) {
#pragma nounroll
  for (int it = 0; it < (1 << 16); ++it) {
    if (__hip_atomic_load(c, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) return;
    __builtin_amdgcn_s_sleep(2);
  }
}

template <int RANK, bool CI4, bool RI4>
__global__ __launch_bounds__(kPipeThreads, 1) void attend_pipe_kernel(const AttendArgs a) {
  __shared__ PipeLds L;
  constexpr int NR = RANK / 64;                 // basis stages per tile
  constexpr int NS = kPipeSteps;                // steps per tile
  static_assert(NR >= 1 && NR <= NS, "rank 64 .. 512");
  constexpr int SL = NR + 1 < 3 ? NR + 1 : 3;   // basis stage registers run SL stages ahead
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
  if (tid == 0) {
    L.sync_stored = 0;
    L.sync_handed[0] = 0;
    L.sync_handed[1] = 0;
    L.sync_released = 0;
  }
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
    auto bas_of = [&](int chead) {
      return buffer_rsrc(a.basis + (size_t)chead * kHeadDim * RANK, kHeadDim * RANK * 2);
    };
    const int r0 = rt >> 3, pb = rt & 7;
    const uint32_t bas_goff = (uint32_t)((row_perm32(r0) * RANK + 8 * pb) * 2);
    auto stage_load = [&](__amdgpu_buffer_rsrc_t bas, int s, u32x4 (&r)[kStageLd]) {
#pragma unroll
      for (int u = 0; u < kStageLd; ++u) r[u] = buffer_ld16(bas, bas_goff, (32 * u * RANK + 64 * s) * 2);
    };
    auto stage_store = [&](int buf, const u32x4 (&r)[kStageLd]) {
      // (the offset is formed here from an opaque thread id, not held across the loop)
      const int t = fresh(rt), q0 = t >> 3, q = t & 7;
      const int bas_loff = (q0 >> 1) * 256 + ((((q0 & 1) << 3) | q) ^ ((q0 >> 1) & 15)) * 16;
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
    // coefficient rows tk of cache sequence cseq, stage s (lane offsets formed
    // here from an opaque lane id, not held across the tile loop)
    auto gather = [&](int s, const int (&tk)[NT], int cseq) {
      const int grp = fresh(lane) >> 4;
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
    // stage registers: stage s of a tile in sreg[s]; the stage of global index
    // G (= tile x NR + s) is loaded at step G - SL and stored to the ring in
    // the middle of step G - 1
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
    // The queries of tile i + 1 go to LDS as fp16 at step 0 of tile i, from
    // 16 bytes per thread loaded at the last step of the tile before.  Three
    // buffers: at step 0 of tile i every producer has passed the wait for that
    // stage, which needs the posts made at the ends of all four tails of tile
    // i - 1, so none still reads the buffer of tile i - 2.
    bf16x8 qld;
    auto load_q = [&](int bh) {
      const int r = fresh(rt), j = r >> 4;
      const bf16x8 v = load_bf16x8(a.q + ((size_t)bh * g + min(j, g - 1)) * kHeadDim + 8 * (r & 15));
      qld = j < g ? v : zero_bf16x8();
    };
    auto store_q = [&](int buf) {
      const int r = fresh(rt), j = r >> 4;
      f16x8 h;
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = (_Float16)(float)qld[e];
      *reinterpret_cast<f16x8*>(&L.qh[buf][j][8 * ((r & 15) ^ j)]) = h;
    };
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
    // stages 0 .. SL - 1; those of the next tile (SL > NR) after stage 0 has
    // left its registers
#pragma unroll
    for (int s = 0; s < SL; ++s)
      if (s < NR) stage_load(bas_of(tc.chead), s, sreg[s]);
#pragma unroll
    for (int s = 0; s < LG; ++s) gather(s, tokA, tc.cseq);
    {
      const double pos = (double)clamp_chunk(sel_at(bh0, tc.lt, 4 * slot + (lane >> 4))) * kChunk;
#pragma unroll
      for (int k = 0; k < 4; ++k) rot_next[k] = rot_of(pos * a.inv_freq[(lane & 15) * 4 + k]);
      store_rot(rot_next[0], rot_next[1], rot_next[2], rot_next[3]);
    }
    stage_store(0, sreg[0]);
#pragma unroll
    for (int s = NR; s < SL; ++s) stage_load(bas_of(tn.chead), s - NR, sreg[s - NR]);
    load_q(bh0);
    store_q(0);
    load_q(tn.bh);
    float mrun = -__builtin_huge_valf(), lrun = 0.f;
    __syncthreads();

    // The ring of two basis stages: stage G is read from buffer G & 1 at
    // step G, once all four producers have stored their quarter of it (the
    // count of stored quarters reaches 4 G).  Each producer posted that store
    // after its reads of stage G - 1 had completed (the post is a release),
    // so at that point the other buffer is free as well: right after reading
    // stage G a producer stores its quarter of stage G + 1 there, and posts it
    // once the first half of the step's products is issued.  A producer can
    // thus run up to about half a step ahead of the slowest one.

    f32x4 acc[NT][8];
    const size_t desc_rows = (size_t)(a.prefix_cap / kChunk);
    int qb = 0;  // i % 3: this tile's query buffer
    for (int i = 0; i < ntiles; ++i) {
      const int chead_c = tc.chead, cseq_c = tc.cseq, cseq_n = tn.cseq;
      const bool grp_end = tc.lt + 1 == tc.gend;  // the group ends with this tile
      int rc_next = 0;   // the next tile's rotation-table chunk (clamped)
      uint32_t rdv = 0;
      uint16_t b2raw = 0;  // this tile's b2, to LDS at the tail
      bf16x8 aop[2][8];
      // ---- the start of step s (stage G = i NR + s): per-tile loads and
      //      hand-offs, then the stage's 16 basis operands from the ring
      auto step_begin = [&](int s) {
        const unsigned G = (unsigned)(i * NR + s);
        // this tile's hand-off structures (parity i & 1) are written from here
        // on: the consumers must have released tile i - 2
        if (s == NR - 1 && i >= 2) pipe_wait(&L.sync_released, 4u * (unsigned)(i - 1));
        if (s == 0) {
          // residual descriptors of this tile's 4 chunks (lane k < 4: chunk k),
          // handed to the consumer with K_pre; token 0 of chunk k sits in
          // tokA[k / 2] of lane 8 (k % 2)
          const int c0 = __shfl(tokA[0], 8 * (lane & 1)), c1 = __shfl(tokA[1], 8 * (lane & 1));
          if (lane < 4) rdv = a.res_desc[(size_t)chead_c * desc_rows + ((lane & 2) ? c1 : c0) / kChunk];
          const int r = fresh(rt);
          b2raw = a.b2[(size_t)chead_c * kHeadDim + (r & (kHeadDim - 1))];
        }
        if (s == (NR > 1 ? 1 : 0)) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) tokB[nt] = clamp_chunk(selN[nt]) * kChunk + (fresh(lane) & 7);
          rc_next = clamp_chunk(rcN);
        }
        if constexpr (LG == 0) gather(s, tokA, cseq_c);  // rank 64: the stage's own rows
        // stage G is in the ring once all four producers have stored their quarter
        if (G > 0) pipe_wait(&L.sync_stored, 4u * G);
        if (s == 0) store_q(qb == 2 ? 0 : qb + 1);  // the next tile's queries
        __builtin_amdgcn_sched_barrier(0);
        // all 16 basis operands of the stage are read first, so that the
        // matrix core is not left waiting on one LDS round trip per pair
        const unsigned char* sb = L.bring[G & 1];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int mt = 0; mt < 8; ++mt) aop[ks][mt] = lds16(sb, ra[ks][mt & 1] + 2048 * mt);
        // this producer's quarter of stage G + 1 into the other buffer
        stage_store((int)((G + 1) & 1), sreg[(s + 1) % NR]);
        __builtin_amdgcn_sched_barrier(0);
      };
      // the coefficient operand of stage s, k-step ks, token half nt
      auto coeff_op = [&](int s, int ks, int nt) -> bf16x8 {
        if constexpr (!CI4) return cv[s][ks][nt];
        else return dequant8(cq[s][nt][ks], csc[s][nt]);
      };
      // ---- the end of step s: the fp64 angle reduction of the step (the next
      //      tile's rotations, one per step from step 1 on, off the tail)
      //      and the loads for later stages
      auto step_end = [&](int s) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (s == (NR > 1 ? (1 + k < NR - 1 ? 1 + k : NR - 1) : 0)) {
            rot_next[k] = rot_of((double)rc_next * kChunk * L.invf[(lane & 15) * 4 + k]);
            // keep the work in this step (the compiler would otherwise sink it into the tail)
            asm volatile("" : "+v"(rot_next[k].x), "+v"(rot_next[k].y));
          }
        }
      };
      // Loads for later stages, issued after the step's products so that a
      // full memory pipeline stalls nothing the step needs.  (Past the last
      // tile they repeat the last tile: harmless, and they keep the code
      // branch-free.)
      auto step_loads = [&](int s) {
        __builtin_amdgcn_sched_barrier(0);
        if (s == NR - 1) load_q(tnn.bh);  // stored at step 0 of the next tile
        // stage G + SL: stage (s + SL) % NR of the tile (s + SL) / NR tiles on
        const int ahead = (s + SL) / NR;
        const int chead_l = ahead == 0 ? tc.chead : ahead == 1 ? tn.chead : tnn.chead;
        stage_load(bas_of(chead_l), (s + SL) % NR, sreg[(s + SL) % NR]);
        if constexpr (LG > 0) {
          if (s + LG < NR) gather(s + LG, tokA, cseq_c);
          else gather(s + LG - NR, tokB, cseq_n);
        }
      };

      // ---- reconstruction stages before the last: k-step major
#pragma unroll
      for (int s = 0; s < NR - 1; ++s) {
        step_begin(s);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          bf16x8 bop[NT];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) bop[nt] = coeff_op(s, ks, nt);
#pragma unroll
          for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              // a tile's first products start from zero (no accumulator to clear)
              acc[nt][mt] = mfma16(aop[ks][mt], bop[nt], s == 0 && ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[nt][mt]);
          if (ks == 0) pipe_post(&L.sync_stored, lane);  // stage G + 1 stored
        }
        step_end(s);
        step_loads(s);
      }

      // ---- the last stage, then the tail.  Its "stored" post goes at the end
      //      of the tail: the other producers need stage G + 1 only for the
      //      next tile, after their own tails, and so no branch separates the
      //      products from the work on their results (the first half's RoPE
      //      and QK can be scheduled under the second half's products).
      {
        constexpr int s = NR - 1;
        step_begin(s);
        step_end(s);
        // this tile's b2 for the consumers (for the group's partial): producer
        // w writes entries 64 (w % 2) + lane, producers 2 and 3 the values 0
        // and 1 write (indexed as slot base + lane, the lane offsets the other
        // writes use; not a branch)
        {
          const int ln = fresh(lane);
          (&L.b2f[i & 1][(slot & 1) * 64])[ln] = bf16_to_f32(b2raw);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const bf16x8 bop = coeff_op(s, ks, nt);
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
              acc[nt][mt] = mfma16(aop[ks][mt], bop, s == 0 && ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[nt][mt]);
          }
        // ---- K_pre done: acc[nt][mt][e] = K_pre[t][d], t = 16 nt + col,
        //      d = 32 (mt / 2) + 8 grp + 4 (mt % 2) + e.  Hand the bf16
        //      operands to the consumer in its register layout, one 16-token
        //      half at a time (the first half's results come first).
        unsigned char* hb = L.hand[i & 1][slot];
        // RoPE on packed fp16 pairs of consecutive frequencies: pair (d, d + 64)
        // = m-tiles (mt, mt + 4) of the same lane; the rotation is the chunk
        // start's composed with the offset's.  K_post stays fp16 (relative
        // error ~3 2^-11, below the 2^-9 of a bf16 operand) and feeds an fp16
        // QK.  One 16-token half at a time, so that only half of K_post is
        // held at once.  (Lane-derived offsets come from an opaque lane id:
        // formed here, not held across the tile loop.)
        const int lq = fresh(lane), cl = lq & 15;
        f16x8 qp[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          qp[ks] = *reinterpret_cast<const f16x8*>(&L.qh[qb][cl][8 * ((4 * ks + (lq >> 4)) ^ cl)]);
        f32x4 zacc[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            *reinterpret_cast<u32x4*>(hb + (nt * 4 + ks) * 1024 + lane * 16) =
                __builtin_bit_cast(u32x4, pack8(acc[nt][2 * ks], acc[nt][2 * ks + 1]));
          const int cs = 2 * nt + (cl >> 3);
          h2 kp[8][2];  // K_post of this half, [mt][e pair]
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            const int p0 = 32 * (mt >> 1) + 8 * (lq >> 4) + 4 * (mt & 1);
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
        pipe_softmax(zacc, slot_valid(tc.lt), a.scale_log2, lq >> 4, mrun, lrun, alpha, pa);
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
        pipe_post(&L.sync_stored, lane);  // stage G + 1 stored
        step_loads(s);
      }
      // tile i is handed to the consumers
      pipe_post(&L.sync_handed[i & 1], lane);
      qb = qb == 2 ? 0 : qb + 1;
      tc = tn;
      tn = tnn;
      tnn = pipe_next(a, tnn);
    }
  } else {
    // ===================================================================== consumer
    // Consumer w owns hidden units [64 w, 64 w + 64) of every token of the
    // tile (all four slots), with its W1 rows and b1 in registers, reloaded
    // when the head changes.  Step c of a tile runs the first MLP layer
    // of the tile's 16-token piece c (slot c / 2, half c % 2, from the K_pre
    // operands the producers handed over) and the GELU of piece c - 1; each
    // pair of pieces (one slot's 32 tokens) then meets that slot's softmax
    // weights in the PH product.  The last piece of a tile finishes at step 0
    // of the next tile (or after the loop).
    //
    // The slots' weights are relative to each slot's running maximum m_s
    // (its producer's).  A consumer puts them on one scale per tile,
    // M = max_s m_s, by multiplying slot s's weights by exp2(m_s - M), and
    // rescales its PH accumulator by exp2(M_old - M) (or clears it when a
    // group starts).  A group's PH is thus relative to the largest of its
    // slots' final maxima, and the merge weights it by the largest of the
    // slots' weights.
    //
    // Consumer w also takes slot w's residual rows (with slot w's weights and
    // running maximum, as the producer keeps them): loaded over steps 1-4
    // (int4: steps 1-2, with each lane's group scale), stored a step later
    // into slot w's residual region of LDS as bf16 rows (int4 rows dequantised
    // on the way), then R share += R^T x p^T at step 7.
    const int hq0 = 64 * slot;  // this wave's first hidden unit
    // W1 rows hq0 + 16 hn + col as MLP1 B operands (k = d = 32 ks + 8 grp .. + 7), and b1 of those units
    bf16x8 w1op[4][4];
    float b1v[4];
    auto load_w1 = [&](int chead) {
      const uint16_t* w = a.w1 + ((size_t)chead * kHidden + hq0 + col) * kHeadDim + 8 * grp;
#pragma unroll
      for (int hn = 0; hn < 4; ++hn)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) w1op[ks][hn] = load_bf16x8(w + 16 * hn * kHeadDim + 32 * ks);
      const uint16_t* bb = a.b1 + (size_t)chead * kHidden + hq0 + col;
#pragma unroll
      for (int hn = 0; hn < 4; ++hn) b1v[hn] = bf16_to_f32(bb[16 * hn]);
    };
    PipeCur tc = pipe_first(a, wg), tp = tc;  // this tile and the one before
    PipeCur tn = pipe_next(a, tc);
    load_w1(tc.chead);
    __syncthreads();

    f32x4 racc[8];   // slot w's residual share (+ nothing else), output space, scale m_w
    f32x4 phacc[4];  // PH of units hq0 + 16 hn + 4 grp + e, query col, scale M
#pragma unroll
    for (int nd = 0; nd < 8; ++nd) racc[nd] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int hn = 0; hn < 4; ++hn) phacc[hn] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 hacc[2][4];  // MLP1 of piece c in hacc[c & 1]
    h2 glo[4][2];      // GELU of the first piece of a pair
    f16x8 pq[4];       // each slot's weights of the tile being finished, on the scale M
    bf16x8 pab;        // slot w's weights, own scale (the residual product)
    float m_run = -__builtin_huge_valf();  // M after the current tile (query col)
    float m_w = 0.f, l_w = 0.f;            // slot w's running (m, l) after the current tile

    // GELU of piece pc (MLP1 result in hacc[pc & 1]); the second piece of a
    // pair completes PH of slot pc / 2:  D[h][j] += gelu^T[h][t] x p^T[t][j]
    auto finish_piece = [&](int pc) {
      h2 x[8];
#pragma unroll
      for (int hn = 0; hn < 4; ++hn) {
        x[2 * hn] = __builtin_convertvector(f32x2{hacc[pc & 1][hn][0], hacc[pc & 1][hn][1]}, h2);
        x[2 * hn + 1] = __builtin_convertvector(f32x2{hacc[pc & 1][hn][2], hacc[pc & 1][hn][3]}, h2);
      }
      gelu_h2x8(x);
      if ((pc & 1) == 0) {
#pragma unroll
        for (int hn = 0; hn < 4; ++hn) {
          glo[hn][0] = x[2 * hn];
          glo[hn][1] = x[2 * hn + 1];
        }
      } else {
#pragma unroll
        for (int hn = 0; hn < 4; ++hn) {
          const f16x8 a8 = __builtin_shufflevector(__builtin_shufflevector(glo[hn][0], glo[hn][1], 0, 1, 2, 3),
                                                   __builtin_shufflevector(x[2 * hn], x[2 * hn + 1], 0, 1, 2, 3),
                                                   0, 1, 2, 3, 4, 5, 6, 7);
          phacc[hn] = mfma16h(a8, pq[pc >> 1], phacc[hn]);
        }
      }
    };
    // group t's partials: slot w's output-space record (m_w, l_w, R share +
    // b2 l_w; b2 of the head from LDS, parity par) at slot 4 gx + w, and this
    // wave's quarter of the group's PH (units hq0 ..) in PH row 4 gx
    auto write_part = [&](const PipeCur& t, float m, float l, int par) {
      if (col >= g) return;
      const size_t sl = (size_t)t.bh * a.n_split + kPipeSlots * t.gx + slot;
      float* pp = a.part + (sl * g + col) * kPartStride;
      if (grp == 0) {
        pp[0] = m;
        pp[1] = l;
      }
#pragma unroll
      for (int nd = 0; nd < 8; ++nd)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int d = 16 * nd + 4 * grp + e;
          pp[2 + d] = fmaf(L.b2f[par][d], l, racc[nd][e]);
        }
      float* ph = a.ph + (((size_t)t.bh * a.n_ph + kPipeSlots * t.gx) * g + col) * kHidden + hq0 + 4 * grp;
#pragma unroll
      for (int hn = 0; hn < 4; ++hn) *reinterpret_cast<f32x4*>(ph + 16 * hn) = phacc[hn];
    };
    // slot w's value among four wave-uniform ones (no indexed register array)
    auto of_slot = [&](auto v0, auto v1, auto v2, auto v3) { return slot == 0 ? v0 : slot == 1 ? v1 : slot == 2 ? v2 : v3; };
    constexpr int RL = RI4 ? 2 : 8;  // 16-byte residual pieces per lane
    for (int i = 0; i < ntiles; ++i) {
      const int chead_c = tc.chead;
      const bool prev_end = i > 0 && tp.lt + 1 == tp.gend;   // the previous tile ended its group
      const bool new_grp = tc.lt == tc.gx * a.pipe_tpw;      // this tile starts one
      const unsigned char* hk = L.hand[i & 1][0];            // this tile's hand-off
      unsigned char* hr = L.rrow[slot];                      // slot w's residual rows
      u32x4 rres[RL];
      uint16_t rsc[RI4 ? RL : 1];
#pragma unroll
      for (int c = 0; c < NS; ++c) {
        if (c == 0) pipe_wait(&L.sync_handed[i & 1], 4u * (unsigned)(i / 2 + 1));  // tile i handed
        // ---- LDS operands first: K_pre of piece c, and at a tile start the
        //      slots' running softmax state and weights
        bf16x8 ka[4];
        {
          const unsigned char* hp = hk + (c >> 1) * kHandSlot + (c & 1) * 4096;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) ka[ks] = lds16(hp, ks * 1024 + lane * 16);
        }
        f32x4 sm[4];
        f16x8 praw[4];
        if (c == 0) {
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) {
            sm[s2] = L.sm[i & 1][s2][col];
            praw[s2] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4*>(hk + s2 * kHandSlot + kHandP + lane * 16));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        // ---- the previous piece (its products finished during the previous
        //      step; at a tile start: the previous tile's last piece with that
        //      tile's weights), under the K_pre reads; then at a tile start
        //      the rescale
        if (c > 0 || i > 0) finish_piece((c + NS - 1) % NS);
        if (c == 0) {
          if (prev_end) write_part(tp, m_w, l_w, (i - 1) & 1);
          // the previous tile's LDS (hand-off, weights, descriptors, b2) is read
          if (i > 0) pipe_post(&L.sync_released, lane);
          float mnew = -__builtin_huge_valf();
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) mnew = fmaxf(mnew, sm[s2][1]);
          const float fac = new_grp || m_run == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(m_run - mnew);
#pragma unroll
          for (int hn = 0; hn < 4; ++hn) phacc[hn] *= fac;
          m_run = mnew;
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) {
            const float f = sm[s2][1] == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(sm[s2][1] - mnew);
            const _Float16 fh = (_Float16)f;
            pq[s2] = praw[s2] * f16x8{fh, fh, fh, fh, fh, fh, fh, fh};
          }
          const f32x4 smw = of_slot(sm[0], sm[1], sm[2], sm[3]);
          const f16x8 pw = of_slot(praw[0], praw[1], praw[2], praw[3]);
          m_w = smw[1];
          l_w = smw[2];
#pragma unroll
          for (int nd = 0; nd < 8; ++nd) racc[nd] *= smw[0];
#pragma unroll
          for (int e = 0; e < 8; ++e) pab[e] = (__bf16)(float)pw[e];
        }
        // ---- MLP1 of piece c: D[t][h] = K_pre[t][d] x W1^T[d][h] (b1 initial value)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int hn = 0; hn < 4; ++hn)
            hacc[c & 1][hn] = mfma16(ka[ks], w1op[ks][hn],
                                     ks == 0 ? f32x4{b1v[hn], b1v[hn], b1v[hn], b1v[hn]} : hacc[c & 1][hn]);

        if (c == NS - 1) {
          // ---- residuals (at the last step, where the producers' tail is the
          //      longer part): bf16 rows t of slot w's region (stored at steps
          //      2-5); R share += R^T[d][t] x p^T[t][j].  The B operand (tokens
          //      4 grp + 0..3 and 16 + 4 grp + 0..3 of column d = 16 nd + col)
          //      comes from two transpose reads of the row-major rows.
          asm volatile("" ::: "memory");  // the reads below take bytes written under other types
          const int rb = (4 * grp + (col >> 2)) * kResRow + 8 * (col & 3);
#pragma unroll
          for (int nd = 0; nd < 8; ++nd) {
            const bf16x8 rop = bf16x8_of(lds_tr16(hr, rb + 32 * nd), lds_tr16(hr, rb + 16 * kResRow + 32 * nd));
            racc[nd] = mfma16(rop, pab, racc[nd]);
          }
        }
        // ---- loads for later steps, after this step's work: at the last
        //      piece of a head's last tile the next head's W1 (used from the
        //      next step on); slot w's residual rows over steps 1-4
        __builtin_amdgcn_sched_barrier(0);
        if (c == NS - 1 && tn.chead != chead_c) load_w1(tn.chead);
        if (c >= 1 && c <= 4) {
          // zeros where a token has none: reads past the end of the buffer return 0
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
            for (int u = 2 * (c - 1); u < 2 * c; ++u) {
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
            if (c <= RL) {
              // token 16 u + lane / 4: its 32 codes of group lane % 4, and that group's scale
              const int u = c - 1;
              const int t = 16 * u + (lane >> 2);
              const int rn = row_of(L.rdesc[i & 1][slot][2 * u + (lane >> 5)], t);
              rres[u] = buffer_ld16(rv, rn >= 0 ? (uint32_t)rn * 64 + (lane & 3) * 16 : nbytes, 0);
              rsc[u] = __builtin_amdgcn_raw_buffer_load_b16(rs, rn >= 0 ? (uint32_t)rn * 8 + (lane & 3) * 2 : sbytes, 0, 0);
            }
          }
        }
        // the residual rows loaded a step ago -> slot w's region, so that no
        // row is held in registers for longer than a step
        if constexpr (!RI4) {
          if (c >= 2 && c <= 5) {
#pragma unroll
            for (int u = 2 * (c - 2); u < 2 * (c - 1); ++u)
              *reinterpret_cast<u32x4*>(hr + (4 * u + (lane >> 4)) * kResRow + (lane & 15) * 16) = rres[u];
          }
        } else {
          // int4 rows are dequantised on the way: 32 bf16 values (64 bytes) of
          // group lane % 4 of token 16 u + lane / 4, in the bf16 row layout
          if (c >= 2 && c - 2 < RL) {
            const int u = c - 2;
            const float sc = f16_to_f32(rsc[u]);
            unsigned char* dst = hr + (16 * u + (lane >> 2)) * kResRow + (lane & 3) * 64;
#pragma unroll
            for (int k = 0; k < 4; ++k) *reinterpret_cast<u32x4*>(dst + 16 * k) = __builtin_bit_cast(u32x4, dequant8(rres[u][k], sc));
          }
        }
      }
      tp = tc;
      tc = tn;
      tn = pipe_next(a, tn);
    }
    // the last tile's last piece, and the partials of the last group
    finish_piece(NS - 1);
    write_part(tp, m_w, l_w, (ntiles - 1) & 1);
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
