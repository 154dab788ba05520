// Landmark scoring (GEMV on MFMA) and exact top-k chunk selection, gfx950.
//
// LowRAM review (agihunt.info), key paragraph: the prefix is cut into chunks
// whose mean key is a landmark; each step ranks the chunks against the
// current query and rebuilds only the top-k.  The score of chunk c for KV
// head h is the maximum over h's query heads j of q_j . L[c]; the k largest
// are kept, exact ties to the lower chunk id, output in ascending chunk id.
#include "common.h"
#include "internal.h"
#include "window.h"

// Grid cap of the score kernel (measured at 262K context, batch 28: 16384,
// i.e. 512 chunks per workgroup, beat 2048-8192 by 3-5% and 32768 by 1-2%)
#ifndef LOWRAM_SCORE_MAX_WG
#define LOWRAM_SCORE_MAX_WG 16384
#endif

namespace lowram {

// ---------------------------------------------------------------------------
// Scoring.  The landmark stream is the HBM-bound half of the step (4 flop/B).
// On the VALU it would cost one bf16->fp32 convert plus g FMAs per element
// and a 16-lane reduction per chunk, close to the whole VALU issue budget at
// full HBM rate; one v_mfma_f32_16x16x32_bf16 instead takes 16 landmarks x
// 32 dims per instruction.  A = the KV head's queries (rows j < g, zero rows
// above), B = 16 landmarks (columns), so lane l (< 16 per 16-lane group) ends
// up owning chunk c0 + l%16 with rows j = 4*(l/16) + e.  Each wave keeps 64
// landmarks (16 KiB) in flight while it multiplies the previous 64 out of LDS.
// ---------------------------------------------------------------------------
#ifndef LOWRAM_SCORE_WG_PER_CU
#define LOWRAM_SCORE_WG_PER_CU 2
#endif
// NBW: batches of 64 landmark rows per wave (a workgroup scores 256 NBW
// chunks), a template parameter so that the batch loop is straight-line code.
// The last win.n_tiles workgroups along x of each (sequence, KV head) run
// that head's exact-window tiles instead: the window needs neither the
// scores nor the selection, and its few rows ride along with the landmark
// stream instead of taking a launch of their own.
template <int NBW>
__global__ __launch_bounds__(256, LOWRAM_SCORE_WG_PER_CU) void score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ landmark,
    uint32_t* __restrict__ keys, float* __restrict__ scores_out, int n_cand, int n_heads_q,
    int n_heads_kv, int cache_bmul, int lm_rows, const ScoreWindow win) {
  constexpr int chunks_per_wg = 256 * NBW;
  const int b = blockIdx.z, h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, col = lane & 15;
  const int g = n_heads_q / n_heads_kv;
  __shared__ __attribute__((aligned(16))) unsigned char tile[4][64 * 256];

  const int wt = (int)blockIdx.x - ((int)gridDim.x - win.n_tiles);  // window tile, if >= 0
  if (wt >= 0) {
    const size_t head = (size_t)b * n_heads_kv + h;
    const size_t chead = (size_t)b * cache_bmul * n_heads_kv + h;
    f32x4 oacc[8];
    float wm, wl;
    window_wave(q + ((size_t)b * n_heads_q + (size_t)h * g) * kHeadDim,
                win.win_k + chead * (size_t)win.window_cap * kHeadDim,
                win.win_v + chead * (size_t)win.window_cap * kHeadDim, wt * kAttTokWG + wave * kAttTokWave,
                win.window, g, win.scale_log2, grp, col, oacc, wm, wl);
    write_partial4(reinterpret_cast<float*>(&tile[0][0]), reinterpret_cast<float*>(&tile[2][0]), oacc, wm, wl,
                   win.part + (head * (size_t)win.n_split + win.slot0 + wt) * g * kPartStride, g,
                   (int)threadIdx.x, wave, grp, col);
    return;
  }

  // the KV head's queries as the A operand (rows j < g; the loads are
  // unconditional, row clamped, and the rows from g on zeroed after them, so
  // that no wait on them precedes the landmark loads)
  bf16x8 qa[4];
  const uint16_t* qb = q + ((size_t)b * n_heads_q + (size_t)h * g) * kHeadDim;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qa[ks] = load_bf16x8(qb + min(col, g - 1) * kHeadDim + 32 * ks + 8 * grp);

  const size_t head = (size_t)b * n_heads_kv + h;
  const uint16_t* lm = landmark + ((size_t)b * cache_bmul * n_heads_kv + h) * (size_t)lm_rows * kHeadDim;
  uint32_t* kout = keys + head * (size_t)n_cand;
  float* sout = scores_out ? scores_out + head * (size_t)n_cand : nullptr;
  const int c_begin = blockIdx.x * chunks_per_wg;
  const int c_end = min(n_cand, c_begin + chunks_per_wg);
  // this workgroup's chunks of the outputs as buffer resources: writes past
  // c_end are dropped by the range check, so the writes need no branch (no
  // score output: a zero-length range, every write dropped)
  const uint32_t out_bytes = (uint32_t)max(0, c_end - c_begin) * 4u;
  const __amdgpu_buffer_rsrc_t kbuf = buffer_rsrc(kout + c_begin, out_bytes);
  const __amdgpu_buffer_rsrc_t sbuf = sout ? buffer_rsrc(sout + c_begin, out_bytes) : buffer_rsrc(kout + c_begin, 0u);

  // Landmark rows reach the MFMA through a per-wave LDS tile.  Each load
  // instruction takes 4 whole rows (1 KiB contiguous) with the non-temporal
  // policy (every 128-byte line is consumed whole by the instruction that
  // reads it); piece p of row r is stored at piece p ^ (r & 15), so that both
  // the stores and the B-operand reads (16 rows, one 16-byte piece each) are
  // conflict-free.  Two batches of 64 rows are in flight per wave, in two
  // register buffers that take turns: a batch goes to LDS, its buffer is
  // refilled with the batch two ahead, and the batch is multiplied while the
  // other buffer's loads fly.  Loads and writes are unconditional (rows past
  // the list are clamped to its last one, writes past c_end are dropped), so
  // the in-order wait before a batch's stores covers that batch's loads only.
  unsigned char* my = tile[wave];
  auto load_rows = [&](int c0, u32x4 (&v)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int cc = min(c0 + 4 * i + grp, n_cand - 1);
      v[i] = load_nt16(lm + (size_t)cc * kHeadDim + 8 * col);
    }
  };
  u32x4 rbuf[2][16];
  const int cw = c_begin + wave * 64;  // this wave's first row
  load_rows(cw, rbuf[0]);
  if constexpr (NBW > 1) load_rows(cw + 256, rbuf[1]);
  if (col >= g)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qa[ks] = zero_bf16x8();
#pragma unroll
  for (int bi = 0; bi < NBW; ++bi) {
    const int c0 = cw + 256 * bi;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = 4 * i + grp;
      *reinterpret_cast<u32x4*>(my + r * 256 + 16 * (col ^ (r & 15))) = rbuf[bi & 1][i];
    }
    if (bi + 2 < NBW) load_rows(c0 + 512, rbuf[bi & 1]);
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const int r = 16 * gi + col;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        acc = mfma16(qa[ks], __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                 my + r * 256 + 16 * ((4 * ks + grp) ^ (r & 15)))), acc);
      float s = -__builtin_huge_valf();
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * grp + e < g) s = fmaxf(s, acc[e]);
      s = fmaxf(s, __shfl_xor(s, 16));
      s = fmaxf(s, __shfl_xor(s, 32));
      // (the four lanes of a chunk hold the same maximum and write it alike)
      const uint32_t off = (uint32_t)(c0 + 16 * gi + col - c_begin) * 4u;
      __builtin_amdgcn_raw_buffer_store_b32(score_key(s), kbuf, off, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s), sbuf, off, 0, 0);
    }
  }
}

// Scoring for many queries against ONE shared context: the 16 A rows of the
// MFMA tile hold 16 / G queries' G query heads (G a power of two <= 16), so
// each landmark block streamed serves all of them.  Lane (grp, col) receives
// rows 4 grp + e of chunk col; a query's G rows lie in one lane (G <= 4,
// max over e) or span 16-lane groups (G = 8, 16: max across them).
template <int G>
__global__ __launch_bounds__(256, LOWRAM_SCORE_WG_PER_CU) void score_multi_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ landmark,
    uint32_t* __restrict__ keys, float* __restrict__ scores_out, int n_cand, int n_heads_q,
    int n_heads_kv, int chunks_per_wg, int nq, int lm_rows) {
  constexpr int QG = 16 / G;  // queries per tile
  const int qb = blockIdx.z, h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, col = lane & 15;

  // A row col = query qb * QG + col / G, head h * G + col % G
  const int aq = qb * QG + col / G;
  bf16x8 qa[4];
  const uint16_t* qrow = q + ((size_t)aq * n_heads_q + (size_t)h * G + col % G) * kHeadDim;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) qa[ks] = aq < nq ? load_bf16x8(qrow + 32 * ks + 8 * grp) : zero_bf16x8();

  const uint16_t* lm = landmark + (size_t)h * lm_rows * kHeadDim;
  const int c_begin = blockIdx.x * chunks_per_wg;
  const int c_end = min(n_cand, c_begin + chunks_per_wg);
  auto load_group = [&](int c0, bf16x8 (&lv)[4][4]) {
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int cc = min(c0 + 16 * gi + col, n_cand - 1);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) lv[gi][ks] = load_bf16x8(lm + (size_t)cc * kHeadDim + 32 * ks + 8 * grp);
    }
  };
  bf16x8 cur[4][4], nxt[4][4];
  int c0 = c_begin + wave * 64;
  if (c0 < c_end) load_group(c0, cur);
  for (; c0 < c_end; c0 += 256) {
    if (c0 + 256 < c_end) load_group(c0 + 256, nxt);
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mfma16(qa[ks], cur[gi][ks], acc);
      const int c = c0 + 16 * gi + col;
      if constexpr (G <= 4) {
        // this lane holds rows 4 grp .. 4 grp + 3 = queries (4 grp) / G ..
#pragma unroll
        for (int e0 = 0; e0 < 4; e0 += G) {
          float sc = acc[e0];
#pragma unroll
          for (int e = 1; e < G; ++e) sc = fmaxf(sc, acc[e0 + e]);
          const int qi = qb * QG + (4 * grp + e0) / G;
          if (qi < nq && c < c_end) {
            const size_t o = ((size_t)qi * n_heads_kv + h) * n_cand + c;
            keys[o] = score_key(sc);
            if (scores_out) scores_out[o] = sc;
          }
        }
      } else {
        float sc = fmaxf(fmaxf(acc[0], acc[1]), fmaxf(acc[2], acc[3]));
        sc = fmaxf(sc, __shfl_xor(sc, 16));
        if constexpr (G == 16) sc = fmaxf(sc, __shfl_xor(sc, 32));
        const int qi = qb * QG + (4 * grp) / G;
        const bool writer = G == 16 ? grp == 0 : (grp & 1) == 0;
        if (writer && qi < nq && c < c_end) {
          const size_t o = ((size_t)qi * n_heads_kv + h) * n_cand + c;
          keys[o] = score_key(sc);
          if (scores_out) scores_out[o] = sc;
        }
      }
    }
#pragma unroll
    for (int gi = 0; gi < 4; ++gi)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) cur[gi][ks] = nxt[gi][ks];
  }
}

// ---------------------------------------------------------------------------
// Exact top-k by radix select on the order-preserving keys.  Three passes on
// the key bits [31:20], [19:8], [7:0] find the k-th largest key T and how many
// keys equal to T are still needed; an ordered compaction then keeps every
// key > T and the first `need` keys == T in candidate order.  Candidates are
// in ascending chunk order, so the output is ascending.  One workgroup of
// 1024 threads per (sequence, KV head).
//
// Thread t owns the `per` consecutive candidates [per t, per t + per), per the
// smallest power of two with 1024 per >= n_cand.  Lists of up to 32768
// candidates keep each thread's keys in registers for the whole selection
// (select_reg_kernel, per a template parameter, so every loop over a
// thread's keys is unrolled); longer lists re-read them from L2 in every pass
// (select_l2_kernel).  12-bit first digits spread the fp32 exponent over 4096
// bins so few lanes of an LDS atomic hit the same bin; the digit search uses
// DPP wave scans with one LDS exchange.  The compaction counts each
// thread's keys > T and == T, takes one block-wide exclusive scan of the two
// counts, and has every thread write its own selected candidates in order:
// no per-key ballot.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelBins = 4096;
constexpr int kSelRegKeys = 32 * kSelThreads;  // longest list kept in registers
constexpr int kSelBatch = 8;                   // L2 variant: loads a thread has in flight at once
constexpr int kSelShift[3] = {20, 8, 0};
constexpr int kSelBits[3] = {12, 12, 8};

struct SelLds {
  uint32_t hist[kSelBins];
  uint32_t wsum[2][kSelWaves];
  uint32_t found[2];
  uint32_t spare[64];  // one word per lane: the passes' and the compaction's writes for keys they skip
};

// inclusive scan of x over the 64 lanes of a wave, from lane 0 up, on DPP
// moves: row shifts by 1, 2, 4 and 8 scan each row of 16 lanes (lanes
// shifted in from outside the row add 0), then the last lane of row 0 is
// added to row 1 and of row 2 to row 3 (row_bcast:15 on rows 1 and 3), and
// the last lane of row 1 to rows 2 and 3 (row_bcast:31); six vector adds,
// no LDS crossbar round trip
__device__ __forceinline__ uint32_t wave_scan_up(uint32_t x) {
  x += __builtin_amdgcn_update_dpp(0u, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0u, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0u, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0u, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0u, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0u, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// inclusive scan of x over the 64 lanes of a wave, from the highest lane down
__device__ __forceinline__ uint32_t wave_scan_down(uint32_t x) {
  const uint32_t up = wave_scan_up(x);
  return __builtin_amdgcn_readlane(up, 63) - up + x;
}

// The digit of one radix pass: the bin D of hist (nbins bins, kSelThreads
// threads) where the count of keys in higher bins first reaches kk.  Thread t
// owns bins [bpt t, bpt t + bpt).  Leaves found[0] = D and found[1] = the
// count in the bins above D, read after the barrier at the end; wsum (one word
// per wave) is scratch.  hist may be LDS or global memory.
template <class H>
__device__ __forceinline__ void pick_digit(H hist, int nbins, uint32_t kk, uint32_t* wsum, uint32_t* found) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bpt = nbins >= kSelThreads ? nbins / kSelThreads : 1;
  const bool owner = tid * bpt < nbins;
  uint32_t mine = 0;
  if (owner)
    for (int j = 0; j < bpt; ++j) mine += hist[tid * bpt + j];
  const uint32_t incl = wave_scan_down(mine);  // this lane and above, in the wave
  if (lane == 0) wsum[wave] = incl;
  __syncthreads();
  uint32_t above = incl - mine;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) above += w > wave ? wsum[w] : 0u;  // (independent reads, not a loop of round trips)
  if (owner) {
    for (int j = bpt - 1; j >= 0; --j) {
      const uint32_t c = hist[tid * bpt + j];
      if (above < kk && kk <= above + c) {
        found[0] = tid * bpt + j;
        found[1] = above;
      }
      above += c;
    }
  }
  __syncthreads();
}

// Exclusive scans over the block, in thread order, of two per-thread counts.
__device__ __forceinline__ void block_scan2(uint32_t a, uint32_t b, uint32_t (*wsum)[kSelWaves], uint32_t& a_before,
                                            uint32_t& b_before) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t a_incl = wave_scan_up(a), b_incl = wave_scan_up(b);
  if (lane == 63) {
    wsum[0][wave] = a_incl;
    wsum[1][wave] = b_incl;
  }
  __syncthreads();
  a_before = a_incl - a;
  b_before = b_incl - b;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    a_before += w < wave ? wsum[0][w] : 0u;
    b_before += w < wave ? wsum[1][w] : 0u;
  }
}

// minimum of x over the 64 lanes of a wave (wave-uniform result): DPP row
// shifts take each row of 16 lanes to its minimum in lane 15 of the row
// (a lane with no source keeps its own value), then the four rows meet in
// scalar registers
__device__ __forceinline__ uint32_t wave_min(uint32_t x) {
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0x111, 0xf, 0xf, false));  // row_shr:1
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0x112, 0xf, 0xf, false));  // row_shr:2
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0x114, 0xf, 0xf, false));  // row_shr:4
  x = min(x, (uint32_t)__builtin_amdgcn_update_dpp(x, x, 0x118, 0xf, 0xf, false));  // row_shr:8
  return min(min(__builtin_amdgcn_readlane(x, 15), __builtin_amdgcn_readlane(x, 31)),
             min(__builtin_amdgcn_readlane(x, 47), __builtin_amdgcn_readlane(x, 63)));
}

// The selection's common start: pads sel_out past k_eff with -1 and takes
// every candidate when there are no more than k.  Returns true when done.
__device__ __forceinline__ bool select_trivial(const int32_t* ids, int32_t* so, int32_t* so2, int n_cand, int k,
                                               int k_eff) {
  const int tid = threadIdx.x;
  if (so2)
    for (int i = k_eff + tid; i < k; i += kSelThreads) so2[i] = -1;
  if (n_cand > k) return false;
  for (int i = tid; i < n_cand; i += kSelThreads) {
    const int32_t c = ids ? ids[i] : i;
    so[i] = c;
    if (so2) so2[i] = c;
  }
  return true;
}

template <int LP>
__global__ __launch_bounds__(kSelThreads) void select_reg_kernel(
    const uint32_t* __restrict__ keys, const int32_t* __restrict__ cand_ids,
    int32_t* __restrict__ sel, int32_t* __restrict__ sel_out, int n_cand, int k, int n_heads_kv,
    int cache_bmul) {
  constexpr int PER = 1 << LP;
  __shared__ SelLds S;
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const size_t head = (size_t)b * n_heads_kv + h;
  const uint32_t* kg = keys + head * (size_t)n_cand;
  const int32_t* ids = cand_ids ? cand_ids + ((size_t)b * cache_bmul * n_heads_kv + h) * (size_t)n_cand : nullptr;
  const int k_eff = min(k, n_cand);
  int32_t* so = sel + head * (size_t)k_eff;
  int32_t* so2 = sel_out ? sel_out + head * (size_t)k : nullptr;
  if (select_trivial(ids, so, so2, n_cand, k, k_eff)) return;

  const int i_begin = tid * PER;                         // this thread's first candidate
  const int cnt = max(0, min(PER, n_cand - i_begin));    // and how many it owns
  // key j of this thread is in the list when bit j of vmask is set; a wave
  // whose threads all own PER keys (every wave but the list's last) takes
  // the loops below without that test (the first pass then has no branch).
  // (A bit mask, not j < cnt: the compiler would turn that into a run-time
  // trip count and index the key registers dynamically.)
  const uint32_t vmask = cnt >= 32 ? 0xffffffffu : (1u << cnt) - 1u;
  const bool wave_full = __all(cnt == PER);
  // This thread's keys.  With 16-byte-aligned lists: at most 4 keys per
  // thread, one 16-byte load each (consecutive lanes, consecutive pieces);
  // more, through LDS, so that every load instruction of a wave reads
  // consecutive 16-byte pieces: piece g of the list (owner g / P4, piece
  // g % P4 of it) goes to slot owner P4 + (piece ^ ((owner >> SW) & (P4 - 1))),
  // which keeps both the stores and each thread's reads of its own pieces off
  // shared banks.  Otherwise one key at a time with indices clamped into the
  // list.  (Keys past the list's end hold anything: vmask excludes them.)
  uint32_t kx[PER];
  const bool aligned = (reinterpret_cast<uintptr_t>(kg) & 15) == 0;
  if constexpr (PER >= 8) {
    constexpr int P4 = PER / 4;                    // 16-byte pieces per thread
    constexpr int SW = P4 == 2 ? 3 : P4 == 4 ? 2 : 1;
    __shared__ u32x4 stage[PER * kSelThreads / 4];
    if (aligned) {
      const int n4 = n_cand >> 2, rem = n_cand & 3;
      const u32x4* kg4 = reinterpret_cast<const u32x4*>(kg);
      u32x4 v[P4];
#pragma unroll
      for (int q = 0; q < P4; ++q) {
        const int g = tid + kSelThreads * q;
        if (g < n4) {
          v[q] = kg4[g];
        } else {  // the list's last, partial piece (indices clamped), or past the end
#pragma unroll
          for (int e = 0; e < 4; ++e) v[q][e] = kg[min(4 * g + e, n_cand - 1)];
        }
      }
#pragma unroll
      for (int q = 0; q < P4; ++q) {
        const int g = tid + kSelThreads * q, o = g / P4, pc = g % P4;
        if (g < n4 + (rem ? 1 : 0)) stage[o * P4 + (pc ^ ((o >> SW) & (P4 - 1)))] = v[q];
      }
      __syncthreads();
#pragma unroll
      for (int pc = 0; pc < P4; ++pc) {
        const u32x4 w = stage[tid * P4 + (pc ^ ((tid >> SW) & (P4 - 1)))];
        kx[4 * pc] = w[0];
        kx[4 * pc + 1] = w[1];
        kx[4 * pc + 2] = w[2];
        kx[4 * pc + 3] = w[3];
      }
    } else {
#pragma unroll
      for (int j = 0; j < PER; ++j) kx[j] = kg[min(i_begin + j, n_cand - 1)];
    }
  } else if (PER == 4 && cnt == PER && aligned) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(kg + i_begin);
#pragma unroll
    for (int e = 0; e < PER; ++e) kx[e] = w[e];
  } else {
#pragma unroll
    for (int j = 0; j < PER; ++j) kx[j] = kg[min(i_begin + j, n_cand - 1)];
  }

  // A lower bound lb on the k-th largest key, so that the histograms skip
  // keys that cannot be selected (the first pass's 12 bits are mostly the
  // fp32 exponent, and its atomics crowd into few bins).  Take each thread's
  // r-th largest key (r = 1 or 2), minimised over the m threads that own at
  // least r keys: those threads hold m r keys at or above the minimum, so
  // for k <= m r the k-th largest is at or above it too.  A key below lb
  // lies below the threshold T, in a bin no higher than T's: leaving it out
  // changes neither the counts above T's bin nor which bin reaches k first,
  // in any pass.  (lb = 0 when k exceeds both products.)
  uint32_t lb = 0;
  const int m1 = min(kSelThreads, (n_cand + PER - 1) / PER);
  const int m2 = min(kSelThreads, n_cand / PER + (n_cand % PER >= 2 ? 1 : 0));
  const int r = k <= m1 ? 1 : k <= 2 * m2 ? 2 : 0;  // uniform over the workgroup
  {
    if (r > 0) {
      uint32_t t1 = 0, t2 = 0;  // this thread's largest and second largest key
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const uint32_t x = ((vmask >> j) & 1u) ? kx[j] : 0u;
        t2 = max(t2, min(t1, x));
        t1 = max(t1, x);
      }
      const uint32_t v = cnt < r ? 0xffffffffu : r == 1 ? t1 : t2;
      const uint32_t wm = wave_min(v);
      if ((tid & 63) == 0) S.wsum[1][tid >> 6] = wm;  // read after the first pass's barrier
    }
  }

  uint32_t prefix = 0, pmask = 0, kk = (uint32_t)k;
  bool whole_bin = false;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = kSelShift[pass], nbins = 1 << kSelBits[pass];
    const uint32_t dmask = (uint32_t)nbins - 1;
    for (int i = tid; i < nbins; i += kSelThreads) S.hist[i] = 0;
    __syncthreads();
    if (pass == 0 && r > 0) {
      lb = 0xffffffffu;
#pragma unroll
      for (int w = 0; w < kSelWaves; ++w) lb = min(lb, S.wsum[1][w]);
    }
    {
      // one LDS atomic per key and no branch in the loop: a key outside the
      // prefix or below lb counts in its lane's spare word (never read)
      uint32_t* const spare = &S.spare[tid & 63];
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const bool in = (wave_full || ((vmask >> j) & 1u)) && (kx[j] & pmask) == prefix && kx[j] >= lb;
        atomicAdd(in ? &S.hist[(kx[j] >> shift) & dmask] : spare, 1u);
      }
    }
    __syncthreads();
    pick_digit(S.hist, nbins, kk, S.wsum[0], S.found);
    const uint32_t digit = S.found[0];
    const uint32_t in_bin = S.hist[digit];
    kk -= S.found[1];
    prefix |= digit << shift;
    pmask |= dmask << shift;
    // The chosen bin holds exactly the kk keys still needed, and it lies
    // wholly at or above lb, so the counts left none of its keys out: the k
    // largest are then exactly the keys >= the bin's lowest value (prefix),
    // and the later passes are skipped with the same result.
    whole_bin = pass < 2 && kk == in_bin && prefix > 0 && prefix >= lb;
    __syncthreads();  // hist, wsum and found are reused next
    if (whole_bin) break;
  }
  // select the keys > T and the first `need` keys == T
  const uint32_t T = whole_bin ? prefix - 1 : prefix, need = whole_bin ? 0u : kk;

  // ordered compaction: this thread's counts of keys > T and == T, their
  // exclusive scans over the block, then this thread's selected candidates
  uint32_t ngt = 0, neq = 0;
  if (wave_full) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      ngt += kx[j] > T ? 1u : 0u;
      neq += kx[j] == T ? 1u : 0u;
    }
  } else {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const bool in = (vmask >> j) & 1u;
      ngt += (in && kx[j] > T) ? 1u : 0u;
      neq += (in && kx[j] == T) ? 1u : 0u;
    }
  }
  uint32_t gt_run, eq_run;
  block_scan2(ngt, neq, S.wsum, gt_run, eq_run);
  // Each thread puts its selected candidates' list indices at their output
  // positions; up to kSelBins of them go to LDS (the histogram's space, free
  // after the last pass) and then out in one coalesced pass, with the id
  // lookup done there; longer outputs are written directly.
  const bool staged = k_eff <= kSelBins;
  const bool mine = !(gt_run + min(eq_run, need) >= (uint32_t)k_eff || (ngt == 0 && (neq == 0 || eq_run >= need)));
  if (staged) {
    // one store per key and no branch in the loop: an unselected key's
    // index goes to this lane's spare word
    if (mine) {
      uint32_t* const spare = &S.spare[tid & 63];
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const bool in = (vmask >> j) & 1u;
        const bool gt = in && kx[j] > T, eq = in && kx[j] == T;
        const uint32_t pos = gt_run + min(eq_run, need);
        const bool put = (gt || (eq && eq_run < need)) && pos < (uint32_t)k_eff;
        *(put ? &S.hist[min(pos, (uint32_t)kSelBins - 1)] : spare) = (uint32_t)(i_begin + j);
        gt_run += gt ? 1u : 0u;
        eq_run += eq ? 1u : 0u;
      }
    }
  } else if (mine) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const bool in = (vmask >> j) & 1u;
      const bool gt = in && kx[j] > T, eq = in && kx[j] == T;
      if (gt || (eq && eq_run < need)) {
        const uint32_t pos = gt_run + min(eq_run, need);
        if (pos < (uint32_t)k_eff) {
          const int i = i_begin + j;
          const int32_t c = ids ? ids[i] : i;
          so[pos] = c;
          if (so2) so2[pos] = c;
        }
      }
      gt_run += gt ? 1u : 0u;
      eq_run += eq ? 1u : 0u;
    }
  }
  if (staged) {
    __syncthreads();
    for (int p = tid; p < k_eff; p += kSelThreads) {
      const int i = (int)S.hist[p];
      const int32_t c = ids ? ids[i] : i;
      so[p] = c;
      if (so2) so2[p] = c;
    }
  }
}

__global__ __launch_bounds__(kSelThreads) void select_l2_kernel(
    const uint32_t* __restrict__ keys, const int32_t* __restrict__ cand_ids,
    int32_t* __restrict__ sel, int32_t* __restrict__ sel_out, int n_cand, int k, int n_heads_kv,
    int cache_bmul) {
  __shared__ SelLds S;
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const size_t head = (size_t)b * n_heads_kv + h;
  const uint32_t* kg = keys + head * (size_t)n_cand;
  const int32_t* ids = cand_ids ? cand_ids + ((size_t)b * cache_bmul * n_heads_kv + h) * (size_t)n_cand : nullptr;
  const int k_eff = min(k, n_cand);
  int32_t* so = sel + head * (size_t)k_eff;
  int32_t* so2 = sel_out ? sel_out + head * (size_t)k : nullptr;
  if (select_trivial(ids, so, so2, n_cand, k, k_eff)) return;

  int lp = 0;  // per = 2^lp candidates per thread
  while (((long long)kSelThreads << lp) < n_cand) ++lp;
  const int per = 1 << lp;
  const int i_begin = tid << lp;                                  // this thread's first candidate
  const int cnt = max(0, min(per, n_cand - i_begin));             // and how many it owns
  auto key_of = [&](int j) -> uint32_t { return kg[i_begin + j]; };  // key j of this thread (j < cnt)

  uint32_t prefix = 0, pmask = 0, kk = (uint32_t)k;
  bool whole_bin = false;
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = kSelShift[pass], nbins = 1 << kSelBits[pass];
    const uint32_t dmask = (uint32_t)nbins - 1;
    for (int i = tid; i < nbins; i += kSelThreads) S.hist[i] = 0;
    __syncthreads();
    for (int j0 = 0; j0 < cnt; j0 += kSelBatch) {
      uint32_t kx[kSelBatch];  // a batch of reads before its atomics
#pragma unroll
      for (int u = 0; u < kSelBatch; ++u) kx[u] = key_of(min(j0 + u, cnt - 1));
#pragma unroll
      for (int u = 0; u < kSelBatch; ++u)
        if (j0 + u < cnt && (kx[u] & pmask) == prefix) atomicAdd(&S.hist[(kx[u] >> shift) & dmask], 1u);
    }
    __syncthreads();
    pick_digit(S.hist, nbins, kk, S.wsum[0], S.found);
    const uint32_t digit = S.found[0];
    const uint32_t in_bin = S.hist[digit];
    kk -= S.found[1];
    prefix |= digit << shift;
    pmask |= dmask << shift;
    // as in select_reg_kernel (every key is counted here): a bin holding
    // exactly the keys still needed ends the passes
    whole_bin = pass < 2 && kk == in_bin && prefix > 0;
    __syncthreads();  // hist, wsum and found are reused next
    if (whole_bin) break;
  }
  const uint32_t T = whole_bin ? prefix - 1 : prefix, need = whole_bin ? 0u : kk;

  uint32_t ngt = 0, neq = 0;
  for (int j0 = 0; j0 < cnt; j0 += kSelBatch) {
    uint32_t kx[kSelBatch];
#pragma unroll
    for (int u = 0; u < kSelBatch; ++u) kx[u] = key_of(min(j0 + u, cnt - 1));
#pragma unroll
    for (int u = 0; u < kSelBatch; ++u) {
      const bool in = j0 + u < cnt;
      ngt += (in && kx[u] > T) ? 1u : 0u;
      neq += (in && kx[u] == T) ? 1u : 0u;
    }
  }
  uint32_t gt_run, eq_run;
  block_scan2(ngt, neq, S.wsum, gt_run, eq_run);
  if (gt_run + min(eq_run, need) >= (uint32_t)k_eff || (ngt == 0 && (neq == 0 || eq_run >= need))) return;
  for (int j0 = 0; j0 < cnt; j0 += kSelBatch) {
    uint32_t kx[kSelBatch];
#pragma unroll
    for (int u = 0; u < kSelBatch; ++u) kx[u] = key_of(min(j0 + u, cnt - 1));
#pragma unroll
    for (int u = 0; u < kSelBatch; ++u) {
      const int j = j0 + u;
      const bool in = j < cnt;
      const bool gt = in && kx[u] > T, eq = in && kx[u] == T;
      if (gt || (eq && eq_run < need)) {
        const uint32_t pos = gt_run + min(eq_run, need);
        if (pos < (uint32_t)k_eff) {
          const int i = i_begin + j;
          const int32_t c = ids ? ids[i] : i;
          so[pos] = c;
          if (so2) so2[pos] = c;
        }
      }
      gt_run += gt ? 1u : 0u;
      eq_run += eq ? 1u : 0u;
    }
  }
}

// ---------------------------------------------------------------------------
// The same exact top-k for few long lists (the cache builder's residual
// ranking: one list of P tokens per KV head): each list is cut into slices
// of kSplitSlice keys so that many workgroups share the passes.  Per radix
// pass, every slice adds its LDS histogram to the list's global histogram,
// then one workgroup per list picks the digit (and clears the histogram for
// the next pass); finally each slice counts its keys > T and == T, and an
// ordered compaction places them after the counts of the slices before it.
// State per list: {prefix, pmask, still needed, k}.
// ---------------------------------------------------------------------------
constexpr int kSplitSlice = 8192;
constexpr int kSplitThreads = 256;

struct SplitWs {
  uint32_t* hist;    // [L][kSelBins]
  uint32_t* state;   // [L][4]
  uint32_t* counts;  // [L][n_slices][2]
};

__global__ __launch_bounds__(kSplitThreads) void split_init_kernel(SplitWs w, int k) {
  const int l = blockIdx.x;
  for (int i = threadIdx.x; i < kSelBins; i += kSplitThreads) w.hist[(size_t)l * kSelBins + i] = 0u;
  if (threadIdx.x == 0) {
    w.state[4 * l + 0] = 0u;
    w.state[4 * l + 1] = 0u;
    w.state[4 * l + 2] = (uint32_t)k;
    w.state[4 * l + 3] = (uint32_t)k;
  }
}

__global__ __launch_bounds__(kSplitThreads) void split_hist_kernel(const uint32_t* __restrict__ keys, SplitWs w,
                                                                   int n, int shift, uint32_t dmask) {
  __shared__ uint32_t hist[kSelBins];
  const int l = blockIdx.y;
  const uint32_t prefix = w.state[4 * l], pmask = w.state[4 * l + 1];
  for (int i = threadIdx.x; i < kSelBins; i += kSplitThreads) hist[i] = 0u;
  __syncthreads();
  const uint32_t* kl = keys + (size_t)l * n;
  const int i0 = blockIdx.x * kSplitSlice, i1 = min(n, i0 + kSplitSlice);
  for (int i = i0 + threadIdx.x; i < i1; i += kSplitThreads) {
    const uint32_t key = kl[i];
    if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
  }
  __syncthreads();
  uint32_t* gh = w.hist + (size_t)l * kSelBins;
  for (int i = threadIdx.x; i <= (int)dmask; i += kSplitThreads)
    if (hist[i]) atomicAdd(&gh[i], hist[i]);
}

// One workgroup per list: the digit whose higher bins first reach the
// needed count; clears the histogram for the next pass.
__global__ __launch_bounds__(kSelThreads) void split_digit_kernel(SplitWs w, int shift, uint32_t dmask) {
  __shared__ uint32_t wsum[kSelWaves];
  __shared__ uint32_t found[2];
  const int l = blockIdx.x, tid = threadIdx.x;
  uint32_t* gh = w.hist + (size_t)l * kSelBins;
  const int nbins = (int)dmask + 1;
  const uint32_t kk = w.state[4 * l + 2];
  pick_digit(gh, nbins, kk, wsum, found);
  const int bpt = nbins >= kSelThreads ? nbins / kSelThreads : 1;
  if (tid * bpt < nbins)
    for (int j = 0; j < bpt; ++j) gh[tid * bpt + j] = 0u;
  if (tid == 0) {
    w.state[4 * l + 0] |= found[0] << shift;
    w.state[4 * l + 1] |= dmask << shift;
    w.state[4 * l + 2] = kk - found[1];
  }
}

// Keys > T and == T of each slice (T = the k-th largest key).
__global__ __launch_bounds__(kSplitThreads) void split_count_kernel(const uint32_t* __restrict__ keys, SplitWs w,
                                                                    int n, int n_slices) {
  __shared__ uint32_t part[2][kSplitThreads / 64];
  const int l = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t T = w.state[4 * l];
  const uint32_t* kl = keys + (size_t)l * n;
  const int i0 = blockIdx.x * kSplitSlice, i1 = min(n, i0 + kSplitSlice);
  uint32_t ngt = 0, neq = 0;
  for (int i = i0 + threadIdx.x; i < i1; i += kSplitThreads) {
    const uint32_t key = kl[i];
    ngt += key > T;
    neq += key == T;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    ngt += __shfl_xor(ngt, o);
    neq += __shfl_xor(neq, o);
  }
  if (lane == 0) {
    part[0][wave] = ngt;
    part[1][wave] = neq;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t a = 0, e = 0;
    for (int v = 0; v < kSplitThreads / 64; ++v) {
      a += part[0][v];
      e += part[1][v];
    }
    w.counts[((size_t)l * n_slices + blockIdx.x) * 2 + 0] = a;
    w.counts[((size_t)l * n_slices + blockIdx.x) * 2 + 1] = e;
  }
}

// Ordered compaction of one slice: wave v walks its quarter of the slice 64
// keys at a time; ballots rank each key among the earlier ones.
__global__ __launch_bounds__(kSplitThreads) void split_compact_kernel(const uint32_t* __restrict__ keys, SplitWs w,
                                                                      int32_t* __restrict__ sel, int n, int n_slices,
                                                                      int sel_stride) {
  constexpr int kW = kSplitThreads / 64;
  __shared__ uint32_t wsum[2][kW];
  const int l = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t T = w.state[4 * l], need = w.state[4 * l + 2], k = w.state[4 * l + 3];
  const uint32_t* kl = keys + (size_t)l * n;
  int32_t* so = sel + (size_t)l * sel_stride;
  uint32_t gt_run = 0, eq_run = 0;
  for (int s2 = 0; s2 < (int)blockIdx.x; ++s2) {
    gt_run += w.counts[((size_t)l * n_slices + s2) * 2 + 0];
    eq_run += w.counts[((size_t)l * n_slices + s2) * 2 + 1];
  }
  const int i0 = blockIdx.x * kSplitSlice, i1 = min(n, i0 + kSplitSlice);
  const int per = (i1 - i0 + kW - 1) / kW;
  const int w0 = min(i1, i0 + wave * per), w1 = min(i1, w0 + per);
  const uint64_t below = (1ull << lane) - 1;
  uint32_t ngt = 0, neq = 0;
  for (int i = w0 + lane; i < w1 + 63; i += 64) {
    const uint32_t key = i < w1 ? kl[i] : 0u;
    ngt += __popcll(__ballot(i < w1 && key > T));
    neq += __popcll(__ballot(i < w1 && key == T));
  }
  if (lane == 0) {
    wsum[0][wave] = ngt;
    wsum[1][wave] = neq;
  }
  __syncthreads();
  for (int v = 0; v < wave; ++v) {
    gt_run += wsum[0][v];
    eq_run += wsum[1][v];
  }
  for (int i = w0 + lane; i < w1 + 63; i += 64) {
    const bool in = i < w1;
    const uint32_t key = in ? kl[i] : 0u;
    const bool gt = in && key > T, eq = in && key == T;
    const uint64_t mg = __ballot(gt), me = __ballot(eq);
    const uint32_t gt_before = gt_run + __popcll(mg & below);
    const uint32_t eq_before = eq_run + __popcll(me & below);
    if (gt || (eq && eq_before < need)) {
      const uint32_t pos = gt_before + min(eq_before, need);
      if (pos < k) so[pos] = i;
    }
    gt_run += __popcll(mg);
    eq_run += __popcll(me);
  }
}

// every index when k >= n: sel[l][i] = i
__global__ __launch_bounds__(kSplitThreads) void split_all_kernel(int32_t* __restrict__ sel, int n, int sel_stride) {
  const int l = blockIdx.y;
  const int i = blockIdx.x * kSplitThreads + threadIdx.x;
  if (i < n) sel[(size_t)l * sel_stride + i] = i;
}

// The value of the k-th largest key of each list (the selection threshold).
__global__ void split_thresh_kernel(SplitWs w, float* __restrict__ thresh, int n_lists) {
  const int l = blockIdx.x * 256 + threadIdx.x;
  if (l < n_lists) thresh[l] = key_score(w.state[4 * l]);
}

__global__ void fill_f32_kernel(float* __restrict__ p, float v, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

size_t split_select_ws_bytes(int n_lists, int n) {
  const int n_slices = (n + kSplitSlice - 1) / kSplitSlice;
  return ((size_t)n_lists * kSelBins + (size_t)n_lists * 4 + (size_t)n_lists * n_slices * 2) * 4;
}

hipError_t launch_select_split(const uint32_t* keys, int32_t* sel, int n_lists, int n, int k, void* ws,
                               hipStream_t st, int sel_stride, float* thresh) {
  if (n_lists == 0) return hipSuccess;
  if (sel_stride < 0) sel_stride = k;
  if (k == 0 || n <= k) {
    // nothing selected (threshold +inf) or every index (threshold 0: errors are >= 0)
    if (thresh)
      hipLaunchKernelGGL(fill_f32_kernel, dim3((n_lists + 255) / 256), dim3(256), 0, st, thresh,
                         k == 0 ? __builtin_huge_valf() : 0.f, n_lists);
    if (k > 0 && n > 0)
      hipLaunchKernelGGL(split_all_kernel, dim3((n + kSplitThreads - 1) / kSplitThreads, n_lists),
                         dim3(kSplitThreads), 0, st, sel, n, sel_stride);
    return hipGetLastError();
  }
  const int n_slices = (n + kSplitSlice - 1) / kSplitSlice;
  SplitWs w;
  w.hist = static_cast<uint32_t*>(ws);
  w.state = w.hist + (size_t)n_lists * kSelBins;
  w.counts = w.state + (size_t)n_lists * 4;
  hipLaunchKernelGGL(split_init_kernel, dim3(n_lists), dim3(kSplitThreads), 0, st, w, k);
  constexpr int kShift[3] = {20, 8, 0};
  constexpr int kBits[3] = {12, 12, 8};
  for (int pass = 0; pass < 3; ++pass) {
    const uint32_t dmask = (1u << kBits[pass]) - 1u;
    hipLaunchKernelGGL(split_hist_kernel, dim3(n_slices, n_lists), dim3(kSplitThreads), 0, st, keys, w, n,
                       kShift[pass], dmask);
    hipLaunchKernelGGL(split_digit_kernel, dim3(n_lists), dim3(kSelThreads), 0, st, w, kShift[pass], dmask);
  }
  hipLaunchKernelGGL(split_count_kernel, dim3(n_slices, n_lists), dim3(kSplitThreads), 0, st, keys, w, n, n_slices);
  hipLaunchKernelGGL(split_compact_kernel, dim3(n_slices, n_lists), dim3(kSplitThreads), 0, st, keys, w, sel, n,
                     n_slices, sel_stride);
  if (thresh)
    hipLaunchKernelGGL(split_thresh_kernel, dim3((n_lists + 255) / 256), dim3(256), 0, st, w, thresh, n_lists);
  return hipGetLastError();
}

hipError_t launch_score(const uint16_t* q, const uint16_t* landmark, uint32_t* keys,
                        float* scores_out, int nb, int n_cand, int hq, int hkv, hipStream_t st,
                        int cache_bmul, int lm_rows, const ScoreWindow& win) {
  if (lm_rows < 0) lm_rows = n_cand;
  if (n_cand <= 0) return hipSuccess;
  // chunks per workgroup: the smallest power of two >= 256 that keeps the
  // grid within LOWRAM_SCORE_MAX_WG workgroups
  const int g = hq / hkv;
  const bool multi = cache_bmul == 0 && nb > 1 && (g == 1 || g == 2 || g == 4 || g == 8 || g == 16);
  const int qblocks = multi ? (nb + 16 / g - 1) / (16 / g) : nb;
  const long long heads = (long long)qblocks * hkv;
  int cpw = 256;
  while ((long long)((n_cand + cpw - 1) / cpw) * heads > LOWRAM_SCORE_MAX_WG && cpw < 4096) cpw *= 2;
  dim3 grid((n_cand + cpw - 1) / cpw, hkv, qblocks);
  // window tiles: only in the one-query-per-context grid
  if (win.n_tiles > 0 && (multi || cache_bmul != 1)) return hipErrorInvalidValue;
  if (!multi) {
    grid.x += win.n_tiles;
#define LOWRAM_SCORE(NBW)                                                                              \
  hipLaunchKernelGGL(score_kernel<NBW>, grid, dim3(256), 0, st, q, landmark, keys, scores_out, n_cand, hq, \
                     hkv, cache_bmul, lm_rows, win)
    switch (cpw / 256) {
      case 1: LOWRAM_SCORE(1); break;
      case 2: LOWRAM_SCORE(2); break;
      case 4: LOWRAM_SCORE(4); break;
      case 8: LOWRAM_SCORE(8); break;
      default: LOWRAM_SCORE(16); break;
    }
#undef LOWRAM_SCORE
  } else {
    switch (g) {
      case 1: hipLaunchKernelGGL(score_multi_kernel<1>, grid, dim3(256), 0, st, q, landmark, keys, scores_out, n_cand, hq, hkv, cpw, nb, lm_rows); break;
      case 2: hipLaunchKernelGGL(score_multi_kernel<2>, grid, dim3(256), 0, st, q, landmark, keys, scores_out, n_cand, hq, hkv, cpw, nb, lm_rows); break;
      case 4: hipLaunchKernelGGL(score_multi_kernel<4>, grid, dim3(256), 0, st, q, landmark, keys, scores_out, n_cand, hq, hkv, cpw, nb, lm_rows); break;
      case 8: hipLaunchKernelGGL(score_multi_kernel<8>, grid, dim3(256), 0, st, q, landmark, keys, scores_out, n_cand, hq, hkv, cpw, nb, lm_rows); break;
      default: hipLaunchKernelGGL(score_multi_kernel<16>, grid, dim3(256), 0, st, q, landmark, keys, scores_out, n_cand, hq, hkv, cpw, nb, lm_rows); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_select(const uint32_t* keys, const int32_t* cand_ids, int32_t* sel,
                         int32_t* sel_out, int nb, int n_cand, int k, int hkv, hipStream_t st,
                         int cache_bmul) {
  if (n_cand <= 0 && !sel_out) return hipSuccess;
  const dim3 grid(hkv, nb), block(kSelThreads);
  if (n_cand > kSelRegKeys) {
    hipLaunchKernelGGL(select_l2_kernel, grid, block, 0, st, keys, cand_ids, sel, sel_out, n_cand, k, hkv, cache_bmul);
    return hipGetLastError();
  }
  int lp = 0;  // 2^lp candidates per thread
  while ((kSelThreads << lp) < n_cand) ++lp;
#define LOWRAM_SEL(LP)                                                                                  \
  hipLaunchKernelGGL(select_reg_kernel<LP>, grid, block, 0, st, keys, cand_ids, sel, sel_out, n_cand, k, \
                     hkv, cache_bmul)
  switch (lp) {
    case 0: LOWRAM_SEL(0); break;
    case 1: LOWRAM_SEL(1); break;
    case 2: LOWRAM_SEL(2); break;
    case 3: LOWRAM_SEL(3); break;
    case 4: LOWRAM_SEL(4); break;
    default: LOWRAM_SEL(5); break;
  }
#undef LOWRAM_SEL
  return hipGetLastError();
}

}  // namespace lowram
