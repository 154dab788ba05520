// Landmark scoring (GEMV on MFMA) and exact top-k chunk selection, gfx950.
//
// LowRAM review (agihunt.info), key paragraph: the prefix is cut into chunks
// whose mean key is a landmark; each step ranks the chunks against the
// current query and rebuilds only the top-k.  The score of chunk c for KV
// head h is the maximum over h's query heads j of q_j . L[c]; the k largest
// are kept, exact ties to the lower chunk id, output in ascending chunk id.
#include <atomic>

#include "common.h"
#include "internal.h"

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
// 32 dims straight from the load registers.  A = the KV head's queries (rows
// j < g, zero rows above), B = 16 landmarks (columns), so lane l (< 16 per
// 16-lane group) ends up owning chunk c0 + l%16 with rows j = 4*(l/16) + e.
// Each wave keeps 4 groups of 16 landmarks (16 KiB) in flight per iteration.
// ---------------------------------------------------------------------------
#ifndef LOWRAM_SCORE_WG_PER_CU
#define LOWRAM_SCORE_WG_PER_CU 1
#endif
__global__ __launch_bounds__(256, LOWRAM_SCORE_WG_PER_CU) void score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ landmark,
    uint32_t* __restrict__ keys, float* __restrict__ scores_out, int n_cand, int n_heads_q,
    int n_heads_kv, int chunks_per_wg, int cache_bmul, int lm_rows) {
  const int b = blockIdx.z, h = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 4, col = lane & 15;
  const int g = n_heads_q / n_heads_kv;

  bf16x8 qa[4];
  const uint16_t* qb = q + ((size_t)b * n_heads_q + (size_t)h * g) * kHeadDim;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qa[ks] = col < g ? load_bf16x8(qb + col * kHeadDim + 32 * ks + 8 * grp) : zero_bf16x8();

  const size_t head = (size_t)b * n_heads_kv + h;
  const uint16_t* lm = landmark + ((size_t)b * cache_bmul * n_heads_kv + h) * (size_t)lm_rows * kHeadDim;
  uint32_t* kout = keys + head * (size_t)n_cand;
  float* sout = scores_out ? scores_out + head * (size_t)n_cand : nullptr;
  const int c_begin = blockIdx.x * chunks_per_wg;
  const int c_end = min(n_cand, c_begin + chunks_per_wg);

  // software pipeline: the next 64 landmarks of this wave are in flight
  // while the current 64 are multiplied
  auto load_group = [&](int c0, bf16x8 (&lv)[4][4]) {
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int cc = min(c0 + 16 * gi + col, n_cand - 1);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        lv[gi][ks] = load_bf16x8(lm + (size_t)cc * kHeadDim + 32 * ks + 8 * grp);
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
      float s = -__builtin_huge_valf();
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * grp + e < g) s = fmaxf(s, acc[e]);
      s = fmaxf(s, __shfl_xor(s, 16));
      s = fmaxf(s, __shfl_xor(s, 32));
      const int c = c0 + 16 * gi + col;
      if (grp == 0 && c < c_end) {
        kout[c] = score_key(s);
        if (sout) sout[c] = s;
      }
    }
#pragma unroll
    for (int gi = 0; gi < 4; ++gi)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) cur[gi][ks] = nxt[gi][ks];
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
// 1024 threads per (sequence, KV head).  The keys of the head are staged in
// LDS once (up to kSelLdsKeys of them; longer lists are re-read from L2 in
// every pass).  12-bit first digits spread the fp32 exponent over 4096 bins
// so few lanes of an LDS atomic hit the same bin; the digit search and the
// compaction offsets use wave-shuffle scans with one LDS exchange.
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelBins = 4096;
constexpr int kSelLdsKeys = 32768;

struct SelLds {  // the key array comes last: the L2-reading variant omits it
  uint32_t hist[kSelBins];
  uint32_t wsum[2][kSelWaves];
  uint32_t found[2];
  alignas(16) uint32_t keys[kSelLdsKeys];
};
constexpr int kSelBatch = 8;  // loads a thread has in flight at once

// inclusive scan of x over the 64 lanes of a wave, from the highest lane down
__device__ __forceinline__ uint32_t wave_scan_down(uint32_t x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_down(x, o);
    if (lane + o < 64) x += y;
  }
  return x;
}

template <bool kLds>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const uint32_t* __restrict__ keys, const int32_t* __restrict__ cand_ids,
    int32_t* __restrict__ sel, int32_t* __restrict__ sel_out, int n_cand, int k, int n_heads_kv,
    int cache_bmul) {
  extern __shared__ unsigned char sel_smem[];
  SelLds& S = *reinterpret_cast<SelLds*>(sel_smem);
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t head = (size_t)b * n_heads_kv + h;
  const uint32_t* kg = keys + head * (size_t)n_cand;
  const int32_t* ids = cand_ids ? cand_ids + ((size_t)b * cache_bmul * n_heads_kv + h) * (size_t)n_cand : nullptr;
  const int k_eff = min(k, n_cand);
  int32_t* so = sel + head * (size_t)k_eff;
  int32_t* so2 = sel_out ? sel_out + head * (size_t)k : nullptr;

  if (so2)
    for (int i = k_eff + tid; i < k; i += kSelThreads) so2[i] = -1;
  if (n_cand <= k) {  // every candidate is selected
    for (int i = tid; i < n_cand; i += kSelThreads) {
      const int32_t c = ids ? ids[i] : i;
      so[i] = c;
      if (so2) so2[i] = c;
    }
    return;
  }
  if constexpr (kLds) {
    // Every load of a batch goes out before the first store waits on one
    // (a plain copy loop kept one load per thread in flight): 16-byte pieces
    // when the list is 16-byte aligned, single keys otherwise.  Indices past
    // the end are clamped to the last element, which is then stored again
    // with its own value: no branch for the compiler to sink a load into.
    if ((reinterpret_cast<uintptr_t>(kg) & 15) == 0 && n_cand >= 4) {
      const int n4 = n_cand >> 2;
      const uint4* kg4 = reinterpret_cast<const uint4*>(kg);
      uint4* ks4 = reinterpret_cast<uint4*>(S.keys);
      for (int i0 = tid; i0 < n4; i0 += kSelThreads * kSelBatch) {
        uint4 v[kSelBatch];
#pragma unroll
        for (int u = 0; u < kSelBatch; ++u) v[u] = kg4[min(i0 + u * kSelThreads, n4 - 1)];
#pragma unroll
        for (int u = 0; u < kSelBatch; ++u) ks4[min(i0 + u * kSelThreads, n4 - 1)] = v[u];
      }
      for (int i = 4 * n4 + tid; i < n_cand; i += kSelThreads) S.keys[i] = kg[i];
    } else {
      for (int i0 = tid; i0 < n_cand; i0 += kSelThreads * kSelBatch) {
        uint32_t v[kSelBatch];
#pragma unroll
        for (int u = 0; u < kSelBatch; ++u) v[u] = kg[min(i0 + u * kSelThreads, n_cand - 1)];
#pragma unroll
        for (int u = 0; u < kSelBatch; ++u) S.keys[min(i0 + u * kSelThreads, n_cand - 1)] = v[u];
      }
    }
  }
  const uint32_t* kv = kLds ? S.keys : kg;

  uint32_t prefix = 0, pmask = 0, kk = (uint32_t)k;
  constexpr int kShift[3] = {20, 8, 0};
  constexpr int kBits[3] = {12, 12, 8};
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = kShift[pass], nbins = 1 << kBits[pass];
    const uint32_t dmask = (uint32_t)nbins - 1;
    for (int i = tid; i < nbins; i += kSelThreads) S.hist[i] = 0;
    __syncthreads();
    for (int i0 = tid; i0 < n_cand; i0 += kSelThreads * kSelBatch) {
      uint32_t kx[kSelBatch];  // a batch of reads before its atomics
#pragma unroll
      for (int u = 0; u < kSelBatch; ++u) kx[u] = kv[min(i0 + u * kSelThreads, n_cand - 1)];
#pragma unroll
      for (int u = 0; u < kSelBatch; ++u)
        if (i0 + u * kSelThreads < n_cand && (kx[u] & pmask) == prefix)
          atomicAdd(&S.hist[(kx[u] >> shift) & dmask], 1u);
    }
    __syncthreads();
    // thread t owns bins [bpt*t, bpt*t + bpt); the digit D is the bin where
    // the count of keys in higher bins first reaches kk
    const int bpt = nbins >= kSelThreads ? nbins / kSelThreads : 1;
    const bool owner = tid * bpt < nbins;
    uint32_t mine = 0;
    if (owner)
      for (int j = 0; j < bpt; ++j) mine += S.hist[tid * bpt + j];
    const uint32_t incl = wave_scan_down(mine, lane);  // this lane and above, in the wave
    if (lane == 0) S.wsum[0][wave] = incl;
    __syncthreads();
    uint32_t above = incl - mine;
    for (int w = wave + 1; w < kSelWaves; ++w) above += S.wsum[0][w];
    if (owner) {
      for (int j = bpt - 1; j >= 0; --j) {
        const uint32_t c = S.hist[tid * bpt + j];
        if (above < kk && kk <= above + c) {
          S.found[0] = tid * bpt + j;
          S.found[1] = above;
        }
        above += c;
      }
    }
    __syncthreads();
    const uint32_t digit = S.found[0];
    kk -= S.found[1];
    prefix |= digit << shift;
    pmask |= dmask << shift;
    __syncthreads();  // hist is cleared by the next pass
  }
  const uint32_t T = prefix, need = kk;

  // ordered compaction: wave w owns candidates [w*per, w*per + per) and walks
  // them 64 at a time (lane-strided, conflict-free LDS reads); ballots give
  // each key its rank among the wave's earlier > T / == T keys.
  const int per = (n_cand + kSelWaves - 1) / kSelWaves;
  const int w0 = min(n_cand, wave * per), w1 = min(n_cand, w0 + per);
  const uint64_t below = (1ull << lane) - 1;  // lanes under this one
  uint32_t ngt = 0, neq = 0;
  // batches of kSelBatch x 64 keys, read before they are counted (the batch
  // loop is uniform over the wave, so every ballot sees all 64 lanes)
  for (int b0 = w0; b0 < w1; b0 += 64 * kSelBatch) {
    uint32_t kx[kSelBatch];
#pragma unroll
    for (int u = 0; u < kSelBatch; ++u) kx[u] = kv[min(b0 + 64 * u + lane, n_cand - 1)];
#pragma unroll
    for (int u = 0; u < kSelBatch; ++u) {
      const bool in = b0 + 64 * u + lane < w1;
      ngt += __popcll(__ballot(in && kx[u] > T));
      neq += __popcll(__ballot(in && kx[u] == T));
    }
  }
  if (lane == 0) {
    S.wsum[0][wave] = ngt;
    S.wsum[1][wave] = neq;
  }
  __syncthreads();
  uint32_t gt_run = 0, eq_run = 0;
  for (int w = 0; w < wave; ++w) {
    gt_run += S.wsum[0][w];
    eq_run += S.wsum[1][w];
  }
  for (int b0 = w0; b0 < w1; b0 += 64 * kSelBatch) {
    uint32_t kx[kSelBatch];
#pragma unroll
    for (int u = 0; u < kSelBatch; ++u) kx[u] = kv[min(b0 + 64 * u + lane, n_cand - 1)];
#pragma unroll
    for (int u = 0; u < kSelBatch; ++u) {
      const int i = b0 + 64 * u + lane;
      const bool in = i < w1;
      const bool gt = in && kx[u] > T, eq = in && kx[u] == T;
      const uint64_t mg = __ballot(gt), me = __ballot(eq);
      const uint32_t gt_before = gt_run + __popcll(mg & below);
      const uint32_t eq_before = eq_run + __popcll(me & below);
      if (gt || (eq && eq_before < need)) {
        const uint32_t pos = gt_before + min(eq_before, need);
        if (pos < (uint32_t)k_eff) {
          const int32_t c = ids ? ids[i] : i;
          so[pos] = c;
          if (so2) so2[pos] = c;
        }
      }
      gt_run += __popcll(mg);
      eq_run += __popcll(me);
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
  const int l = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t* gh = w.hist + (size_t)l * kSelBins;
  const int nbins = (int)dmask + 1;
  const uint32_t kk = w.state[4 * l + 2];
  const int bpt = nbins >= kSelThreads ? nbins / kSelThreads : 1;
  const bool owner = tid * bpt < nbins;
  uint32_t mine = 0;
  if (owner)
    for (int j = 0; j < bpt; ++j) mine += gh[tid * bpt + j];
  const uint32_t incl = wave_scan_down(mine, lane);
  if (lane == 0) wsum[wave] = incl;
  __syncthreads();
  uint32_t above = incl - mine;
  for (int v = wave + 1; v < kSelWaves; ++v) above += wsum[v];
  if (owner) {
    for (int j = bpt - 1; j >= 0; --j) {
      const uint32_t c = gh[tid * bpt + j];
      if (above < kk && kk <= above + c) {
        found[0] = tid * bpt + j;
        found[1] = above;
      }
      above += c;
    }
  }
  __syncthreads();
  if (owner)
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
                        int cache_bmul, int lm_rows) {
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
  if (!multi) {
    hipLaunchKernelGGL(score_kernel, grid, dim3(256), 0, st, q, landmark, keys, scores_out,
                       n_cand, hq, hkv, cpw, cache_bmul, lm_rows);
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
  // dynamic LDS above 64 KiB must be allowed once per device (the attribute
  // belongs to the function on the current device); bit d: done on device d
  static std::atomic<uint64_t> attr_set{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  const uint64_t bit = dev >= 0 && dev < 64 ? 1ull << dev : 0;  // devices past 63: set on every call
  if (!bit || !(attr_set.load(std::memory_order_acquire) & bit)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(select_kernel<true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(SelLds)) != hipSuccess)
      return hipErrorInvalidValue;
    attr_set.fetch_or(bit, std::memory_order_release);
  }
  if (n_cand <= kSelLdsKeys) {
    hipLaunchKernelGGL(select_kernel<true>, grid, block, sizeof(SelLds), st, keys, cand_ids, sel, sel_out,
                       n_cand, k, hkv, cache_bmul);
  } else {
    hipLaunchKernelGGL(select_kernel<false>, grid, block, sizeof(SelLds) - kSelLdsKeys * 4, st, keys,
                       cand_ids, sel, sel_out, n_cand, k, hkv, cache_bmul);
  }
  return hipGetLastError();
}

}  // namespace lowram
