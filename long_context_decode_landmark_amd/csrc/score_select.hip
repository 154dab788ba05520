// Landmark scoring (GEMV on MFMA) and exact top-k chunk selection, gfx950.
//
// LowRAM review (agihunt.info), key paragraph: the prefix is cut into chunks
// whose mean key is a landmark; each step ranks the chunks against the
// current query and rebuilds only the top-k.  The score of chunk c for KV
// head h is the maximum over h's query heads j of q_j . L[c]; the k largest
// are kept, exact ties to the lower chunk id, output in ascending chunk id.
#include "common.h"
#include "internal.h"

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
__global__ __launch_bounds__(256) void score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ landmark,
    uint32_t* __restrict__ keys, float* __restrict__ scores_out, int n_cand, int n_heads_q,
    int n_heads_kv, int chunks_per_wg) {
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
  const uint16_t* lm = landmark + head * (size_t)n_cand * kHeadDim;
  uint32_t* kout = keys + head * (size_t)n_cand;
  float* sout = scores_out ? scores_out + head * (size_t)n_cand : nullptr;
  const int c_begin = blockIdx.x * chunks_per_wg;
  const int c_end = min(n_cand, c_begin + chunks_per_wg);

  for (int c0 = c_begin + wave * 64; c0 < c_end; c0 += 256) {
    bf16x8 lv[4][4];
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      const int cc = min(c0 + 16 * gi + col, n_cand - 1);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        lv[gi][ks] = load_bf16x8(lm + (size_t)cc * kHeadDim + 32 * ks + 8 * grp);
    }
#pragma unroll
    for (int gi = 0; gi < 4; ++gi) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mfma16(qa[ks], lv[gi][ks], acc);
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
  }
}

// ---------------------------------------------------------------------------
// Exact top-k by radix select on the order-preserving keys: four 8-bit
// passes find the k-th largest key T and how many keys equal to T are still
// needed; a final ordered compaction keeps every key > T and the first
// `need` keys == T in candidate order.  Candidates are in ascending chunk
// order, so the output is ascending.  One workgroup per (sequence, KV head);
// keys are read from L2 (the whole score vector of a head is <= 128 KiB).
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;

__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const uint32_t* __restrict__ keys, const int32_t* __restrict__ cand_ids,
    int32_t* __restrict__ sel, int32_t* __restrict__ sel_out, int n_cand, int k, int n_heads_kv) {
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t head = (size_t)b * n_heads_kv + h;
  const uint32_t* kv = keys + head * (size_t)n_cand;
  const int32_t* ids = cand_ids ? cand_ids + head * (size_t)n_cand : nullptr;
  const int k_eff = min(k, n_cand);
  int32_t* so = sel + head * (size_t)k_eff;
  int32_t* so2 = sel_out ? sel_out + head * (size_t)k : nullptr;

  __shared__ uint32_t hist[kSelWaves][256];
  __shared__ uint32_t suffix[257];
  __shared__ uint32_t found[2];
  __shared__ uint32_t scan_gt[kSelThreads], scan_eq[kSelThreads];

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

  uint32_t prefix = 0, pmask = 0, kk = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < kSelWaves * 256; i += kSelThreads) (&hist[0][0])[i] = 0;
    __syncthreads();
    for (int i = tid; i < n_cand; i += kSelThreads) {
      const uint32_t key = kv[i];
      if ((key & pmask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t s = 0;
#pragma unroll
      for (int w = 0; w < kSelWaves; ++w) s += hist[w][tid];
      suffix[tid] = s;
    }
    if (tid == 256) suffix[256] = 0;
    __syncthreads();
    // inclusive suffix sums over the 256 digit counts (Hillis-Steele)
    for (int off = 1; off < 256; off <<= 1) {
      uint32_t v = 0;
      if (tid < 256 && tid + off < 256) v = suffix[tid + off];
      __syncthreads();
      if (tid < 256) suffix[tid] += v;
      __syncthreads();
    }
    if (tid < 256) {
      const uint32_t above = suffix[tid + 1], incl = suffix[tid];
      if (above < kk && kk <= incl) { found[0] = tid; found[1] = above; }
    }
    __syncthreads();
    const uint32_t digit = found[0], above = found[1];
    kk -= above;
    prefix |= digit << shift;
    pmask |= 0xFFu << shift;
    __syncthreads();
  }
  const uint32_t T = prefix, need = kk;

  // ordered compaction: thread tid owns candidates [tid*per, tid*per + per)
  const int per = (n_cand + kSelThreads - 1) / kSelThreads;
  const int i0 = min(n_cand, tid * per), i1 = min(n_cand, i0 + per);
  uint32_t ngt = 0, neq = 0;
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = kv[i];
    ngt += key > T;
    neq += key == T;
  }
  scan_gt[tid] = ngt;
  scan_eq[tid] = neq;
  __syncthreads();
  for (int off = 1; off < kSelThreads; off <<= 1) {
    uint32_t a = 0, c = 0;
    if (tid >= off) { a = scan_gt[tid - off]; c = scan_eq[tid - off]; }
    __syncthreads();
    scan_gt[tid] += a;
    scan_eq[tid] += c;
    __syncthreads();
  }
  uint32_t eq_before = scan_eq[tid] - neq;
  uint32_t pos = (scan_gt[tid] - ngt) + min(eq_before, need);
  for (int i = i0; i < i1; ++i) {
    const uint32_t key = kv[i];
    bool take = key > T;
    if (key == T) { take = eq_before < need; ++eq_before; }
    if (take && pos < (uint32_t)k_eff) {
      const int32_t c = ids ? ids[i] : i;
      so[pos] = c;
      if (so2) so2[pos] = c;
      ++pos;
    }
  }
  (void)lane;
}

hipError_t launch_score(const uint16_t* q, const uint16_t* landmark, uint32_t* keys,
                        float* scores_out, int nb, int n_cand, int hq, int hkv, hipStream_t st) {
  if (n_cand <= 0) return hipSuccess;
  // enough workgroups to cover the chip even at batch 1
  const long long heads = (long long)nb * hkv;
  int cpw = 256;
  while ((long long)((n_cand + cpw - 1) / cpw) * heads > 4096 && cpw < 4096) cpw *= 2;
  dim3 grid((n_cand + cpw - 1) / cpw, hkv, nb);
  hipLaunchKernelGGL(score_kernel, grid, dim3(256), 0, st, q, landmark, keys, scores_out,
                     n_cand, hq, hkv, cpw);
  return hipGetLastError();
}

hipError_t launch_select(const uint32_t* keys, const int32_t* cand_ids, int32_t* sel,
                         int32_t* sel_out, int nb, int n_cand, int k, int hkv, hipStream_t st) {
  if (n_cand <= 0 && !sel_out) return hipSuccess;
  hipLaunchKernelGGL(select_kernel, dim3(hkv, nb), dim3(kSelThreads), 0, st, keys, cand_ids, sel,
                     sel_out, n_cand, k, hkv);
  return hipGetLastError();
}

}  // namespace lowram
