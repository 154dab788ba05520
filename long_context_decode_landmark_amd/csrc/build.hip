// Cache builder (prefill side) of the LowRAM compressed cache, gfx950.
//
// From a layer group's exact pre-RoPE keys, its shared basis, each layer's
// values and value MLP, it writes every array the decode step reads:
//   coefficients  C = X B^T of the prefix tokens (LowRAM review, key
//                 paragraph: cross-layer low-rank keys; LowRAM explainer,
//                 "How the method works": low-rank keys), bf16 or int4 g32
//   basis blocks  this layer's columns of B, transposed per KV head
//   landmarks     the mean post-RoPE key of each chunk (review, key paragraph)
//   residuals     R = V - MLP(K_pre) against the keys decode rebuilds from the
//                 STORED coefficients; per KV head the n_resid prefix tokens
//                 with the largest ||R||, ascending (review, value paragraph;
//                 explainer, "Residuals for difficult tokens")
//   window        the last W tokens exact: post-RoPE keys and values
// The per-token predictions MLP(K_pre) are computed to fp32 accuracy (exact
// three-piece bf16 operands on MFMA, erf GELU), so the residual ranking is the
// exact one up to fp32 rounding; decode's own bf16 prediction differs from it
// only by decode's rounding, which its output tolerance covers.
#include <cmath>

#include "common.h"
#include "internal.h"

namespace lowram {

// ---------------------------------------------------------------------------
// Projection C[t][m] = sum_j X[t][j] B[m][j] over the P prefix tokens, with
// the storage encoding fused into the epilogue.
//   workgroup tile  128 tokens x TN basis rows (TN = 128, or 64 at rank 64)
//   waves           2 x 2; wave (wm, wn) owns 64 tokens x TN/2 rows
//   k loop          64 columns per stage; X and B tiles go global -> VGPR ->
//                   LDS (double buffered, rows of 128 B with the 16-byte
//                   pieces XOR-swizzled by row & 7), one barrier per stage
//   epilogue        fp32 tile to LDS, then one thread per group of 32 rows
//                   writes bf16 or int4 codes + fp16 scale
// ---------------------------------------------------------------------------
constexpr int kProjTM = 128;
constexpr int kProjBK = 64;

template <int TN>
struct ProjLds {
  static constexpr int kStage = (kProjTM + TN) * kProjBK * 2;
  static constexpr int kTileStride = TN + 4;  // padded fp32 row of the epilogue tile
  static constexpr int kTile = kProjTM * kTileStride * 4;
  static constexpr int kBytes = 2 * kStage > kTile ? 2 * kStage : kTile;
};

__device__ __forceinline__ int swz(int row, int piece) { return row * 128 + ((piece ^ (row & 7)) << 4); }

// fp32 group of 32 -> bf16 (RNE) or int4 codes (symmetric, scale =
// fp16(absmax / 7), code = clamp(rint(x / scale), -7, 7), even element in the
// low nibble; an all-zero group stores scale 0 and zero codes).
__device__ __forceinline__ void encode_group32(const float* __restrict__ x, bool int4,
                                               uint16_t* __restrict__ bf, uint8_t* __restrict__ codes,
                                               uint16_t* __restrict__ scale) {
  if (!int4) {
#pragma unroll
    for (int i = 0; i < 32; i += 8) {
      f32x4 lo, hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo[e] = x[i + e];
        hi[e] = x[i + 4 + e];
      }
      *reinterpret_cast<bf16x8*>(bf + i) = pack8(lo, hi);
    }
    return;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const _Float16 sh = static_cast<_Float16>(amax / 7.0f);
  const float s = static_cast<float>(sh);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  if (s > 0.f) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float q = fminf(fmaxf(rintf(x[i] / s), -7.f), 7.f);
      w[i >> 3] |= (static_cast<uint32_t>(static_cast<int>(q)) & 0xFu) << (4 * (i & 7));
    }
  }
  *reinterpret_cast<u32x4*>(codes) = u32x4{w[0], w[1], w[2], w[3]};
  *scale = __builtin_bit_cast(uint16_t, sh);
}

struct ProjArgs {
  const uint16_t* keys;   // [NB][T][D]
  const uint16_t* basis;  // [NB][r][D]
  void* coeff;            // bf16 [NB][P][r] or int4 [NB][P][r/2]
  uint16_t* scale;        // int4: [NB][P][r/32]
  int T, P, D, r, n_tb, n_rb, total, padded_total;
  int out_rows, row0;  // output row of (b, t): b * out_rows + row0 + t
  bool int4;
  int mode;            // 0: cache encoding (bf16 / int4); 1: fp32 rows [row][r] into out_f32;
                       // 2: bf16 transposed into out_t[(b * r + m) * ld_t + t]
  float* out_f32;
  uint16_t* out_t;
  int ld_t;
  int splits;          // K split into `splits` ranges of k_split columns (mode 1: partial sums
  int k_split;         // go to out_f32 + split * rows * r)
};

template <int TN>
__global__ __launch_bounds__(256, 2) void proj_kernel(const ProjArgs a) {
  using L = ProjLds<TN>;
  __shared__ __attribute__((aligned(16))) unsigned char lds[L::kBytes];
  constexpr int NTW = TN / 32;       // n-tiles per wave
  constexpr int BPC = TN * 8 / 256;  // B pieces per thread per stage
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, col = lane & 15;
  const int wm = wave >> 1, wn = wave & 1;

  const int logical = xcd_logical_block(blockIdx.x, a.padded_total);
  if (logical >= a.total) return;
  const int rb = logical % a.n_rb;
  const int tb = (logical / a.n_rb) % a.n_tb;
  const int bs_ = logical / (a.n_rb * a.n_tb);  // (split, sequence)
  const int b = bs_ % (a.total / (a.n_rb * a.n_tb * a.splits));
  const int split = bs_ / (a.total / (a.n_rb * a.n_tb * a.splits));
  const int t0 = tb * kProjTM, m0 = rb * TN;
  const int kbeg = split * a.k_split;
  const uint16_t* xs = a.keys + (size_t)b * a.T * a.D + kbeg;
  const uint16_t* bs = a.basis + ((size_t)b * a.r + m0) * a.D + kbeg;

  // staging assignment: piece tid % 8 of rows tid / 8 + 32 u
  const int srow = tid >> 3, spc = tid & 7;
  u32x4 xa[4], xb[BPC];
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = min(t0 + srow + 32 * u, a.P - 1);
      xa[u] = *reinterpret_cast<const u32x4*>(xs + (size_t)t * a.D + k0 + 8 * spc);
    }
#pragma unroll
    for (int u = 0; u < BPC; ++u)
      xb[u] = *reinterpret_cast<const u32x4*>(bs + (size_t)(srow + 32 * u) * a.D + k0 + 8 * spc);
  };
  auto store_stage = [&](int buf) {
    unsigned char* sa = lds + buf * L::kStage;
    unsigned char* sb = sa + kProjTM * 128;
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<u32x4*>(sa + swz(srow + 32 * u, spc)) = xa[u];
#pragma unroll
    for (int u = 0; u < BPC; ++u) *reinterpret_cast<u32x4*>(sb + swz(srow + 32 * u, spc)) = xb[u];
  };

  f32x4 acc[4][NTW];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = min(a.k_split, a.D - kbeg) / kProjBK;
  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int kb = 0; kb < nk; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < nk) load_stage((kb + 1) * kProjBK);
    const unsigned char* sa = lds + cur * L::kStage;
    const unsigned char* sb = sa + kProjTM * 128;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 av[4], bv[NTW];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        av[mt] = __builtin_bit_cast(bf16x8,
                                    *reinterpret_cast<const u32x4*>(sa + swz(64 * wm + 16 * mt + col, 4 * ks + grp)));
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt)
        bv[nt] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(sb + swz((TN / 2) * wn + 16 * nt + col, 4 * ks + grp)));
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) acc[mt][nt] = mfma16(av[mt], bv[nt], acc[mt][nt]);
    }
    if (kb + 1 < nk) store_stage(cur ^ 1);
    __syncthreads();
  }

  // epilogue: D[token][row] -> LDS tile, then encode groups of 32 rows
  float* tile = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        tile[(64 * wm + 16 * mt + 4 * grp + e) * L::kTileStride + (TN / 2) * wn + 16 * nt + col] = acc[mt][nt][e];
  __syncthreads();
  if (a.mode == 1) {
    // fp32 rows: thread -> (row tl, 4 consecutive m); 128 x TN values
    for (int idx = tid; idx < kProjTM * (TN / 4); idx += 256) {
      const int tl = idx / (TN / 4), m4 = 4 * (idx % (TN / 4));
      const int t = t0 + tl;
      if (t >= a.P) continue;
      const float* src = tile + tl * L::kTileStride + m4;
      *reinterpret_cast<f32x4*>(a.out_f32 + (size_t)split * a.P * a.r +
                                ((size_t)b * a.out_rows + a.row0 + t) * a.r + m0 + m4) =
          f32x4{src[0], src[1], src[2], src[3]};
    }
    return;
  }
  if (a.mode == 2) {
    // bf16 transposed: thread -> (m, 8 consecutive rows t)
    for (int idx = tid; idx < TN * (kProjTM / 8); idx += 256) {
      const int ml = idx / (kProjTM / 8), t8 = 8 * (idx % (kProjTM / 8));
      if (t0 + t8 >= a.P) continue;
      f32x4 lo, hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo[e] = tile[(t8 + e) * L::kTileStride + ml];
        hi[e] = tile[(t8 + 4 + e) * L::kTileStride + ml];
      }
      uint16_t* dst = a.out_t + ((size_t)b * a.r + m0 + ml) * a.ld_t + t0 + t8;
      if (t0 + t8 + 8 <= a.P) {
        *reinterpret_cast<bf16x8*>(dst) = pack8(lo, hi);
      } else {
        const bf16x8 v = pack8(lo, hi);
        for (int e = 0; e < 8 && t0 + t8 + e < a.P; ++e) dst[e] = __builtin_bit_cast(uint16_t, v[e]);
      }
    }
    return;
  }
  constexpr int GPT = TN / 32;  // groups per token row of the tile
  for (int gi = tid; gi < kProjTM * GPT; gi += 256) {
    const int tl = gi / GPT, j = gi % GPT;
    const int t = t0 + tl;
    if (t >= a.P) continue;
    const size_t row = (size_t)b * a.out_rows + a.row0 + t;
    const int m = m0 + 32 * j;
    if (a.int4)
      encode_group32(tile + tl * L::kTileStride + 32 * j, true, nullptr,
                     static_cast<uint8_t*>(a.coeff) + row * (a.r / 2) + m / 2, a.scale + row * (a.r / 32) + m / 32);
    else
      encode_group32(tile + tl * L::kTileStride + 32 * j, false, static_cast<uint16_t*>(a.coeff) + row * a.r + m,
                     nullptr, nullptr);
  }
}

hipError_t launch_proj(const uint16_t* keys, const uint16_t* basis, void* coeff, uint16_t* scale, int nb, int T,
                       int P, int D, int r, bool int4, hipStream_t st, int out_rows, int row0) {
  if (P == 0) return hipSuccess;
  ProjArgs a{};
  a.keys = keys; a.basis = basis; a.coeff = coeff; a.scale = scale;
  a.T = T; a.P = P; a.D = D; a.r = r; a.int4 = int4;
  a.out_rows = out_rows < 0 ? P : out_rows;
  a.row0 = row0;
  a.mode = 0;
  a.splits = 1;
  a.k_split = D;
  const int tn = r >= 128 ? 128 : 64;
  a.n_tb = (P + kProjTM - 1) / kProjTM;
  a.n_rb = r / tn;
  a.total = nb * a.n_tb * a.n_rb;
  a.padded_total = (a.total + 7) & ~7;
  if (tn == 128) hipLaunchKernelGGL(proj_kernel<128>, dim3(a.padded_total), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(proj_kernel<64>, dim3(a.padded_total), dim3(256), 0, st, a);
  return hipGetLastError();
}

// C[t][m] = sum_j A[b][t][j] B[b][m][j] for t < rows, m < r (A: T rows per
// sequence, K columns; B: [NB][r][K]); K a multiple of 64.  mode 1: fp32
// [NB][rows][r]; mode 2: bf16 transposed [NB][r][ld_t].
__global__ __launch_bounds__(256) void split_sum_kernel(float* __restrict__ out, const float* __restrict__ part,
                                                        size_t n, int splits) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  f32x4 acc = *reinterpret_cast<const f32x4*>(part + i);
  for (int s = 1; s < splits; ++s) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(part + (size_t)s * n + i);
    acc[0] += v[0]; acc[1] += v[1]; acc[2] += v[2]; acc[3] += v[3];
  }
  *reinterpret_cast<f32x4*>(out + i) = acc;
}

hipError_t launch_gemm_nt(const uint16_t* A, const uint16_t* B, int nb, int T, int rows, int K, int r, int mode,
                          float* out_f32, uint16_t* out_t, int ld_t, hipStream_t st, int splits,
                          float* partials) {
  if (rows == 0) return hipSuccess;
  ProjArgs a{};
  a.keys = A; a.basis = B;
  a.T = T; a.P = rows; a.D = K; a.r = r;
  a.out_rows = rows; a.row0 = 0; a.mode = mode; a.out_f32 = out_f32; a.out_t = out_t; a.ld_t = ld_t;
  if (mode != 1 || nb != 1 || !partials) splits = 1;
  a.k_split = ((K / kProjBK + splits - 1) / splits) * kProjBK;
  splits = (K + a.k_split - 1) / a.k_split;  // no empty split
  a.splits = splits;
  if (splits > 1) a.out_f32 = partials;
  const int tn = r >= 128 ? 128 : 64;
  a.n_tb = (rows + kProjTM - 1) / kProjTM;
  a.n_rb = r / tn;
  a.total = nb * a.n_tb * a.n_rb * splits;
  a.padded_total = (a.total + 7) & ~7;
  if (tn == 128) hipLaunchKernelGGL(proj_kernel<128>, dim3(a.padded_total), dim3(256), 0, st, a);
  else hipLaunchKernelGGL(proj_kernel<64>, dim3(a.padded_total), dim3(256), 0, st, a);
  if (splits > 1) {
    const size_t n = (size_t)rows * r;
    hipLaunchKernelGGL(split_sum_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, st, out_f32, partials,
                       n, splits);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-layer arrays that need no MLP: basis blocks, landmarks, window.
// ---------------------------------------------------------------------------

// Basis blocks: blk[b][h][i][m] = B[b][m][col(layer, h, i)].
// Grid (r / 64, Hkv, NB); LDS transpose of a 64 x 128 block.
__global__ __launch_bounds__(256) void basis_block_kernel(const uint16_t* __restrict__ basis,
                                                          uint16_t* __restrict__ blk, const BuildGeo g) {
  __shared__ uint16_t tile[64][kHeadDim + 2];
  const int m0 = blockIdx.x * 64, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int col0 = (g.layer_in_group * g.hkv + h) * kHeadDim;
  const uint16_t* bs = basis + (size_t)b * g.r * g.D;
  for (int idx = tid; idx < 64 * kHeadDim; idx += 256) {
    const int m = idx / kHeadDim, i = idx % kHeadDim;
    tile[m][i] = bs[(size_t)(m0 + m) * g.D + col0 + i];
  }
  __syncthreads();
  uint16_t* o = blk + ((size_t)b * g.hkv + h) * kHeadDim * g.r;
  for (int idx = tid; idx < 64 * kHeadDim; idx += 256) {
    const int i = idx / 64, m = idx % 64;
    o[(size_t)i * g.r + m0 + m] = tile[m][i];
  }
}

// Landmarks: one wave per (chunk, head), lane p owns the rotate-half pair
// (p, p + 64); the chunk's S keys are rotated at their positions and averaged
// in fp32.  Grid (ceil(nC / 4), Hkv, NB).
__global__ __launch_bounds__(256) void landmark_kernel(const uint16_t* __restrict__ keys, uint16_t* __restrict__ lm,
                                                       const BuildGeo g) {
  const int c = blockIdx.x * 4 + (threadIdx.x >> 6), p = threadIdx.x & 63, h = blockIdx.y, b = blockIdx.z;
  if (c >= g.n_chunks) return;
  const uint16_t* xs = keys + (size_t)b * g.T * g.D + (g.layer_in_group * g.hkv + h) * kHeadDim;
  float y1 = 0.f, y2 = 0.f;
#pragma unroll
  for (int i = 0; i < kChunk; ++i) {
    const int t = c * kChunk + i;
    const float x1 = bf16_to_f32(xs[(size_t)t * g.D + p]);
    const float x2 = bf16_to_f32(xs[(size_t)t * g.D + p + 64]);
    const float2 cs = rot_of((double)t * g.inv_freq[p]);
    y1 += x1 * cs.x - x2 * cs.y;
    y2 += x2 * cs.x + x1 * cs.y;
  }
  uint16_t* o = lm + (((size_t)b * g.hkv + h) * (g.prefix_cap / kChunk) + c) * kHeadDim;
  o[p] = __builtin_bit_cast(uint16_t, (__bf16)(y1 * (1.0f / kChunk)));
  o[p + 64] = __builtin_bit_cast(uint16_t, (__bf16)(y2 * (1.0f / kChunk)));
}

// Window: rotated keys and the values of tokens P .. T-1.
// Grid (ceil(W / 4), Hkv, NB), one wave per token.
__global__ __launch_bounds__(256) void window_kernel(const uint16_t* __restrict__ keys,
                                                     const uint16_t* __restrict__ values, uint16_t* __restrict__ wk,
                                                     uint16_t* __restrict__ wv, const BuildGeo g) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6), p = threadIdx.x & 63, h = blockIdx.y, b = blockIdx.z;
  if (w >= g.W) return;
  const int t = g.P + w;
  const size_t head = (size_t)b * g.hkv + h;
  const uint16_t* xr = keys + ((size_t)b * g.T + t) * g.D + (g.layer_in_group * g.hkv + h) * kHeadDim;
  const float x1 = bf16_to_f32(xr[p]);
  const float x2 = bf16_to_f32(xr[p + 64]);
  const float2 cs = rot_of((double)t * g.inv_freq[p]);
  uint16_t* ko = wk + (head * g.window_cap + w) * kHeadDim;
  ko[p] = __builtin_bit_cast(uint16_t, (__bf16)(x1 * cs.x - x2 * cs.y));
  ko[p + 64] = __builtin_bit_cast(uint16_t, (__bf16)(x2 * cs.x + x1 * cs.y));
  const uint16_t* vi = values + (head * g.T + t) * kHeadDim;
  uint16_t* vo = wv + (head * g.window_cap + w) * kHeadDim;
  vo[p] = vi[p];
  vo[p + 64] = vi[p + 64];
}

// ---------------------------------------------------------------------------
// Residual side.
// ---------------------------------------------------------------------------

// Three bf16 pieces whose sum is the fp32 value, for 8 floats (lo4, hi4):
// each piece is the upper half of the remainder (truncation), so the
// remainders are exact and the third piece holds the last 8 significand bits.
// Products with a bf16 weight are then exact in the MFMA and only its fp32
// accumulation rounds.
__device__ __forceinline__ uint32_t hi_halves(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

__device__ __forceinline__ void split3(f32x4 lo4, f32x4 hi4, bf16x8 (&s)[3]) {
  float v[8] = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
#pragma unroll
  for (int piece = 0; piece < 3; ++piece) {
    u32x4 w;
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = hi_halves(v[2 * q], v[2 * q + 1]);
    s[piece] = __builtin_bit_cast(bf16x8, w);
    if (piece < 2) {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] -= __uint_as_float(__float_as_uint(v[e]) & 0xFFFF0000u);
    }
  }
}

// Exact-GELU x Phi(x) to fp32 accuracy without a branchy library erf:
// with z = |x| / sqrt(2) and t = 1 / (1 + z / 2), erfc(z) = t exp(P(t) - z^2).
// That form is the Chebyshev-fitted erfc of Press, Teukolsky, Vetterling and
// Flannery, Numerical Recipes (routine erfcc); here P is a degree-7 polynomial
// refitted for this use (weighted least squares on
// z in [0, 6], largest error of log erfc 4.3e-7); Phi(x) = 1 - erfc(z) / 2 for
// x >= 0 and erfc(z) / 2 below.  Largest deviation of the fp32 evaluation from
// x Phi(x) over the reals: 2.4e-7 absolute (the rounding of x - x erfc / 2).
constexpr float kErfcP[8] = {-1.266052961e+00f, 1.006492019e+00f, 3.495076001e-01f, 9.338895231e-02f,
                             1.200157702e-01f,  -7.711301446e-01f, 6.278482676e-01f, -1.600698978e-01f};

__device__ __forceinline__ float gelu_erf(float x) {
  const float z = fabsf(x) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.5f, z, 1.0f));
  float p = kErfcP[7];
#pragma unroll
  for (int k = 6; k >= 0; --k) p = fmaf(p, t, kErfcP[k]);
  const float ec = t * __builtin_amdgcn_exp2f(fmaf(-z, z, p) * kLog2e);  // erfc(z)
  const float half = 0.5f * x * ec;
  return x >= 0.f ? x - half : half;
}

struct PredictArgs {
  const void* coeff;            // bf16 [NB][P][r] or int4 [NB][P][r/2]
  const uint16_t* coeff_scale;  // int4: [NB][P][r/32]
  const uint16_t* blk;          // [NB][Hkv][d][r]
  const uint16_t *w1, *b1, *w2, *b2;
  const uint16_t* values;       // [NB][Hkv][T][d]
  float* r;                     // out [NB][Hkv][P][d]
  uint32_t* keys;               // out [NB][Hkv][P]
  int T, P, hkv, n_tb, total, padded_total;
  int coeff_rows;               // coefficient rows per sequence
};

constexpr int kPredTokWG = 128;   // 4 waves x 32 tokens
constexpr int kPredStage = 16384;  // bytes per LDS stage

// LDS swizzles of the prediction kernel's stages (16-byte pieces); each makes
// the 16 rows one MFMA operand read touches land on distinct banks.
// blk stage: 128 rows x 128 B (64 basis columns)
__device__ __forceinline__ int pred_blk_off(int row, int piece) {
  return row * 128 + ((piece ^ (((row >> 1) & 1) | ((row >> 2) & 6))) << 4);
}
// W1 block: 32 rows x 256 B (one hidden unit per row, 128 inputs)
__device__ __forceinline__ int pred_w1_off(int row, int piece) {
  return row * 256 + ((piece ^ ((row & 3) | ((row >> 1) & 12))) << 4);
}
// W2 block: 128 rows x 64 B (one output per row, 32 hidden units)
__device__ __forceinline__ int pred_w2_off(int row, int piece) {
  return 8192 + row * 64 + ((piece ^ ((row >> 2) & 3)) << 4);
}

// Residuals of every prefix token of one KV head against an fp32-accurate
// prediction: K^T = blk C^T (rebuilt pre-RoPE keys), Z^T = W1 K^T + b1,
// V~^T = W2 gelu(Z)^T + b2, R = V - V~ and the selection key of ||R||.
// Tokens are the MFMA column dimension (wave: 2 tiles of 16 tokens); the A
// rows of blk and W1 are taken in row_perm32 order so each product's
// accumulators are the next one's B operand.  The weights stream through LDS
// in 16 KiB stages shared by the 4 waves: RANK/64 stages of blk columns, then
// per block of 32 hidden units one stage of W1 rows + W2 columns.  A stage is
// loaded one step ahead into registers and stored after the step's MFMAs,
// with one barrier per step; the coefficient operands of the next blk stage
// are loaded one step ahead too.
#ifndef LOWRAM_PRED_WG_PER_CU
#define LOWRAM_PRED_WG_PER_CU 2
#endif

template <int RANK, bool CI4>
__global__ __launch_bounds__(256, LOWRAM_PRED_WG_PER_CU) void predict_resid_kernel(const PredictArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2 * kPredStage];
  constexpr int NS1 = RANK / 64;      // blk stages
  constexpr int NS = NS1 + kHidden / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, col = lane & 15;
  const int logical = xcd_logical_block(blockIdx.x, a.padded_total);
  if (logical >= a.total) return;  // whole workgroup: before any barrier
  const int h = logical % a.hkv;
  const int tb = (logical / a.hkv) % a.n_tb;
  const int b = logical / (a.hkv * a.n_tb);
  const size_t head = (size_t)b * a.hkv + h;
  const int t0 = tb * kPredTokWG + 32 * wave;
  int tok[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) tok[tt] = min(t0 + 16 * tt + col, a.P - 1);  // waves past P repeat token P-1

  const uint16_t* blk = a.blk + head * kHeadDim * RANK;
  const uint16_t* w1 = a.w1 + head * kHidden * kHeadDim;
  const uint16_t* b1 = a.b1 + head * kHidden;
  const uint16_t* w2 = a.w2 + head * kHeadDim * kHidden;

  // stage s -> 4 pieces of 16 B per thread
  u32x4 sreg[4];
  auto stage_load = [&](int s) {
    if (s < NS1) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        sreg[u] = *reinterpret_cast<const u32x4*>(blk + (tid / 8 + 32 * u) * RANK + 64 * s + 8 * (tid % 8));
    } else {
      const int jb = s - NS1;
#pragma unroll
      for (int u = 0; u < 2; ++u)
        sreg[u] = *reinterpret_cast<const u32x4*>(w1 + (32 * jb + tid / 16 + 16 * u) * kHeadDim + 8 * (tid % 16));
#pragma unroll
      for (int u = 0; u < 2; ++u)
        sreg[2 + u] = *reinterpret_cast<const u32x4*>(w2 + (tid / 4 + 64 * u) * kHidden + 32 * jb + 8 * (tid % 4));
    }
  };
  auto stage_store = [&](int s, unsigned char* buf) {
    if (s < NS1) {
#pragma unroll
      for (int u = 0; u < 4; ++u) *reinterpret_cast<u32x4*>(buf + pred_blk_off(tid / 8 + 32 * u, tid % 8)) = sreg[u];
    } else {
#pragma unroll
      for (int u = 0; u < 2; ++u) *reinterpret_cast<u32x4*>(buf + pred_w1_off(tid / 16 + 16 * u, tid % 16)) = sreg[u];
#pragma unroll
      for (int u = 0; u < 2; ++u) *reinterpret_cast<u32x4*>(buf + pred_w2_off(tid / 4 + 64 * u, tid % 4)) = sreg[2 + u];
    }
  };
  // coefficient operands of blk stage s: k-steps 2 s, 2 s + 1, both token tiles
  constexpr int CW = CI4 ? 1 : 4;  // 32-bit words per (k-step, token tile)
  uint32_t creg[2][2][CW];
  uint16_t csc[2][2];
  auto coeff_load = [&](int s) {
#pragma unroll
    for (int kl = 0; kl < 2; ++kl)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const size_t row = (size_t)b * a.coeff_rows + tok[tt];
        const int ks = 2 * s + kl;
        if constexpr (!CI4) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.coeff) + row * RANK +
                                                          32 * ks + 8 * grp);
#pragma unroll
          for (int q = 0; q < 4; ++q) creg[kl][tt][q] = v[q];
        } else {
          creg[kl][tt][0] = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(a.coeff) +
                                                               row * (RANK / 2) + 16 * ks + 4 * grp);
          csc[kl][tt] = a.coeff_scale[row * (RANK / 32) + ks];
        }
      }
  };

  stage_load(0);
  coeff_load(0);
  stage_store(0, lds);
  __syncthreads();

  // phase 1: K^T[i][t] = sum_m blk[i][m] C[t][m], 64 columns per stage
  bf16x8 kb[4][2][3];
  {
    f32x4 kacc[8][2];
#pragma unroll
    for (int it = 0; it < 8; ++it)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) kacc[it][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int s = 0; s < NS1; ++s) {
      const unsigned char* cur = lds + (s & 1) * kPredStage;
      uint32_t cnow[2][2][CW];
      uint16_t snow[2][2];
#pragma unroll
      for (int kl = 0; kl < 2; ++kl)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
          for (int q = 0; q < CW; ++q) cnow[kl][tt][q] = creg[kl][tt][q];
          snow[kl][tt] = CI4 ? csc[kl][tt] : 0;
        }
      stage_load(s + 1);  // NS > NS1: the next stage always exists
      if (s + 1 < NS1) coeff_load(s + 1);
#pragma unroll
      for (int kl = 0; kl < 2; ++kl) {
        bf16x8 cb[2][CI4 ? 2 : 1];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          if constexpr (!CI4) {
            cb[tt][0] = __builtin_bit_cast(bf16x8, u32x4{cnow[kl][tt][0], cnow[kl][tt][1], cnow[kl][tt][2],
                                                         cnow[kl][tt][3]});
          } else {
            // code * scale has at most 15 significant bits: two bf16 pieces hold it exactly
            const uint32_t w = cnow[kl][tt][0];
            const float sc = f16_to_f32(snow[kl][tt]);
            f32x4 lo, hi;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              lo[e] = (float)(((int)(w << (28 - 4 * e))) >> 28) * sc;
              hi[e] = (float)(((int)(w << (12 - 4 * e))) >> 28) * sc;
            }
            cb[tt][0] = pack8(lo, hi);
            cb[tt][1] = pack8_lo(lo, hi, cb[tt][0]);
          }
        }
#pragma unroll
        for (int it = 0; it < 8; ++it) {
          const int irow = 32 * (it >> 1) + row_perm32(16 * (it & 1) + col);
          const bf16x8 af = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                           cur + pred_blk_off(irow, 4 * kl + grp)));
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int sp = 0; sp < (CI4 ? 2 : 1); ++sp) kacc[it][tt] = mfma16(af, cb[tt][sp], kacc[it][tt]);
        }
      }
      stage_store(s + 1, lds + ((s + 1) & 1) * kPredStage);
      __syncthreads();
    }
    // B operands of the next product: k-step q (i = 32 q + 8 g + 0..7) from tiles 2 q, 2 q + 1
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) split3(kacc[2 * q][tt], kacc[2 * q + 1][tt], kb[q][tt]);
  }

  // phases 2 and 3, one block of 32 hidden units per stage:
  // Z^T = W1 K^T + b1, h = gelu(Z), V~^T += W2[:, block] h^T
  f32x4 vacc[8][2];
#pragma unroll
  for (int nd = 0; nd < 8; ++nd)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) vacc[nd][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int s = NS1; s < NS; ++s) {
    const unsigned char* cur = lds + (s & 1) * kPredStage;
    const int jb = s - NS1;
    if (s + 1 < NS) stage_load(s + 1);
    f32x4 z[2][2];
#pragma unroll
    for (int jt = 0; jt < 2; ++jt) {
      f32x4 bias;
#pragma unroll
      for (int e = 0; e < 4; ++e) bias[e] = bf16_to_f32(b1[32 * jb + 8 * grp + 4 * jt + e]);
      z[jt][0] = bias;
      z[jt][1] = bias;
      const int jl = row_perm32(16 * jt + col);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bf16x8 af = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                         cur + pred_w1_off(jl, 4 * q + grp)));
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int sp = 0; sp < 3; ++sp) z[jt][tt] = mfma16(af, kb[q][tt][sp], z[jt][tt]);
      }
    }
    bf16x8 hb[2][3];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
#pragma unroll
      for (int jt = 0; jt < 2; ++jt)
#pragma unroll
        for (int e = 0; e < 4; ++e) z[jt][tt][e] = gelu_erf(z[jt][tt][e]);
      split3(z[0][tt], z[1][tt], hb[tt]);
    }
#pragma unroll
    for (int nd = 0; nd < 8; ++nd) {
      const bf16x8 af = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
                                                       cur + pred_w2_off(16 * nd + col, grp)));
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int sp = 0; sp < 3; ++sp) vacc[nd][tt] = mfma16(af, hb[tt][sp], vacc[nd][tt]);
    }
    if (s + 1 < NS) stage_store(s + 1, lds + ((s + 1) & 1) * kPredStage);
    __syncthreads();
  }

  // R = V - (V~ + b2) for d = 16 nd + 4 g + e, token column col
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int t = t0 + 16 * tt + col;
    const bool valid = t < a.P;
    const uint16_t* vr = a.values + (head * a.T + tok[tt]) * kHeadDim;
    float* rr = a.r + (head * a.P + tok[tt]) * kHeadDim;
    float ss = 0.f;
#pragma unroll
    for (int nd = 0; nd < 8; ++nd) {
      const int d0 = 16 * nd + 4 * grp;
      const u32x2 vv = *reinterpret_cast<const u32x2*>(vr + d0);
      f32x4 res;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint16_t vb = (uint16_t)(vv[e >> 1] >> (16 * (e & 1)));
        res[e] = bf16_to_f32(vb) - (vacc[nd][tt][e] + bf16_to_f32(a.b2[head * kHeadDim + d0 + e]));
        ss = fmaf(res[e], res[e], ss);
      }
      if (valid) *reinterpret_cast<f32x4*>(rr + d0) = res;
    }
    ss += __shfl_xor(ss, 16);
    ss += __shfl_xor(ss, 32);
    if (valid && grp == 0) a.keys[head * a.P + t] = score_key(sqrtf(ss));
  }
}

// Selected residual rows -> storage format; one thread per (row, group of 32).
__global__ __launch_bounds__(256) void resid_store_kernel(const float* __restrict__ r, const int32_t* __restrict__ idx,
                                                          void* __restrict__ res_val, uint16_t* __restrict__ res_scale,
                                                          size_t n_rows, const BuildGeo g, bool int4) {
  const size_t gi = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (gi >= n_rows * 4) return;
  const size_t sel_row = gi >> 2;  // (b * Hkv + h) * nR + i
  const int j = (int)(gi & 3);
  const size_t head = sel_row / (size_t)g.n_resid;
  const size_t row = head * g.resid_cap + sel_row % (size_t)g.n_resid;  // stored row
  const int t = idx[row];
  const float* src = r + (head * g.P + t) * kHeadDim + 32 * j;
  if (int4)
    encode_group32(src, true, nullptr, static_cast<uint8_t*>(res_val) + row * (kHeadDim / 2) + 16 * j,
                   res_scale + row * (kHeadDim / 32) + j);
  else
    encode_group32(src, false, static_cast<uint16_t*>(res_val) + row * kHeadDim + 32 * j, nullptr, nullptr);
}

hipError_t launch_build_layer_arrays(const uint16_t* keys, const uint16_t* values, const uint16_t* basis,
                                     uint16_t* blk, uint16_t* lm, uint16_t* wk, uint16_t* wv, const BuildGeo& g,
                                     hipStream_t st) {
  hipLaunchKernelGGL(basis_block_kernel, dim3(g.r / 64, g.hkv, g.nb), dim3(256), 0, st, basis, blk, g);
  if (g.n_chunks > 0)
    hipLaunchKernelGGL(landmark_kernel, dim3((g.n_chunks + 3) / 4, g.hkv, g.nb), dim3(256), 0, st, keys, lm, g);
  if (g.W > 0)
    hipLaunchKernelGGL(window_kernel, dim3((g.W + 3) / 4, g.hkv, g.nb), dim3(256), 0, st, keys, values, wk, wv, g);
  return hipGetLastError();
}

template <int RANK>
static void launch_predict_rank(const PredictArgs& a, bool ci4, hipStream_t st) {
  if (ci4) hipLaunchKernelGGL((predict_resid_kernel<RANK, true>), dim3(a.padded_total), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((predict_resid_kernel<RANK, false>), dim3(a.padded_total), dim3(256), 0, st, a);
}

hipError_t launch_predict_resid(const void* coeff, const uint16_t* coeff_scale, const uint16_t* blk,
                                const uint16_t* w1, const uint16_t* b1, const uint16_t* w2, const uint16_t* b2,
                                const uint16_t* values, float* r, uint32_t* keys, bool ci4, const BuildGeo& g,
                                hipStream_t st) {
  if (g.P == 0) return hipSuccess;
  PredictArgs a{};
  a.coeff = coeff; a.coeff_scale = coeff_scale; a.blk = blk;
  a.w1 = w1; a.b1 = b1; a.w2 = w2; a.b2 = b2; a.values = values; a.r = r; a.keys = keys;
  a.T = g.T; a.P = g.P; a.hkv = g.hkv;
  a.coeff_rows = g.prefix_cap;
  a.n_tb = (g.P + kPredTokWG - 1) / kPredTokWG;
  a.total = g.nb * g.hkv * a.n_tb;
  a.padded_total = (a.total + 7) & ~7;
  switch (g.r) {
    case 64:
      if (ci4) return hipErrorInvalidValue;  // int4 coefficients need rank % 128 == 0
      launch_predict_rank<64>(a, false, st);
      break;
    case 128: launch_predict_rank<128>(a, ci4, st); break;
    case 256: launch_predict_rank<256>(a, ci4, st); break;
    case 512: launch_predict_rank<512>(a, ci4, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Window rollover: the oldest S window tokens (positions P .. P+S-1) become
// prefix chunk P / S.  One workgroup per (sequence, KV head):
//   landmark   mean of RoPE(x_t, t) over the S tokens (x: pre-RoPE keys)
//   residuals  R_t = v_t - MLP(C_t B_blk) in fp32 (the coefficient rows of the
//              S tokens are already in the cache); every token with
//              ||R_t|| >= the head's threshold gets the next residual row,
//              while rows remain (otherwise it is counted as dropped)
//   descriptor (first new row << 8) | mask of the kept tokens
//   window     rows S .. W-1 move to 0 .. W-S-1 (k and v)
// ---------------------------------------------------------------------------


__global__ __launch_bounds__(256) void append_kernel(const AppendArgs a) {
  __shared__ float cs[kChunk][512];          // coefficient rows (decoded)
  __shared__ float kp[kChunk][kHeadDim];     // rebuilt pre-RoPE keys
  __shared__ float hid[kChunk][kHidden];     // GELU activations
  __shared__ float res[kChunk][kHeadDim];    // residual rows
  __shared__ float err2[kChunk];
  __shared__ int rowmap[kChunk];
  const int tid = threadIdx.x, h = blockIdx.x, b = blockIdx.y;
  const size_t head = (size_t)b * a.hkv + h;
  const int r = a.r;

  // coefficient rows of the S tokens
  for (int idx = tid; idx < kChunk * r; idx += 256) {
    const int i = idx / r, m = idx % r;
    const size_t row = (size_t)b * a.prefix_cap + a.P + i;
    float c;
    if (!a.ci4) {
      c = bf16_to_f32(static_cast<const uint16_t*>(a.coeff)[row * r + m]);
    } else {
      const uint8_t byte = static_cast<const uint8_t*>(a.coeff)[row * (r / 2) + m / 2];
      const int code = ((int)((uint32_t)byte << (28 - 4 * (m & 1)) ) ) >> 28;
      c = (float)code * f16_to_f32(a.coeff_scale[row * (r / 32) + m / 32]);
    }
    cs[i][m] = c;
  }
  __syncthreads();
  // K_pre[i][d] = sum_m C[i][m] blk[d][m]: thread -> d = tid % 128, tokens 4 (tid / 128) .. + 3
  {
    const int d = tid & 127, i0 = 4 * (tid >> 7);
    const uint16_t* br = a.blk + (head * kHeadDim + d) * r;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int m = 0; m < r; ++m) {
      const float bv = bf16_to_f32(br[m]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(cs[i0 + e][m], bv, acc[e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) kp[i0 + e][d] = acc[e];
  }
  __syncthreads();
  // hidden unit j = tid: z = W1[j] . K_pre + b1[j], h = x Phi(x) (erf form)
  {
    const int j = tid;
    const uint16_t* wr = a.w1 + (head * kHidden + j) * kHeadDim;
    float acc[kChunk];
    const float bias = bf16_to_f32(a.b1[head * kHidden + j]);
#pragma unroll
    for (int i = 0; i < kChunk; ++i) acc[i] = bias;
    for (int d = 0; d < kHeadDim; ++d) {
      const float wv = bf16_to_f32(wr[d]);
#pragma unroll
      for (int i = 0; i < kChunk; ++i) acc[i] = fmaf(wv, kp[i][d], acc[i]);
    }
#pragma unroll
    for (int i = 0; i < kChunk; ++i) hid[i][j] = 0.5f * acc[i] * (1.0f + erff(acc[i] * 0.70710678118654752f));
  }
  __syncthreads();
  // V~[i][d] = W2[d] . h[i] + b2[d]; R = v - V~  (v: window rows 0 .. S-1)
  {
    const int d = tid & 127, i0 = 4 * (tid >> 7);
    const uint16_t* wr = a.w2 + (head * kHeadDim + d) * kHidden;
    const float bias = bf16_to_f32(a.b2[head * kHeadDim + d]);
    float acc[4] = {bias, bias, bias, bias};
    for (int j = 0; j < kHidden; ++j) {
      const float wv = bf16_to_f32(wr[j]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = fmaf(wv, hid[i0 + e][j], acc[e]);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float v = bf16_to_f32(a.win_v[(head * a.window_cap + i0 + e) * kHeadDim + d]);
      res[i0 + e][d] = v - acc[e];
    }
  }
  __syncthreads();
  // ||R_i||^2: token i = tid / 32, 4 dims per lane, 32-lane reduction
  {
    const int i = tid >> 5, l = tid & 31;
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) ss = fmaf(res[i][l + 32 * k], res[i][l + 32 * k], ss);
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    if (l == 0) err2[i] = ss;
  }
  __syncthreads();
  const int nc = a.P / kChunk;
  if (tid == 0) {
    const float tau = a.thresh[head];
    int cnt = a.count[head], drop = 0;
    const int first = cnt;
    uint32_t mask = 0;
    for (int i = 0; i < kChunk; ++i) {
      rowmap[i] = -1;
      if (sqrtf(err2[i]) >= tau) {
        if (cnt < a.resid_cap) {
          rowmap[i] = cnt;
          a.res_idx[head * a.resid_cap + cnt] = a.P + i;
          mask |= 1u << i;
          ++cnt;
        } else {
          ++drop;
        }
      }
    }
    a.desc[head * (a.prefix_cap / kChunk) + nc] = ((uint32_t)first << 8) | mask;
    a.count[head] = cnt;
    a.dropped[head] += drop;
  }
  // landmark: thread p < 64 owns the rotate-half pair (p, p + 64)
  if (tid < 64) {
    const int p = tid;
    const uint16_t* xs = a.keys_new + (size_t)b * kChunk * a.D + (a.layer_in_group * a.hkv + h) * kHeadDim;
    float y1 = 0.f, y2 = 0.f;
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const float x1 = bf16_to_f32(xs[(size_t)i * a.D + p]);
      const float x2 = bf16_to_f32(xs[(size_t)i * a.D + p + 64]);
      const float2 cs2 = rot_of((double)(a.P + i) * a.inv_freq[p]);
      y1 += x1 * cs2.x - x2 * cs2.y;
      y2 += x2 * cs2.x + x1 * cs2.y;
    }
    uint16_t* o = a.landmark + (head * (a.prefix_cap / kChunk) + nc) * kHeadDim;
    o[p] = __builtin_bit_cast(uint16_t, (__bf16)(y1 * (1.0f / kChunk)));
    o[p + 64] = __builtin_bit_cast(uint16_t, (__bf16)(y2 * (1.0f / kChunk)));
  }
  __syncthreads();
  // residual rows of the kept tokens: thread -> (token tid / 4, group tid % 4)
  if (tid < kChunk * 4) {
    const int i = tid >> 2, j = tid & 3;
    const int row = rowmap[i];
    if (row >= 0) {
      const size_t orow = head * a.resid_cap + row;
      if (a.ri4)
        encode_group32(&res[i][32 * j], true, nullptr,
                       static_cast<uint8_t*>(a.res_val) + orow * (kHeadDim / 2) + 16 * j,
                       a.res_scale + orow * (kHeadDim / 32) + j);
      else
        encode_group32(&res[i][32 * j], false, static_cast<uint16_t*>(a.res_val) + orow * kHeadDim + 32 * j,
                       nullptr, nullptr);
    }
  }
  // window rows S .. W-1 -> 0 .. W-S-1, 16 rows per pass (read all, then write)
  for (int arr = 0; arr < 2; ++arr) {
    uint16_t* wb = (arr == 0 ? a.win_k : a.win_v) + head * a.window_cap * kHeadDim;
    for (int r0 = 0; r0 < a.W - kChunk; r0 += 16) {
      const int row = r0 + (tid >> 4), piece = tid & 15;
      const bool live = row < a.W - kChunk;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (live) v = *reinterpret_cast<const u32x4*>(wb + (size_t)(row + kChunk) * kHeadDim + 8 * piece);
      __syncthreads();
      if (live) *reinterpret_cast<u32x4*>(wb + (size_t)row * kHeadDim + 8 * piece) = v;
      __syncthreads();
    }
  }
}

hipError_t launch_append(const AppendArgs& a, int nb, hipStream_t st) {
  hipLaunchKernelGGL(append_kernel, dim3(a.hkv, nb), dim3(256), 0, st, a);
  return hipGetLastError();
}

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int n, int32_t v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t st) {
  if (n > 0) hipLaunchKernelGGL(fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

hipError_t launch_resid_store(const float* r, const int32_t* idx, void* res_val, uint16_t* res_scale,
                              const BuildGeo& g, bool int4, hipStream_t st) {
  const size_t n_rows = (size_t)g.nb * g.hkv * g.n_resid;
  if (n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(resid_store_kernel, dim3((unsigned)((n_rows * 4 + 255) / 256)), dim3(256), 0, st, r, idx,
                     res_val, res_scale, n_rows, g, int4);
  return hipGetLastError();
}

}  // namespace lowram
