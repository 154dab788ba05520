// Dense GQA flash-decode over the full bf16 KV cache (the uncompressed
// baseline of the LowRAM review's results paragraph), gfx950, and the
// residual chunk-descriptor helper of the compressed cache layout.
//
// One workgroup = 4 waves covers a split of the context; each wave walks
// 32-token blocks with an online softmax, loading block n + 1 while block n
// computes.  QK on MFMA (K rows straight from HBM as the A operand, 16 B per
// lane).  PV on MFMA with V as the B operand: V rows arrive in 16-byte pieces,
// go through a per-wave LDS block, and come back transposed (token-major per
// lane) with gfx950's LDS transpose read.  Every HBM load is a 16-byte
// non-temporal one: the streaming policy lifts the read rate, and each 128-byte
// line is consumed by the same or the next load instruction.
// Partial states go through the same split merge as the LowRAM step.
#include "common.h"
#include "internal.h"

namespace lowram {

constexpr int kDenseVBlock = kAttTokWave * kHeadDim * 2;  // bytes of one wave's V block in LDS

// Byte offset in a wave's V block of byte `byte` of token row r: rows of
// 256 B whose 32-byte groups are XOR-swizzled by (r & 7), so that the 16 rows
// one transpose read touches spread over all banks.
__device__ __forceinline__ int dense_voff(int r, int byte) {
  return r * 256 + ((((byte >> 5) ^ (r & 7)) << 5) | (byte & 31));
}

__global__ __launch_bounds__(kAttWaves * 64) void dense_kernel(
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const uint16_t* __restrict__ q, float* __restrict__ part, int ctx, int hq, int hkv,
    int n_split, int tok_per_split, float scale_log2, int total, int padded_total) {
  // per wave: its V block during the walk, its 16 x 128 fp32 output rows after
  __shared__ __attribute__((aligned(16))) unsigned char vblk[kAttWaves * kDenseVBlock];
  __shared__ float ml[2 * kAttWaves * 16];
  static_assert(kDenseVBlock == 16 * kHeadDim * 4, "output rows reuse the V block");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = lane >> 4, col = lane & 15;
  const int logical = xcd_logical_block(blockIdx.x, padded_total);
  if (logical >= total) return;
  const int bh = logical / n_split, split = logical % n_split;
  const int b = bh / hkv, h = bh % hkv;
  const int g = hq / hkv;
  const size_t head = (size_t)b * hkv + h;
  const uint16_t* qh = q + ((size_t)b * hq + (size_t)h * g) * kHeadDim;
  const uint16_t* kh = kc + head * (size_t)ctx * kHeadDim;
  const uint16_t* vh = vc + head * (size_t)ctx * kHeadDim;
  unsigned char* vb_lds = vblk + wave * kDenseVBlock;

  bf16x8 qn[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qn[s] = col < g ? load_bf16x8(qh + col * kHeadDim + 32 * s + 8 * grp) : zero_bf16x8();

  // LDS offsets: the V piece a lane writes (row 4 i + grp, bytes 16 col ..),
  // and the row piece it addresses for transpose read (h, nt): row
  // 16 h + 4 grp + col / 4, bytes 32 nt + 8 (col % 4) ..
  int woff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) woff[i] = dense_voff(4 * i + grp, 16 * col);
  int roff[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) roff[hh] = dense_voff(16 * hh + 4 * grp + (col >> 2), 8 * (col & 3));

  float m = -__builtin_huge_valf(), lsum = 0.f;
  f32x4 oacc[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) oacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int t_begin = split * tok_per_split;
  const int t_end = min(ctx, t_begin + tok_per_split);
  // K rows w0 + 16 nt + col (16-byte piece grp of each 64-byte quarter), V rows
  // w0 + 4 i + grp (16-byte piece col); block n + 1 is loaded while block n computes
  bf16x8 kr[2][4];
  u32x4 vr[8];
  auto load_block = [&](int w0) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int t = min(w0 + 16 * nt + col, ctx - 1);
#pragma unroll
      for (int s = 0; s < 4; ++s) kr[nt][s] = __builtin_bit_cast(bf16x8, load_nt16(kh + (size_t)t * kHeadDim + 32 * s + 8 * grp));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = min(w0 + 4 * i + grp, ctx - 1);
      vr[i] = load_nt16(vh + (size_t)t * kHeadDim + 8 * col);
    }
  };
  constexpr int kStride = kAttWaves * kAttTokWave;
  if (t_begin + wave * kAttTokWave < t_end) load_block(t_begin + wave * kAttTokWave);
  for (int w0 = t_begin + wave * kAttTokWave; w0 < t_end; w0 += kStride) {
    const int nvalid = min(kAttTokWave, t_end - w0);
    f32x4 zacc[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) z = mfma16(kr[nt][s], qn[s], z);
      zacc[nt] = z;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(vb_lds + woff[i]) = vr[i];
    if (w0 + kStride < t_end) load_block(w0 + kStride);
    float p[2][4];
    float mb = -__builtin_huge_valf();
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * nt + 4 * grp + e;
        p[nt][e] = t < nvalid ? zacc[nt][e] * scale_log2 : -__builtin_huge_valf();
        mb = fmaxf(mb, p[nt][e]);
      }
    mb = fmaxf(mb, __shfl_xor(mb, 16));
    mb = fmaxf(mb, __shfl_xor(mb, 32));
    const float mnew = fmaxf(m, mb);  // finite: every block has a valid token
    const float alpha = m == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f(m - mnew);
    float ls = 0.f;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[nt][e] = __builtin_amdgcn_exp2f(p[nt][e] - mnew);
        ls += p[nt][e];
      }
    ls += __shfl_xor(ls, 16);
    ls += __shfl_xor(ls, 32);
    lsum = lsum * alpha + ls;
    m = mnew;
    // o rows j = 4*grp + e need alpha of head j, held by lane j (col == j)
    float al[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) al[e] = __shfl(alpha, 4 * grp + e);
    // A operand: lane (grp, col) supplies P[head col][tokens 16 (e / 4) + 4 grp + e % 4]
    const bf16x8 pa = pack8(f32x4{p[0][0], p[0][1], p[0][2], p[0][3]},
                            f32x4{p[1][0], p[1][1], p[1][2], p[1][3]});
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      // B operand: lane (grp, col) receives V[tokens 16 hh + 4 grp + 0..3][16 nt + col]
      // from the transpose reads hh = 0, 1 (the same token order as pa)
      const s16x4 lo = lds_tr16(vb_lds, roff[0] ^ (nt << 5));
      const s16x4 hi = lds_tr16(vb_lds, roff[1] ^ (nt << 5));
      const bf16x8 vbn = bf16x8_of(lo, hi);
#pragma unroll
      for (int e = 0; e < 4; ++e) oacc[nt][e] *= al[e];
      oacc[nt] = mfma16(pa, vbn, oacc[nt]);
    }
  }

  float* mo = reinterpret_cast<float*>(vb_lds);  // this wave's 16 output rows
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
#pragma unroll
    for (int e = 0; e < 4; ++e) mo[(4 * grp + e) * kHeadDim + 16 * nt + col] = oacc[nt][e];
  if (grp == 0) {
    ml[wave * 16 + col] = m;
    ml[kAttWaves * 16 + wave * 16 + col] = lsum;
  }
  __syncthreads();
  const float* mall = reinterpret_cast<const float*>(vblk);
  float* pp = part + ((head * n_split + split) * (size_t)g) * kPartStride;
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
      o += mall[(w * 16 + j) * kHeadDim + d] * sc;
    }
    if (d == 0) {
      pp[j * kPartStride] = M;
      pp[j * kPartStride + 1] = lt;
    }
    pp[j * kPartStride + 2 + d] = o;
  }
}

hipError_t launch_dense(const uint16_t* k, const uint16_t* v, const uint16_t* q, float* part,
                        int nb, int ctx, int hq, int hkv, int n_split, int tok_per_split,
                        float scale_log2, hipStream_t st) {
  const int total = nb * hkv * n_split;
  const int padded = (total + 7) & ~7;
  hipLaunchKernelGGL(dense_kernel, dim3(padded), dim3(kAttWaves * 64), 0, st, k, v, q, part, ctx,
                     hq, hkv, n_split, tok_per_split, scale_log2, total, padded);
  return hipGetLastError();
}

// desc[l][c] = (lower bound of c*chunk in res_idx[l]) << 8 | bitmask of the
// chunk's tokens present in res_idx[l]
__global__ __launch_bounds__(256) void chunk_desc_kernel(const int32_t* __restrict__ idx, int n_resid,
                                                         int n_chunks, int chunk,
                                                         uint32_t* __restrict__ desc, int idx_stride,
                                                         int desc_stride) {
  const int l = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= n_chunks) return;
  const int32_t* r = idx + (size_t)l * idx_stride;
  const int key = c * chunk;
  int lo = 0, hi = n_resid;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (r[mid] < key) lo = mid + 1;
    else hi = mid;
  }
  uint32_t mask = 0;
  for (int i = lo; i < n_resid && r[i] < key + chunk; ++i) mask |= 1u << (r[i] - key);
  desc[(size_t)l * desc_stride + c] = ((uint32_t)lo << 8) | mask;
}

hipError_t launch_chunk_desc(const int32_t* res_idx, int n_lists, int n_resid, int n_chunks, int chunk,
                             uint32_t* desc, hipStream_t st, int idx_stride, int desc_stride) {
  const dim3 grid((n_chunks + 255) / 256, n_lists);
  hipLaunchKernelGGL(chunk_desc_kernel, grid, dim3(256), 0, st, res_idx, n_resid, n_chunks, chunk, desc,
                     idx_stride < 0 ? n_resid : idx_stride, desc_stride < 0 ? n_chunks : desc_stride);
  return hipGetLastError();
}

}  // namespace lowram
