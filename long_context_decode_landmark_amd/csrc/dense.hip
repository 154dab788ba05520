// Dense GQA flash-decode over the full bf16 KV cache (the uncompressed
// baseline of the LowRAM review's results paragraph), gfx950, and the
// residual chunk-descriptor helper of the compressed cache layout.
//
// One workgroup = 4 waves covers a split of the context; each wave walks
// 32-token blocks with an online softmax.  QK on MFMA (K rows straight from
// HBM as the A operand, 16 B per lane), PV on MFMA with V as the B operand.
// Partial states go through the same split merge as the LowRAM step.
#include "common.h"
#include "internal.h"

namespace lowram {

__global__ __launch_bounds__(kAttWaves * 64) void dense_kernel(
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const uint16_t* __restrict__ q, float* __restrict__ part, int ctx, int hq, int hkv,
    int n_split, int tok_per_split, float scale_log2, int total, int padded_total) {
  __shared__ float mo[kAttWaves * 16 * kHeadDim];
  __shared__ float ml[2 * kAttWaves * 16];
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

  bf16x8 qn[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qn[s] = col < g ? load_bf16x8(qh + col * kHeadDim + 32 * s + 8 * grp) : zero_bf16x8();

  float m = -__builtin_huge_valf(), lsum = 0.f;
  f32x4 oacc[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) oacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int t_begin = split * tok_per_split;
  const int t_end = min(ctx, t_begin + tok_per_split);
  for (int w0 = t_begin + wave * kAttTokWave; w0 < t_end; w0 += kAttWaves * kAttTokWave) {
    const int nvalid = min(kAttTokWave, t_end - w0);
    f32x4 zacc[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int t = min(w0 + 16 * nt + col, ctx - 1);
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) z = mfma16(load_bf16x8(kh + (size_t)t * kHeadDim + 32 * s + 8 * grp), qn[s], z);
      zacc[nt] = z;
    }
    bf16x8 vb[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = min(w0 + 16 * (e >> 2) + 4 * grp + (e & 3), ctx - 1);
        vb[nt][e] = __builtin_bit_cast(__bf16, vh[(size_t)t * kHeadDim + 16 * nt + col]);
      }
    }
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
    const bf16x8 pa = pack8(f32x4{p[0][0], p[0][1], p[0][2], p[0][3]},
                            f32x4{p[1][0], p[1][1], p[1][2], p[1][3]});
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
#pragma unroll
      for (int e = 0; e < 4; ++e) oacc[nt][e] *= al[e];
      oacc[nt] = mfma16(pa, vb[nt], oacc[nt]);
    }
  }

#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
#pragma unroll
    for (int e = 0; e < 4; ++e) mo[(wave * 16 + 4 * grp + e) * kHeadDim + 16 * nt + col] = oacc[nt][e];
  if (grp == 0) {
    ml[wave * 16 + col] = m;
    ml[kAttWaves * 16 + wave * 16 + col] = lsum;
  }
  __syncthreads();
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
      o += mo[(w * 16 + j) * kHeadDim + d] * sc;
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
