// Device helpers shared by the two attention kernels (the 4-wave kernel of
// attend.hip and the producer/consumer kernel of attend_pipe.hip).
#pragma once

#include "common.h"

namespace lowram {

// GELU without transcendental instructions (v_exp / v_rcp issue at a
// quarter of the FMA rate): Phi(x) = 0.5 + x Q(x^2) for |x| <= 4, with Q of
// degree 6 fitted by linear-programming minimax of the GELU error x (Phi~ - Phi)
// under the constraint Phi~(4) = 1, and x clamped to +-4 (so Phi~ is exactly
// 1 or 0 beyond).  Largest deviation from x Phi(x) (erf form) over the real
// line in fp32: 1.9e-4, a fortieth of a bf16 step at 1, and the hidden
// activations are rounded to bf16 right after.
constexpr float kGeluClamp = 4.0f;
constexpr float kGeluQ[7] = {3.978703618e-01f, -6.455454975e-02f, 8.763747290e-03f, -8.121979772e-04f,
                             4.776486458e-05f, -1.588871555e-06f, 2.258899912e-08f};

// Reductions over the lane pairs {l, l ^ 16} and {l, l ^ 32} of a wave on
// the vector ALUs instead of the LDS crossbar: v_permlane16_swap with both
// operands the same register gives, at lane l, the values of lanes l & ~16
// and l | 16 (v_permlane32_swap: l & ~32 and l | 32).  Both lanes of a pair
// get the same result (the sum adds the lower lane's value first).
__device__ __forceinline__ float pair_max16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_max32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_add16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair_add32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float gelu_fast(float x) {
  const float xc = __builtin_amdgcn_fmed3f(x, -kGeluClamp, kGeluClamp);
  const float u = xc * xc;
  float q = kGeluQ[6];
#pragma unroll
  for (int k = 5; k >= 0; --k) q = fmaf(q, u, kGeluQ[k]);
  return x * fmaf(xc, q, 0.5f);
}

// The same GELU on packed fp16 pairs (two values per instruction), for a
// result that feeds an fp16 MFMA operand.  Phi(x) = 0.5 + x Q(s) with
// s = min(x^2 / 8 - 1, 1) in [-1, 1], where Q has degree 6 and fp16
// coefficients (least-squares fit with |x| weights on 0 <= x <= 4, then
// adjusted by single fp16 ulps to minimise the largest error of the whole
// fp16 evaluation).  The clamp of 0.5 + x Q(s) to [0, 1] (a free output
// modifier) makes Phi exactly 0 or 1 for |x| > 4, where s saturates.
// Against x Phi(x) (erf form) in fp16 arithmetic: rms error 9.2e-4 over
// N(0, 1.5) inputs, largest 3.9e-3 at |x| = 12 (the fp16 rounding of x
// itself); rounding the fp32 result to bf16 instead costs rms 3.6e-3.
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
constexpr float kGeluH[7] = {1.7590332031e-01f, -8.4167480469e-02f, 5.5480957031e-02f, -3.7506103516e-02f,
                             2.5482177734e-02f, -1.4076232910e-02f, 3.8471221924e-03f};

__device__ __forceinline__ h2 gelu_h2(h2 x) {
  const h2 u = x * x;
  h2 s = __builtin_elementwise_fma(u, h2{(_Float16)0.125f, (_Float16)0.125f}, h2{(_Float16)-1.f, (_Float16)-1.f});
  s = __builtin_elementwise_min(s, h2{(_Float16)1.f, (_Float16)1.f});
  h2 q = {(_Float16)kGeluH[6], (_Float16)kGeluH[6]};
#pragma unroll
  for (int k = 5; k >= 0; --k) q = __builtin_elementwise_fma(q, s, h2{(_Float16)kGeluH[k], (_Float16)kGeluH[k]});
  h2 t = __builtin_elementwise_fma(x, q, h2{(_Float16)0.5f, (_Float16)0.5f});
  t = __builtin_elementwise_min(__builtin_elementwise_max(t, h2{(_Float16)0.f, (_Float16)0.f}),
                                h2{(_Float16)1.f, (_Float16)1.f});
  return x * t;
}

// GELU of 8 fp32 values (lo[0..3], hi[0..3]) as one fp16 MFMA operand
__device__ __forceinline__ f16x8 gelu8_h(f32x4 lo, f32x4 hi) {
  const h2 a = gelu_h2(__builtin_convertvector(f32x2{lo[0], lo[1]}, h2));
  const h2 b = gelu_h2(__builtin_convertvector(f32x2{lo[2], lo[3]}, h2));
  const h2 c = gelu_h2(__builtin_convertvector(f32x2{hi[0], hi[1]}, h2));
  const h2 d = gelu_h2(__builtin_convertvector(f32x2{hi[2], hi[3]}, h2));
  return __builtin_shufflevector(__builtin_shufflevector(a, b, 0, 1, 2, 3), __builtin_shufflevector(c, d, 0, 1, 2, 3),
                                 0, 1, 2, 3, 4, 5, 6, 7);
}

// GELU (gelu_h2) of eight fp16 pairs in place, evaluated level by level
// across the pairs so that the dependent Horner chains interleave (one chain
// alone stalls on every step).
__device__ __forceinline__ void gelu_h2x8(h2 (&x)[8]) {
  h2 s[8], q[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) s[p] = x[p] * x[p];
#pragma unroll
  for (int p = 0; p < 8; ++p)
    s[p] = __builtin_elementwise_fma(s[p], h2{(_Float16)0.125f, (_Float16)0.125f}, h2{(_Float16)-1.f, (_Float16)-1.f});
#pragma unroll
  for (int p = 0; p < 8; ++p) s[p] = __builtin_elementwise_min(s[p], h2{(_Float16)1.f, (_Float16)1.f});
#pragma unroll
  for (int p = 0; p < 8; ++p)
    q[p] = __builtin_elementwise_fma(s[p], h2{(_Float16)kGeluH[6], (_Float16)kGeluH[6]},
                                     h2{(_Float16)kGeluH[5], (_Float16)kGeluH[5]});
#pragma unroll
  for (int k = 4; k >= 0; --k)
#pragma unroll
    for (int p = 0; p < 8; ++p) q[p] = __builtin_elementwise_fma(q[p], s[p], h2{(_Float16)kGeluH[k], (_Float16)kGeluH[k]});
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    h2 t = __builtin_elementwise_fma(x[p], q[p], h2{(_Float16)0.5f, (_Float16)0.5f});
    t = __builtin_elementwise_min(__builtin_elementwise_max(t, h2{(_Float16)0.f, (_Float16)0.f}),
                                  h2{(_Float16)1.f, (_Float16)1.f});
    x[p] = x[p] * t;
  }
}

// GELU of two 8-value operands at once.  Operand hn is (lo[hn], hi[hn]) as
// for gelu8_h.
__device__ __forceinline__ void gelu16_h(const f32x4 (&lo)[2], const f32x4 (&hi)[2], f16x8 (&out)[2]) {
  h2 x[8];
#pragma unroll
  for (int hn = 0; hn < 2; ++hn) {
    x[4 * hn + 0] = __builtin_convertvector(f32x2{lo[hn][0], lo[hn][1]}, h2);
    x[4 * hn + 1] = __builtin_convertvector(f32x2{lo[hn][2], lo[hn][3]}, h2);
    x[4 * hn + 2] = __builtin_convertvector(f32x2{hi[hn][0], hi[hn][1]}, h2);
    x[4 * hn + 3] = __builtin_convertvector(f32x2{hi[hn][2], hi[hn][3]}, h2);
  }
  gelu_h2x8(x);
#pragma unroll
  for (int hn = 0; hn < 2; ++hn)
    out[hn] = __builtin_shufflevector(__builtin_shufflevector(x[4 * hn], x[4 * hn + 1], 0, 1, 2, 3),
                                      __builtin_shufflevector(x[4 * hn + 2], x[4 * hn + 3], 0, 1, 2, 3),
                                      0, 1, 2, 3, 4, 5, 6, 7);
}

// Eight floats -> f16x8 (round to nearest even)
__device__ __forceinline__ f16x8 pack8h(f32x4 lo, f32x4 hi) {
  const h2 a = __builtin_convertvector(f32x2{lo[0], lo[1]}, h2);
  const h2 b = __builtin_convertvector(f32x2{lo[2], lo[3]}, h2);
  const h2 c = __builtin_convertvector(f32x2{hi[0], hi[1]}, h2);
  const h2 d = __builtin_convertvector(f32x2{hi[2], hi[3]}, h2);
  return __builtin_shufflevector(__builtin_shufflevector(a, b, 0, 1, 2, 3), __builtin_shufflevector(c, d, 0, 1, 2, 3),
                                 0, 1, 2, 3, 4, 5, 6, 7);
}

// v_mfma_f32_16x16x32_f16: the lane layout of mfma16 with fp16 operands
__device__ __forceinline__ f32x4 mfma16h(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

constexpr int kStage = 16384;  // bytes of one staged operand slice
constexpr int kStageLd = 4;    // 16-byte loads per thread per stage (256 threads)

constexpr int kResRow = 272;   // LDS stride of a bf16 residual row (256 + 16: rows on different banks)
constexpr int kResRow4 = 80;   // int4 residual row: 64 bytes of codes, 8 of scales, 8 unused

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

__device__ __forceinline__ bf16x8 lds16(const unsigned char* base, int off) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(base + off));
}

}  // namespace lowram
