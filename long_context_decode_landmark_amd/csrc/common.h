// Internal helpers shared by the gfx950 kernels of the LowRAM decode library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lowram {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 128;
constexpr int kChunk = 8;
constexpr int kHidden = 256;
constexpr float kLog2e = 1.4426950408889634f;

// v_mfma_f32_16x16x32_bf16.  Lane l supplies A[l%16][8*(l/16)+e] and
// B[8*(l/16)+e][l%16] (e = 0..7); it receives D[4*(l/16)+e][l%16] (e = 0..3).
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Row order of a 32-row operand block: position 16 m + 4 g + e holds row
// 8 g + 4 m + e (m, g, e: m < 2, g < 4, e < 4).  With the A rows of MFMA tiles
// 2 s and 2 s + 1 taken in this order, the accumulators a lane (group g)
// receives for one output column are rows 32 s + 8 g + 0..7 in natural order:
// exactly the 8 consecutive k values that lane supplies as a B operand of a
// following MFMA, so a chain of products needs no transpose.
__device__ __forceinline__ constexpr int row_perm32(int pos) {
  return 8 * ((pos >> 2) & 3) + 4 * (pos >> 4) + (pos & 3);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t u) {
  return static_cast<float>(__builtin_bit_cast(_Float16, u));
}

// Eight floats -> bf16x8 (round to nearest even).
__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) {
  bf16x8 r;
  r[0] = (__bf16)lo[0]; r[1] = (__bf16)lo[1]; r[2] = (__bf16)lo[2]; r[3] = (__bf16)lo[3];
  r[4] = (__bf16)hi[0]; r[5] = (__bf16)hi[1]; r[6] = (__bf16)hi[2]; r[7] = (__bf16)hi[3];
  return r;
}

// Residual of the bf16 rounding of pack8, as a second bf16x8 (hi + lo split).
__device__ __forceinline__ bf16x8 pack8_lo(f32x4 lo, f32x4 hi, bf16x8 h) {
  bf16x8 r;
  r[0] = (__bf16)(lo[0] - (float)h[0]); r[1] = (__bf16)(lo[1] - (float)h[1]);
  r[2] = (__bf16)(lo[2] - (float)h[2]); r[3] = (__bf16)(lo[3] - (float)h[3]);
  r[4] = (__bf16)(hi[0] - (float)h[4]); r[5] = (__bf16)(hi[1] - (float)h[5]);
  r[6] = (__bf16)(hi[2] - (float)h[6]); r[7] = (__bf16)(hi[3] - (float)h[7]);
  return r;
}

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// 16-byte load with the non-temporal (streaming) cache policy: for data read
// once, whose 128-byte lines are consumed whole by neighbouring loads.
__device__ __forceinline__ u32x4 load_nt16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// ds_read_b64_tr_b16 (gfx950): in each block of 16 lanes, lane i receives
// element i % 4 of the 4-element (8-byte) row addressed by lane 4 j + i / 4 of
// its block, as its element j (j = 0..3).  Two of them give a lane the eight
// k values of an MFMA B operand from rows stored k-major (one row per k).
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ s16x4 lds_tr16(const unsigned char* base, int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(base + off));
}
__device__ __forceinline__ bf16x8 bf16x8_of(s16x4 lo, s16x4 hi) {
  return __builtin_bit_cast(bf16x8, s16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

// Two 4-element (8-byte) pieces -> one MFMA operand.
__device__ __forceinline__ bf16x8 load_bf16x4x2(const uint16_t* p0, const uint16_t* p1) {
  u32x2 a = *reinterpret_cast<const u32x2*>(p0);
  u32x2 b = *reinterpret_cast<const u32x2*>(p1);
  return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
}

// Raw buffer resource over `bytes` bytes at `base` (reads past the end
// return 0).  Loads through it take a 32-bit lane offset plus a wave-uniform
// SGPR offset, so no 64-bit address is kept per load.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buffer_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
}

// Order-preserving map fp32 -> uint32 (larger float -> larger key); -0 == +0.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// 2*pi split for the Cody-Waite reduction of large RoPE angles in fp64.
constexpr double kTwoPiHi = 6.283185307179586;
constexpr double kTwoPiLo = 2.4492935982947064e-16;
constexpr double kInvTwoPi = 0.15915494309189535;

// sin and cos on [-pi, pi]: odd / even minimax polynomials (linear-programming
// fit over the interval), largest error in fp32 7e-7 / 5e-7.  The argument
// arrives reduced, so no range reduction of a general sinf / cosf is paid.
constexpr float kSinP[6] = {9.9999964237e-01f, -1.6666558385e-01f, 8.3324396983e-03f,
                            -1.9809571677e-04f, 2.7007711196e-06f, -2.0404730350e-08f};
constexpr float kCosP[7] = {1.0000000000e+00f, -5.0000000000e-01f, 4.1666641831e-02f,
                            -1.3888442190e-03f, 2.4781049433e-05f, -2.7166586847e-07f,
                            1.7499086624e-09f};

// (cos, sin) of an angle, reduced mod 2 pi in fp64 (Cody-Waite, 2 pi in two parts)
__device__ __forceinline__ float2 rot_of(double angle) {
  const double k = rint(angle * kInvTwoPi);
  double r = fma(-k, kTwoPiHi, angle);
  r = fma(-k, kTwoPiLo, r);
  const float x = static_cast<float>(r), u = x * x;
  float sn = kSinP[5];
#pragma unroll
  for (int i = 4; i >= 0; --i) sn = fmaf(sn, u, kSinP[i]);
  float cs = kCosP[6];
#pragma unroll
  for (int i = 5; i >= 0; --i) cs = fmaf(cs, u, kCosP[i]);
  return make_float2(cs, x * sn);
}

// Map a 1-D grid onto logical work items so that each of the 8 XCDs (which
// receive workgroups round-robin) gets one contiguous range of items:
// neighbouring items share their per-head weights in that XCD's L2.
__device__ __forceinline__ int xcd_logical_block(int lin, int padded_total) {
  const int per = padded_total >> 3;
  return (lin & 7) * per + (lin >> 3);
}

}  // namespace lowram
