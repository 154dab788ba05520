// Randomised Cholesky-QR fit of a layer group's key basis, gfx950.
//
// LowRAM review (agihunt.info), key paragraph: adjacent layers share one
// low-rank basis of their pre-RoPE keys, and a randomised Cholesky-QR
// replaces the exact SVD.  For X [P][D] (a group's prefix keys) and a
// Gaussian Omega [P][r] (an input, given transposed [r][P]):
//   Y = X^T Omega                          (MFMA GEMM, contraction over tokens)
//   Y = CholQR2(Y)                         (G = Y^T Y, R = chol(G), Y <- Y R^-1, twice)
//   power passes: W = X Y, Y = CholQR2(X^T W)
//   B = Y^T                                ([r][D] bf16, orthonormal rows)
// The GEMMs use the projection kernel (both operands contiguous along the
// contraction: X^T is materialised once).  The small r x r algebra runs in
// fp64 with 64 x 64 blocks: a Gram kernel, a blocked right-looking Cholesky
// (diagonal block factor + inverse in one workgroup, panel solve, trailing
// update) and a blocked triangular solve that overwrites Y with Q.
#include <cmath>

#include "common.h"
#include "internal.h"

namespace lowram {

constexpr int kBlk = 64;

// out[c][r] = in[r * ld_in + c] (bf16), a rows x cols tile transpose per workgroup of 64 x 64
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ in, uint16_t* __restrict__ out,
                                                             int rows, int cols, int ld_in, int ld_out) {
  __shared__ uint16_t t[64][66];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64, tid = threadIdx.x;
  for (int i = tid; i < 64 * 64; i += 256) {
    const int rr = i / 64, cc = i % 64;
    if (r0 + rr < rows && c0 + cc < cols) t[rr][cc] = in[(size_t)(r0 + rr) * ld_in + c0 + cc];
  }
  __syncthreads();
  for (int i = tid; i < 64 * 64; i += 256) {
    const int cc = i / 64, rr = i % 64;
    if (r0 + rr < rows && c0 + cc < cols) out[(size_t)(c0 + cc) * ld_out + r0 + rr] = t[rr][cc];
  }
}

// out[c][r] = bf16(in[r][c]) for an fp32 [rows][cols] matrix
__global__ __launch_bounds__(256) void transpose_f32_bf16_kernel(const float* __restrict__ in, uint16_t* __restrict__ out,
                                                                 int rows, int cols) {
  __shared__ float t[64][65];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64, tid = threadIdx.x;
  for (int i = tid; i < 64 * 64; i += 256) {
    const int rr = i / 64, cc = i % 64;
    if (r0 + rr < rows && c0 + cc < cols) t[rr][cc] = in[(size_t)(r0 + rr) * cols + c0 + cc];
  }
  __syncthreads();
  for (int i = tid; i < 64 * 64; i += 256) {
    const int cc = i / 64, rr = i % 64;
    if (r0 + rr < rows && c0 + cc < cols)
      out[(size_t)(c0 + cc) * rows + r0 + rr] = __builtin_bit_cast(uint16_t, (__bf16)t[rr][cc]);
  }
}

// Partial G[z][i][j] = sum over rows n of chunk z of Y[n][i] Y[n][j] (fp64), one 64 x 64
// block per workgroup (grid r/64 x r/64 x chunks; chunk = rows per split)
__global__ __launch_bounds__(256) void gram_kernel(const float* __restrict__ y, double* __restrict__ g, int n, int r,
                                                   int chunk) {
  __shared__ float ya[16][kBlk + 1], yb[16][kBlk + 1];
  const int i0 = blockIdx.x * kBlk, j0 = blockIdx.y * kBlk, tid = threadIdx.x;
  const int ti = tid / 16, tj = tid % 16;  // 4 x 4 outputs: rows ti + 16 a, cols tj + 16 b
  const int nbeg = blockIdx.z * chunk, nend = min(n, nbeg + chunk);
  g += (size_t)blockIdx.z * r * r;
  double acc[4][4] = {};
  for (int n0 = nbeg; n0 < nend; n0 += 16) {
    for (int idx = tid; idx < 16 * kBlk; idx += 256) {
      const int rr = idx / kBlk, cc = idx % kBlk;
      const bool in = n0 + rr < nend;
      ya[rr][cc] = in ? y[(size_t)(n0 + rr) * r + i0 + cc] : 0.f;
      yb[rr][cc] = in ? y[(size_t)(n0 + rr) * r + j0 + cc] : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int k = 0; k < 16; ++k) {
      double av[4], bv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) av[a] = ya[k][ti + 16 * a];
#pragma unroll
      for (int b = 0; b < 4; ++b) bv[b] = yb[k][tj + 16 * b];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fma(av[a], bv[b], acc[a][b]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) g[(size_t)(i0 + ti + 16 * a) * r + j0 + tj + 16 * b] = acc[a][b];
}

// Diagonal block kb: factor A_kk = R_kk^T R_kk in LDS, write R_kk into the
// upper triangle of g and R_kk^-1 into dinv[kb].  Symmetric elimination with
// one barrier per step (a_ik -= a_ji a_jk / a_jj on the upper triangle, rows
// below j), then R[j][k] = a[j][k] / sqrt(a[j][j]); the inverse by the same
// kind of sweep, bottom row first (x_j = b_j / R_jj, then b_i -= R_ij x_j).
// A non-positive pivot sets *status = 1 and continues with pivot 1.
__global__ __launch_bounds__(256) void chol_diag_kernel(double* __restrict__ g, double* __restrict__ dinv, int r, int kb,
                                                        int* __restrict__ status) {
  __shared__ double a[kBlk][kBlk + 1];
  __shared__ double xs[kBlk][kBlk + 1];
  const int tid = threadIdx.x, o = kb * kBlk;
  for (int idx = tid; idx < kBlk * kBlk; idx += 256) a[idx / kBlk][idx % kBlk] = g[(size_t)(o + idx / kBlk) * r + o + idx % kBlk];
  __syncthreads();
  // thread -> column k = tid % 64, rows i = tid / 64 + 4 q
  const int k = tid & 63, i0 = tid >> 6;
  for (int j = 0; j < kBlk; ++j) {
    double d = a[j][j];
    if (!(d > 0.0)) d = 1.0;
    const double ajk = a[j][k] / d;
    // all loads of the step first (row j is not written in step j), then the updates
    double rj[kBlk / 4], aik[kBlk / 4];
#pragma unroll
    for (int q = 0; q < kBlk / 4; ++q) {
      rj[q] = a[j][i0 + 4 * q];
      aik[q] = a[i0 + 4 * q][k];
    }
#pragma unroll
    for (int q = 0; q < kBlk / 4; ++q) {
      const int i = i0 + 4 * q;
      if (k > j && i > j && i <= k) a[i][k] = aik[q] - rj[q] * ajk;
    }
    __syncthreads();
  }
  if (tid < kBlk && !(a[tid][tid] > 0.0)) *status = 1;
  // R = a / sqrt(diag) by rows (upper); lower part 0
  for (int idx = tid; idx < kBlk * kBlk; idx += 256) {
    const int ii = idx / kBlk, kk = idx % kBlk;
    const double dd = a[ii][ii] > 0.0 ? a[ii][ii] : 1.0;
    xs[ii][kk] = kk >= ii ? a[ii][kk] / sqrt(dd) : 0.0;
  }
  __syncthreads();
  for (int idx = tid; idx < kBlk * kBlk; idx += 256) {
    const int ii = idx / kBlk, kk = idx % kBlk;
    g[(size_t)(o + ii) * r + o + kk] = xs[ii][kk];
    a[ii][kk] = ii == kk ? 1.0 : 0.0;  // b = I
  }
  __syncthreads();
  // inverse: rows of x from the bottom; x_j = b_j / R_jj; b_i -= R_ij x_j (i < j)
  for (int jj = kBlk - 1; jj >= 0; --jj) {
    const double xj = a[jj][k] / xs[jj][jj];
    double rij[kBlk / 4], bik[kBlk / 4];
#pragma unroll
    for (int q = 0; q < kBlk / 4; ++q) {
      rij[q] = xs[i0 + 4 * q][jj];
      bik[q] = a[i0 + 4 * q][k];
    }
#pragma unroll
    for (int q = 0; q < kBlk / 4; ++q)
      if (i0 + 4 * q < jj) a[i0 + 4 * q][k] = bik[q] - rij[q] * xj;
    __syncthreads();
    if (tid < kBlk) a[jj][k] = xj;  // row jj is final (not read again by the update)
    __syncthreads();
  }
  double* inv = dinv + (size_t)kb * kBlk * kBlk;
  for (int idx = tid; idx < kBlk * kBlk; idx += 256) inv[idx] = a[idx / kBlk][idx % kBlk];
}

// Panel: R_kj = R_kk^-T A_kj for every block column j > kb (one per workgroup).
__global__ __launch_bounds__(256) void chol_panel_kernel(double* __restrict__ g, const double* __restrict__ dinv, int r,
                                                         int kb) {
  __shared__ double inv[kBlk][kBlk + 1], a[kBlk][kBlk + 1];
  const int tid = threadIdx.x, o = kb * kBlk, j0 = (kb + 1 + blockIdx.x) * kBlk;
  const double* di = dinv + (size_t)kb * kBlk * kBlk;
  for (int idx = tid; idx < kBlk * kBlk; idx += 256) {
    inv[idx / kBlk][idx % kBlk] = di[idx];
    a[idx / kBlk][idx % kBlk] = g[(size_t)(o + idx / kBlk) * r + j0 + idx % kBlk];
  }
  __syncthreads();
  const int ti = tid / 16, tj = tid % 16;
  double acc[4][4] = {};
  for (int l = 0; l < kBlk; ++l) {
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[p][q] = fma(inv[l][ti + 16 * p], a[l][tj + 16 * q], acc[p][q]);
  }
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) g[(size_t)(o + ti + 16 * p) * r + j0 + tj + 16 * q] = acc[p][q];
}

// Trailing update A_ij -= R_ki^T R_kj for kb < i <= j (grid nbr x nbr, lower half idle).
__global__ __launch_bounds__(256) void chol_update_kernel(double* __restrict__ g, int r, int kb) {
  const int bi = kb + 1 + blockIdx.x, bj = kb + 1 + blockIdx.y;
  if (bi > bj) return;
  __shared__ double ri[kBlk][kBlk + 1], rj[kBlk][kBlk + 1];
  const int tid = threadIdx.x, o = kb * kBlk;
  for (int idx = tid; idx < kBlk * kBlk; idx += 256) {
    const int l = idx / kBlk, c = idx % kBlk;
    ri[l][c] = g[(size_t)(o + l) * r + bi * kBlk + c];
    rj[l][c] = g[(size_t)(o + l) * r + bj * kBlk + c];
  }
  __syncthreads();
  const int ti = tid / 16, tj = tid % 16;
  double acc[4][4] = {};
  for (int l = 0; l < kBlk; ++l) {
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[p][q] = fma(ri[l][ti + 16 * p], rj[l][tj + 16 * q], acc[p][q]);
  }
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) g[(size_t)(bi * kBlk + ti + 16 * p) * r + bj * kBlk + tj + 16 * q] -= acc[p][q];
}

// Block column kb of Q = Y R^-1, in place over Y [n][r] (fp32):
// Q[:, kb] = (Y[:, kb] - sum_{i < kb} Q[:, i] R[i][kb]) R_kk^-1, 64 rows per workgroup.
__global__ __launch_bounds__(256) void trsm_kernel(float* __restrict__ y, const double* __restrict__ g,
                                                   const double* __restrict__ dinv, int n, int r, int kb) {
  __shared__ float qt[kBlk][kBlk + 1];
  __shared__ double rb[kBlk][kBlk + 1];
  const int tid = threadIdx.x, n0 = blockIdx.x * kBlk, o = kb * kBlk;
  const int ti = tid / 16, tj = tid % 16;  // rows ti + 16 p, cols tj + 16 q
  double acc[4][4];
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = n0 + ti + 16 * p;
      acc[p][q] = row < n ? (double)y[(size_t)row * r + o + tj + 16 * q] : 0.0;
    }
  for (int ib = 0; ib < kb; ++ib) {
    __syncthreads();
    for (int idx = tid; idx < kBlk * kBlk; idx += 256) {
      const int a = idx / kBlk, c = idx % kBlk;
      qt[a][c] = n0 + a < n ? y[(size_t)(n0 + a) * r + ib * kBlk + c] : 0.f;
      rb[a][c] = g[(size_t)(ib * kBlk + a) * r + o + c];
    }
    __syncthreads();
    for (int l = 0; l < kBlk; ++l) {
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[p][q] = fma(-(double)qt[ti + 16 * p][l], rb[l][tj + 16 * q], acc[p][q]);
    }
  }
  // times R_kk^-1: stage the partial rows (fp64 through two fp32 halves would lose bits; use rb for inv)
  __shared__ double part[kBlk][kBlk + 1];
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) part[ti + 16 * p][tj + 16 * q] = acc[p][q];
  const double* di = dinv + (size_t)kb * kBlk * kBlk;
  for (int idx = tid; idx < kBlk * kBlk; idx += 256) rb[idx / kBlk][idx % kBlk] = di[idx];
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 4; ++p)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      double v = 0.0;
      for (int l = 0; l < kBlk; ++l) v = fma(part[ti + 16 * p][l], rb[l][tj + 16 * q], v);
      const int row = n0 + ti + 16 * p;
      if (row < n) y[(size_t)row * r + o + tj + 16 * q] = (float)v;
    }
}

__global__ void zero_i32_kernel(int* p) { *p = 0; }

// g[i] = sum_z part[z][i] (fp64)
__global__ __launch_bounds__(256) void gram_sum_kernel(double* __restrict__ g, const double* __restrict__ part, int n,
                                                       int splits) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  double v = 0.0;
  for (int z = 0; z < splits; ++z) v += part[(size_t)z * n + i];
  g[i] = v;
}

constexpr int kGramRows = 256;   // rows of Y per Gram split
constexpr int kGemmSplits = 16;  // K splits of the token-contraction GEMMs

// One Cholesky-QR pass over y [n][r] in place; g [r][r], dinv [r/64][64][64], gpart
// [ceil(n / kGramRows)][r][r] scratch.
static hipError_t cholqr_pass(float* y, int n, int r, double* g, double* dinv, double* gpart, int* status,
                              hipStream_t st) {
  const int nbk = r / kBlk;
  const int gs = (n + kGramRows - 1) / kGramRows;
  hipLaunchKernelGGL(gram_kernel, dim3(nbk, nbk, gs), dim3(256), 0, st, y, gpart, n, r, kGramRows);
  hipLaunchKernelGGL(gram_sum_kernel, dim3((r * r + 255) / 256), dim3(256), 0, st, g, gpart, r * r, gs);
  for (int kb = 0; kb < nbk; ++kb) {
    hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(256), 0, st, g, dinv, r, kb, status);
    const int rest = nbk - kb - 1;
    if (rest > 0) {
      hipLaunchKernelGGL(chol_panel_kernel, dim3(rest), dim3(256), 0, st, g, dinv, r, kb);
      hipLaunchKernelGGL(chol_update_kernel, dim3(rest, rest), dim3(256), 0, st, g, r, kb);
    }
  }
  for (int kb = 0; kb < nbk; ++kb)
    hipLaunchKernelGGL(trsm_kernel, dim3((n + kBlk - 1) / kBlk), dim3(256), 0, st, y, g, dinv, n, r, kb);
  return hipGetLastError();
}

hipError_t launch_fit_basis(const uint16_t* keys, const uint16_t* omega_t, uint16_t* basis_out, int nb, int T,
                            int P, int D, int r, int power, void* ws, int* status, hipStream_t st) {
  unsigned char* w = static_cast<unsigned char*>(ws);
  uint16_t* xt = reinterpret_cast<uint16_t*>(w);                       // [D][P]
  w += ((size_t)D * P * 2 + 255) & ~(size_t)255;
  float* y = reinterpret_cast<float*>(w);                               // [D][r]
  w += ((size_t)D * r * 4 + 255) & ~(size_t)255;
  double* g = reinterpret_cast<double*>(w);                             // [r][r]
  w += ((size_t)r * r * 8 + 255) & ~(size_t)255;
  double* dinv = reinterpret_cast<double*>(w);                          // [r/64][64][64]
  w += ((size_t)r * kBlk * 8 + 255) & ~(size_t)255;
  uint16_t* qt = reinterpret_cast<uint16_t*>(w);                        // [r][D] bf16
  w += ((size_t)r * D * 2 + 255) & ~(size_t)255;
  uint16_t* wt = reinterpret_cast<uint16_t*>(w);                        // [r][P] bf16
  w += ((size_t)r * P * 2 + 255) & ~(size_t)255;
  double* gpart = reinterpret_cast<double*>(w);                         // [D/256][r][r]
  w += ((size_t)((D + kGramRows - 1) / kGramRows) * r * r * 8 + 255) & ~(size_t)255;
  float* ypart = reinterpret_cast<float*>(w);                           // [splits][D][r]
  for (int b = 0; b < nb; ++b) {
    const uint16_t* xb = keys + (size_t)b * T * D;
    int* sb = status + b;
    hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(1), 0, st, sb);
    hipLaunchKernelGGL(transpose_bf16_kernel, dim3((P + 63) / 64, (D + 63) / 64), dim3(256), 0, st, xb, xt, P, D, D,
                       P);
    // Y = X^T Omega: rows D, contraction P
    hipError_t e = launch_gemm_nt(xt, omega_t + (size_t)b * r * P, 1, D, D, P, r, 1, y, nullptr, 0, st,
                                  kGemmSplits, ypart);
    if (e != hipSuccess) return e;
    for (int pass = 0; pass < 2; ++pass)
      if ((e = cholqr_pass(y, D, r, g, dinv, gpart, sb, st)) != hipSuccess) return e;
    for (int it = 0; it < power; ++it) {
      hipLaunchKernelGGL(transpose_f32_bf16_kernel, dim3((D + 63) / 64, (r + 63) / 64), dim3(256), 0, st, y, qt, D, r);
      // W^T = (X Q)^T: rows P (tokens), contraction D
      if ((e = launch_gemm_nt(xb, qt, 1, T, P, D, r, 2, nullptr, wt, P, st)) != hipSuccess) return e;
      // Y = X^T W: rows D, contraction P
      if ((e = launch_gemm_nt(xt, wt, 1, D, D, P, r, 1, y, nullptr, 0, st, kGemmSplits, ypart)) != hipSuccess)
        return e;
      for (int pass = 0; pass < 2; ++pass)
        if ((e = cholqr_pass(y, D, r, g, dinv, gpart, sb, st)) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(transpose_f32_bf16_kernel, dim3((D + 63) / 64, (r + 63) / 64), dim3(256), 0, st, y,
                       basis_out + (size_t)b * r * D, D, r);
  }
  return hipGetLastError();
}

size_t fit_basis_ws_bytes(int P, int D, int r) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al((size_t)D * P * 2) + al((size_t)D * r * 4) + al((size_t)r * r * 8) + al((size_t)r * kBlk * 8) +
         al((size_t)r * D * 2) + al((size_t)r * P * 2) + al((size_t)((D + kGramRows - 1) / kGramRows) * r * r * 8) +
         al((size_t)kGemmSplits * D * r * 4);
}

}  // namespace lowram
