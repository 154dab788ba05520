// Achievable-peak probes for the benchmark (not part of the decode library):
// a streaming HBM read and a register-only MFMA loop, each timed with HIP
// events around a few launches on the caller's device.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// workgroup b reads 16-byte pieces [b per, (b + 1) per), 8 non-temporal loads
// in flight per thread; per is a multiple of 2048
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ p, size_t per, uint32_t* out) {
  const u32x4* q = p + (size_t)blockIdx.x * per;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t i = threadIdx.x; i < per; i += 2048) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(q + i + 256 * u);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// 8 independent accumulator chains of v_mfma_f32_16x16x32_bf16 per wave
__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(0.001f * (lane + e));
    b[e] = (__bf16)(0.002f * (lane - e));
  }
  f32x4 c[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) c[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[k], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) s += c[k][0] + c[k][1] + c[k][2] + c[k][3];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

template <typename F>
int time_ms(F launch, int reps, float* ms) {
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess) return -1;
  if (hipEventCreate(&b) != hipSuccess) return -1;
  launch();
  int rc = 0;
  if (hipEventRecord(a, 0) != hipSuccess) rc = -1;
  for (int r = 0; r < reps && rc == 0; ++r) launch();
  if (rc == 0 && hipEventRecord(b, 0) != hipSuccess) rc = -1;
  if (rc == 0 && hipEventSynchronize(b) != hipSuccess) rc = -1;
  if (rc == 0 && hipEventElapsedTime(ms, a, b) != hipSuccess) rc = -1;
  if (rc == 0 && hipGetLastError() != hipSuccess) rc = -1;
  *ms /= reps;
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  return rc;
}

}  // namespace

extern "C" {

// Read rate of `bytes` (a multiple of n_wg * 32 KiB) at device pointer buf,
// split over n_wg workgroups: GB/s in *gbs.  0 on success, -1 on a HIP error.
int peaks_read_gbs(const void* buf, size_t bytes, int n_wg, void* scratch, double* gbs) {
  if (n_wg <= 0 || bytes % ((size_t)n_wg * 32768) != 0) return -2;
  const size_t per = bytes / 16 / n_wg;
  float ms = 0.f;
  const int rc = time_ms([&] {
    hipLaunchKernelGGL(read_kernel, dim3(n_wg), dim3(256), 0, 0, static_cast<const u32x4*>(buf), per,
                       static_cast<uint32_t*>(scratch));
  }, 5, &ms);
  *gbs = rc == 0 ? bytes / (ms * 1e-3) / 1e9 : 0.0;
  return rc;
}

// Dense bf16 MFMA rate (2 * 16 * 16 * 32 flops per instruction) of n_wg
// workgroups of 4 waves: TFLOP/s in *tfs.  scratch holds n_wg * 256 floats.
int peaks_mfma_tfs(int n_wg, int iters, void* scratch, double* tfs) {
  if (n_wg <= 0 || iters <= 0) return -2;
  float ms = 0.f;
  const int rc = time_ms([&] {
    hipLaunchKernelGGL(mfma_kernel, dim3(n_wg), dim3(256), 0, 0, iters, static_cast<float*>(scratch));
  }, 5, &ms);
  const double flops = (double)n_wg * 4 * iters * 8 * 2.0 * 16 * 16 * 32;
  *tfs = rc == 0 ? flops / (ms * 1e-3) / 1e12 : 0.0;
  return rc;
}

}  // extern "C"
