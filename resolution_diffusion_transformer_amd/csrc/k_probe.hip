// Measurement kernel: the matrix-core rate the chip sustains on a
// register-only v_mfma_f32_32x32x16_f16 stream (no memory traffic, no VALU
// work).  It is the ceiling the attention kernels are compared with next to
// the published peak, since the shader clock under load sits below the
// nominal 2.4 GHz.
#include <hip/hip_runtime.h>

#include <string>

#include "area_internal.h"

namespace area {

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kProbeWgPerCu = 8;    // 256-thread work-groups per CU (2 waves per SIMD)
constexpr int kProbeIters = 8192;   // loop trips per wave, 4 MFMAs each

// Four independent accumulator chains keep the matrix pipe full; the
// operands depend on the lane so the loop cannot be folded, and the result
// is stored only under a condition that never holds for these operands.
__global__ __launch_bounds__(256) void mfma_peak_kernel(float* __restrict__ sink, int iters) {
  f16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(1e-3f * (float)((threadIdx.x + i) & 7));
    b[i] = (_Float16)(1e-3f * (float)((threadIdx.x * 3 + i) & 7));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (s == -1.0f) sink[0] = s;
}

int hip_fail(const char* what, hipError_t e) {
  return fail(AREA_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace

int measure_mfma_peak(void* sink, double* tflops, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail("device query", e);
  const int blocks = cus * kProbeWgPerCu;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  int rc = AREA_OK;
  e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e != hipSuccess) rc = hip_fail("hipEventCreate", e);
  float ms = 0.0f;
  for (int pass = 0; pass < 2 && rc == AREA_OK; ++pass) {  // pass 0 warms up the clock
    e = hipEventRecord(e0, st);
    if (e == hipSuccess) {
      hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (float*)sink, kProbeIters);
      e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(e1, st);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e != hipSuccess) rc = hip_fail("mfma_peak_kernel", e);
  }
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (rc) return rc;
  const double flops = (double)blocks * 4.0 /* waves */ * kProbeIters * 4.0 * (32.0 * 32.0 * 16.0 * 2.0);
  *tflops = ms > 0.0f ? flops / (ms * 1e-3) / 1e12 : 0.0;
  return AREA_OK;
}

}  // namespace area
