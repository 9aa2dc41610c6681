// Peak-rate loop of the bf16 matrix cores and the device clocks (see include/cpa_diag.h).
//
// Each wave keeps four independent 32x32 accumulators and issues one v_mfma_f32_32x32x16_bf16
// into each per iteration, so the matrix core of its SIMD never waits for a result; nothing else
// runs in the loop.  Workgroup 0 reads the shader clock (s_memtime) and the constant-rate clock
// (s_memrealtime) around its loop, which gives the engine clock under a pure MFMA load.
#include "cpa_diag.h"

#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(512) void mfma_loop_kernel(int iters, float* sink, unsigned long long* clk) {
  const int tid = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1e-3f * (float)((tid + e) & 63));
    b[e] = (__bf16)(-1e-3f * (float)((tid * 3 + e) & 63));
  }
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  __syncthreads();
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  sink[(size_t)blockIdx.x * blockDim.x + tid] = s;
  if (blockIdx.x == 0 && tid == 0) {
    clk[0] = t1 - t0;
    clk[1] = r1 - r0;
  }
}

}  // namespace

extern "C" {

cpa_status cpa_diag_mfma_loop(int blocks, int threads, int iters, float* sink, unsigned long long* clk,
                              hipStream_t stream) {
  if (blocks < 1 || threads < 64 || threads > 512 || threads % 64 != 0 || iters < 1 || iters > 10000000)
    return CPA_ERR_SHAPE;
  if (!sink || !clk) return CPA_ERR_NULL;
  if (((uintptr_t)clk & 7u) != 0 || ((uintptr_t)sink & 3u) != 0) return CPA_ERR_ALIGN;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(threads), 0, stream, iters, sink, clk);
  return hipGetLastError() == hipSuccess ? CPA_OK : CPA_ERR_LAUNCH;
}

cpa_status cpa_diag_clock_rates(int device, int* engine_khz, int* wall_khz) {
  if (!engine_khz || !wall_khz) return CPA_ERR_NULL;
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n) return CPA_ERR_SHAPE;
  if (hipDeviceGetAttribute(engine_khz, hipDeviceAttributeClockRate, device) != hipSuccess) return CPA_ERR_SHAPE;
  if (hipDeviceGetAttribute(wall_khz, hipDeviceAttributeWallClockRate, device) != hipSuccess) return CPA_ERR_SHAPE;
  return CPA_OK;
}

}  // extern "C"
