// Measured peaks of this GPU for the benchmark's roofline lines, next to the
// published ones: the bf16 matrix-core issue rate (v_mfma_f32_32x32x16_bf16,
// the instruction of the attention kernel, on independent accumulators) and
// the shader clock while it runs (s_memtime counts core cycles, s_memrealtime
// a constant 100 MHz). Built into libress_probe.so, which only the benchmark
// loads; it is not part of the attention library.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Every wave issues `iters` rounds of 8 independent 32x32x16 MFMAs; lane 0 of
// wave 0 of workgroup 0 records the core-clock and 100 MHz counters around
// its loop. out_sink keeps the results live.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* out_sink,
                                                        unsigned long long* clocks) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1e-3f * (threadIdx.x + e));
    b[e] = (__bf16)(1e-3f * (blockIdx.x + e));
  }
  f32x16 acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  const bool rec = blockIdx.x == 0 && threadIdx.x == 0;
  unsigned long long c0 = 0, r0 = 0;
  if (rec) {
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[t], 0, 0, 0);
  }
  if (rec) {
    clocks[0] = __builtin_amdgcn_s_memtime() - c0;
    clocks[1] = __builtin_amdgcn_s_memrealtime() - r0;
  }
  float s = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[t][r];
  out_sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

extern "C" int ress_probe_mfma(int workgroups, int iters, float* sink, unsigned long long* clocks,
                               void* stream) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(workgroups), dim3(256), 0,
                     static_cast<hipStream_t>(stream), iters, sink, clocks);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
