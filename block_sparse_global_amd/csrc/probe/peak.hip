// Measured peaks of this GPU for the benchmark's roofline lines, next to the
// published ones: the bf16 matrix-core issue rate (v_mfma_f32_32x32x16_bf16,
// the instruction of the attention kernel, on independent accumulators), the
// shader clock while it runs (s_memtime counts core cycles, s_memrealtime a
// constant 100 MHz), and the HBM read bandwidth (a streaming sum over a
// buffer much larger than the caches, non-temporal 16-byte loads). Built into
// libress_probe.so, which only the benchmark loads; it is not part of the
// attention library.
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

// Every thread sums the 16-byte words i, i + stride, ... of the buffer (all
// loads in flight in batches of 8); one partial per thread keeps them live.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void hbm_read_kernel(const u32x4* __restrict__ src, size_t n16,
                                                       unsigned int* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  unsigned int acc = 0;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

extern "C" int ress_probe_hbm_read(const void* src, size_t bytes, int workgroups, void* sink,
                                   void* stream) {
  hipLaunchKernelGGL(hbm_read_kernel, dim3(workgroups), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), bytes / 16,
                     static_cast<unsigned int*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
