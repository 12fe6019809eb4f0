// Mean pooling per block ("ReSS: Residual-Restoring Sparse Attention for 3D
// Vision Transformers", §3 step (1)): xpool[h][b] = mean of the valid tokens
// of block b. HBM-streaming kernel: every input byte is read once with
// 16-byte loads, accumulated in float64 and reduced in a fixed order, so the
// result does not depend on scheduling.
#include "ress_internal.h"

namespace ress {
namespace {

constexpr int kThreads = 256;
constexpr int kD = 64;

// 8 consecutive elements of one token row, widened exactly to float64.
// Every input byte is read once, so the loads are non-temporal (streamed
// past the caches' retention policy).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ inline void load8(const uint16_t* p, double (&v)[8]) {
  const u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = (double)__uint_as_float(u[i] << 16);
    v[2 * i + 1] = (double)__uint_as_float(u[i] & 0xFFFF0000u);
  }
}

__device__ inline void load8(const float* p, double (&v)[8]) {
  const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// One workgroup per (block, head, tensor): blockIdx.z picks one of up to
// three tensors pooled in the same launch (the grid covers the largest block
// count; workgroups past a tensor's own count return). Thread t reads dims
// 8*(t%8)..+7 of the rows lo + t/8, lo + t/8 + 32, ...; the 32 row groups
// are then summed per dim in ascending order.
template <typename T, int BLK>
__global__ __launch_bounds__(kThreads) void pool_kernel(PoolJobs jobs, int N, int N_pad) {
  const PoolJob job = jobs.job[blockIdx.z];
  const int n = job.nb;
  const int b = blockIdx.x;
  if (b >= n) return;
  const T* __restrict__ x = static_cast<const T*>(job.x);
  double* __restrict__ out = job.out;
  const int h = blockIdx.y;
  const int t = threadIdx.x;
  const int chunk = t & 7;
  const int rg = t >> 3;  // 0..31
  const int lo = b * BLK;
  const int hi = min(lo + BLK, N);
  const T* base = x + (size_t)h * N_pad * kD + chunk * 8;

  double acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.0;

  constexpr int kIters = BLK / 32;
  double v[kIters][8];
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int r = lo + rg + 32 * it;
    if (r < hi) {
      load8(base + (size_t)r * kD, v[it]);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) v[it][k] = 0.0;
    }
  }
#pragma unroll
  for (int it = 0; it < kIters; ++it)
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] += v[it][k];

  __shared__ double red[32][kD + 1];
#pragma unroll
  for (int k = 0; k < 8; ++k) red[rg][chunk * 8 + k] = acc[k];
  __syncthreads();
  if (t < kD) {
    double s = 0.0;
#pragma unroll 8
    for (int g = 0; g < 32; ++g) s += red[g][t];
    out[((size_t)h * n + b) * kD + t] = s / (double)(hi - lo);
  }
}

template <typename T>
hipError_t launch_t(const PoolJobs& jobs, const ress_shape& s, int blk, hipStream_t st) {
  int nb_max = 0;
  for (int a = 0; a < jobs.count; ++a) nb_max = max(nb_max, jobs.job[a].nb);
  dim3 grid(nb_max, s.H, jobs.count);
  if (blk == 128)
    hipLaunchKernelGGL((pool_kernel<T, 128>), grid, dim3(kThreads), 0, st, jobs, s.N, s.N_pad);
  else
    hipLaunchKernelGGL((pool_kernel<T, 64>), grid, dim3(kThreads), 0, st, jobs, s.N, s.N_pad);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_block_pool(const PoolJobs& jobs, int dtype, const ress_shape& s, int blk,
                             hipStream_t st) {
  if (jobs.count <= 0) return hipSuccess;
  if (dtype == RESS_DTYPE_BF16) return launch_t<uint16_t>(jobs, s, blk, st);
  return launch_t<float>(jobs, s, blk, st);
}

}  // namespace ress
