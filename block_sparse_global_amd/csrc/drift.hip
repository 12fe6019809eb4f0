// Realised residual drift of a sparse attention output ("ReSS: Residual-
// Restoring Sparse Attention for 3D Vision Transformers", §4.2 Eq. 6 and 9
// at token level): for every (head h, query block i),
//   drift[h][i] = mean over the valid tokens t of block i of
//                 e_t^T M_h e_t,  e_t = out_sparse[h][t] - out_dense[h][t],
// i.e. the mean squared change ||W_O^h e_t||^2 that sparsification leaves in
// the residual stream when M_h = (W_O^h)^T W_O^h (||e_t||^2 when M is NULL).
// One workgroup per (query block, head): M_h in LDS, one wave per token at a
// time (lane d holds e_d and forms (M e)_d from the symmetric M's column d);
// each lane sums its dim's terms over the wave's tokens and the wave reduces
// once. Without M, each thread takes four consecutive dims of every 16th
// token instead. Fixed-order sums, so repeated calls give identical bits.
#include "ress_internal.h"

namespace ress {
namespace {

constexpr int kD = 64;

__device__ inline double elem(const uint16_t* p, size_t i) {
  return (double)__uint_as_float((uint32_t)p[i] << 16);
}
__device__ inline double elem(const float* p, size_t i) { return (double)p[i]; }

template <typename T>
__global__ __launch_bounds__(256) void drift_kernel(const T* __restrict__ os,
                                                    const T* __restrict__ od,
                                                    const double* __restrict__ M, int B, int N,
                                                    int N_pad, double* __restrict__ drift) {
  __shared__ double Ms[kD][kD];
  __shared__ double ev[4][kD];
  __shared__ double part[4];
  const int i = blockIdx.x, h = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, d = tid & 63;
  if (M != nullptr)
    for (int e = tid; e < kD * kD; e += 256) Ms[e / kD][e % kD] = M[(size_t)h * kD * kD + e];
  __syncthreads();
  const int t0 = i * B, t1 = min(t0 + B, N);
  double accl = 0.0;  // this lane's terms over its tokens, in order
  if (M == nullptr) {
    // ||e_t||^2 only: thread tid takes dims 4 (tid % 16) .. + 3 of tokens
    // t0 + tid / 16, + 16, ... (one load instruction covers four tokens)
    const int tl = tid >> 4, d4 = 4 * (tid & 15);
    for (int t = t0 + tl; t < t1; t += 16) {
      const size_t off = ((size_t)h * N_pad + t) * kD + d4;
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const double e = elem(os, off + e4) - elem(od, off + e4);
        accl = fma(e, e, accl);
      }
    }
  }
  for (int t = t0 + w; M != nullptr && t < t1; t += 4) {
    const size_t off = ((size_t)h * N_pad + t) * kD + d;
    const double e = elem(os, off) - elem(od, off);
    double me = e;
    if (M != nullptr) {
      ev[w][d] = e;
      wave_lds_sync();
      me = 0.0;
#pragma unroll 8
      for (int f = 0; f < kD; ++f) me = fma(Ms[f][d], ev[w][f], me);
      wave_lds_sync();
    }
    accl = fma(e, me, accl);
  }
  const double acc = wave_sum64(accl);  // one reduction per wave
  if (d == 0) part[w] = acc;
  __syncthreads();
  if (tid == 0) {
    const double s = (part[0] + part[1]) + (part[2] + part[3]);
    drift[(size_t)h * gridDim.x + i] = t1 > t0 ? s / (double)(t1 - t0) : 0.0;
  }
}

}  // namespace

hipError_t launch_residual_drift(const void* os, const void* od, int dtype, const double* M,
                                 const ress_shape& s, double* drift, hipStream_t st) {
  const dim3 grid(n_qblocks(s), s.H);
  if (dtype == RESS_DTYPE_BF16)
    hipLaunchKernelGGL((drift_kernel<uint16_t>), grid, dim3(256), 0, st,
                       static_cast<const uint16_t*>(os), static_cast<const uint16_t*>(od), M,
                       s.B, s.N, s.N_pad, drift);
  else
    hipLaunchKernelGGL((drift_kernel<float>), grid, dim3(256), 0, st,
                       static_cast<const float*>(os), static_cast<const float*>(od), M, s.B, s.N,
                       s.N_pad, drift);
  return hipGetLastError();
}

}  // namespace ress
