// Per-head Gram matrices of the output projection ("ReSS: Residual-Restoring
// Sparse Attention for 3D Vision Transformers", §4.2 Eq. 8):
//   M_h = (W_O^h)^T W_O^h,  W_O^h = columns h*D .. h*D+D-1 of W_O [d][H*D],
// so that q = e^T M_h e is the squared residual-space norm ||W_O^h e||^2 of
// Eq. 9. One workgroup per head; the head's D = 64 columns stream through
// LDS 32 rows at a time, converted to float64, and thread (ti, tj) owns
// M[ti + 16a][tj + 16b] (a, b < 4) as one fused multiply-add chain over the
// rows in ascending order, so repeated calls give identical bits.
#include "ress_internal.h"

namespace ress {
namespace {

constexpr int kD = 64;
constexpr int kRows = 32;  // rows of W_O per LDS stage

__device__ inline void load8w(const uint16_t* p, double (&v)[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = (double)__uint_as_float(u[i] << 16);
    v[2 * i + 1] = (double)__uint_as_float(u[i] & 0xFFFF0000u);
  }
}
__device__ inline void load8w(const float* p, double (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

template <typename T>
__global__ __launch_bounds__(256) void gram_kernel(const T* __restrict__ W, int d, int ldw,
                                                   double* __restrict__ M) {
  __shared__ double Ws[kRows][kD + 1];
  const int h = blockIdx.x;
  const int tid = threadIdx.x;
  const int ti = tid >> 4, tj = tid & 15;
  const int lr = tid >> 3, lc = (tid & 7) * 8;  // staging: row, first column
  double acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0;
  for (int r0 = 0; r0 < d; r0 += kRows) {
    double x[8];
    const int r = r0 + lr;
    if (r < d) {
      load8w(W + (size_t)r * ldw + (size_t)h * kD + lc, x);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.0;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) Ws[lr][lc + e] = x[e];
    __syncthreads();
    const int kn = min(kRows, d - r0);
    for (int k = 0; k < kn; ++k) {
      double av[4], bv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) av[a] = Ws[k][ti + 16 * a];
#pragma unroll
      for (int b = 0; b < 4; ++b) bv[b] = Ws[k][tj + 16 * b];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fma(av[a], bv[b], acc[a][b]);
    }
    __syncthreads();
  }
  double* Mh = M + (size_t)h * kD * kD;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) Mh[(ti + 16 * a) * kD + tj + 16 * b] = acc[a][b];
}

}  // namespace

hipError_t launch_gram(const void* w_o, int dtype, int d_model, const ress_shape& s, double* M,
                       hipStream_t st) {
  const int ldw = s.H * kD;
  if (dtype == RESS_DTYPE_BF16)
    hipLaunchKernelGGL((gram_kernel<uint16_t>), dim3(s.H), dim3(256), 0, st,
                       static_cast<const uint16_t*>(w_o), d_model, ldw, M);
  else
    hipLaunchKernelGGL((gram_kernel<float>), dim3(s.H), dim3(256), 0, st,
                       static_cast<const float*>(w_o), d_model, ldw, M);
  return hipGetLastError();
}

}  // namespace ress
