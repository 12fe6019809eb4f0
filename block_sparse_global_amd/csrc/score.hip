// Pooled block map and block scores, in float64 on the vector ALUs.
//
// Map ("ReSS: Residual-Restoring Sparse Attention for 3D Vision
// Transformers", §4.1): P_ij = softmax over every key block j of
// scale * qpool_i . kpool_j.
// Drift key (same page, §4.2, Eq. 1, 5-9): vout_i = sum_j P_ij V_j,
// q_ij = vout^T M vout - 2 vout^T M V_j + V_j^T M V_j (the Eq. 9 expansion,
// so no per-pair D-vector is formed), key = P sqrt(max(q,0)) / max(1-P, eps).
//
// All reductions run in a fixed order (no atomics), so repeated calls give
// identical bits.
#include "ress_internal.h"

namespace ress {
namespace {

constexpr int kD = 64;
constexpr int kThreads = 256;
constexpr int kRows = 8;    // query-block rows per workgroup
constexpr int kJTile = 32;  // key blocks staged per LDS tile

__device__ inline double half_wave_max(double v) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o, 32));
  return v;
}

__device__ inline double half_wave_sum(double v) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, 32);
  return v;
}

__device__ inline double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Logits, row max, exponentials and normalisation of kRows map rows. Thread
// t owns row r = t / 32 and key blocks j = jj, jj + 32, ... (jj = t % 32);
// the P row itself holds the intermediate values, and each element is only
// ever touched by its owning thread.
__global__ __launch_bounds__(kThreads) void map_kernel(
    const double* __restrict__ qpool, const double* __restrict__ kpool,
    double scale, int n, double* __restrict__ P) {
  const int h = blockIdx.y;
  const int i0 = blockIdx.x * kRows;
  const int t = threadIdx.x;
  const int r = t >> 5;
  const int jj = t & 31;
  const int i = i0 + r;

  __shared__ double qs[kRows][kD];
  __shared__ double kt[kD][kJTile + 1];

  for (int e = t; e < kRows * kD; e += kThreads) {
    const int rr = e / kD, d = e % kD;
    qs[rr][d] = (i0 + rr < n) ? qpool[((size_t)h * n + i0 + rr) * kD + d] : 0.0;
  }
  double* Prow = P + ((size_t)h * n + (i < n ? i : 0)) * n;
  const double* kh = kpool + (size_t)h * n * kD;

  double mx = -INFINITY;
  for (int j0 = 0; j0 < n; j0 += kJTile) {
    __syncthreads();
    // stage 32 key blocks transposed: thread loads 8 dims of one key block
    {
      const int kk = t >> 3, d0 = (t & 7) * 8;
      const int j = j0 + kk;
#pragma unroll
      for (int d = 0; d < 8; ++d)
        kt[d0 + d][kk] = (j < n) ? kh[(size_t)j * kD + d0 + d] : 0.0;
    }
    __syncthreads();
    const int j = j0 + jj;
    if (i < n && j < n) {
      double dot = 0.0;
#pragma unroll 16
      for (int d = 0; d < kD; ++d) dot = fma(qs[r][d], kt[d][jj], dot);
      const double l = scale * dot;
      Prow[j] = l;
      mx = fmax(mx, l);
    }
  }
  mx = half_wave_max(mx);
  double sum = 0.0;
  if (i < n) {
    for (int j = jj; j < n; j += kJTile) {
      const double e = exp(Prow[j] - mx);
      Prow[j] = e;
      sum += e;
    }
  }
  sum = half_wave_sum(sum);
  if (i < n) {
    for (int j = jj; j < n; j += kJTile) Prow[j] = Prow[j] / sum;
  }
}

__global__ __launch_bounds__(kThreads) void copy_kernel(
    const double* __restrict__ src, double* __restrict__ dst, size_t count) {
  for (size_t e = (size_t)blockIdx.x * kThreads + threadIdx.x; e < count;
       e += (size_t)gridDim.x * kThreads)
    dst[e] = src[e];
}

// vmv[h][j] = V_j^T M_h V_j (V_j^T V_j when M is NULL): one wave per block.
__global__ __launch_bounds__(kThreads) void vmv_kernel(
    const double* __restrict__ vpool, const double* __restrict__ M, int n,
    double* __restrict__ vmv) {
  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  __shared__ double vs[kThreads / 64][kD];
  const int w = threadIdx.x >> 6;
  const double vj = (j < n) ? vpool[((size_t)h * n + j) * kD + lane] : 0.0;
  vs[w][lane] = vj;
  __syncthreads();
  double mv = vj;
  if (M != nullptr) {
    const double* Mrow = M + ((size_t)h * kD + lane) * kD;
    mv = 0.0;
#pragma unroll 16
    for (int e = 0; e < kD; ++e) mv = fma(Mrow[e], vs[w][e], mv);
  }
  const double s = wave_sum(vj * mv);
  if (j < n && lane == 0) vmv[(size_t)h * n + j] = s;
}

// Drift key of kRows map rows. Phase 1: vout = P V (thread owns dim t%64 of
// rows t/64 and t/64 + 4). Phase 2: w = M vout and a = vout . w. Phase 3:
// for every key block, q = a - 2 w . V_j + vmv_j and the key.
__global__ __launch_bounds__(kThreads) void drift_kernel(
    const double* __restrict__ P, const double* __restrict__ vpool,
    const double* __restrict__ M, const double* __restrict__ vmv, int n,
    double eps, double* __restrict__ key, double* __restrict__ vout) {
  const int h = blockIdx.y;
  const int i0 = blockIdx.x * kRows;
  const int t = threadIdx.x;
  const int d = t & 63;
  const int rg = t >> 6;  // 0..3

  __shared__ double ps[kRows][kJTile];
  __shared__ double vt[kJTile][kD + 1];
  __shared__ double vo[kRows][kD];
  __shared__ double ws[kRows][kD];
  __shared__ double as[kRows];

  const double* Ph = P + (size_t)h * n * n;
  const double* Vh = vpool + (size_t)h * n * kD;

  // ---- phase 1: vout rows
  double acc0 = 0.0, acc1 = 0.0;
  for (int j0 = 0; j0 < n; j0 += kJTile) {
    __syncthreads();
    {
      const int rr = t >> 5, jj = t & 31;
      const int i = i0 + rr, j = j0 + jj;
      ps[rr][jj] = (i < n && j < n) ? Ph[(size_t)i * n + j] : 0.0;
    }
    for (int e = t; e < kJTile * kD; e += kThreads) {
      const int jj = e >> 6, dd = e & 63;
      const int j = j0 + jj;
      vt[jj][dd] = (j < n) ? Vh[(size_t)j * kD + dd] : 0.0;
    }
    __syncthreads();
    const int jmax = min(kJTile, n - j0);
    for (int jj = 0; jj < jmax; ++jj) {
      acc0 = fma(ps[rg][jj], vt[jj][d], acc0);
      acc1 = fma(ps[rg + 4][jj], vt[jj][d], acc1);
    }
  }
  vo[rg][d] = acc0;
  vo[rg + 4][d] = acc1;
  if (i0 + rg < n) vout[((size_t)h * n + i0 + rg) * kD + d] = acc0;
  if (i0 + rg + 4 < n) vout[((size_t)h * n + i0 + rg + 4) * kD + d] = acc1;
  __syncthreads();

  // ---- phase 2: w = M vout, a = vout . w
  {
    double w0 = vo[rg][d], w1 = vo[rg + 4][d];
    if (M != nullptr) {
      const double* Mrow = M + ((size_t)h * kD + d) * kD;
      w0 = 0.0;
      w1 = 0.0;
#pragma unroll 8
      for (int e = 0; e < kD; ++e) {
        const double m = Mrow[e];
        w0 = fma(m, vo[rg][e], w0);
        w1 = fma(m, vo[rg + 4][e], w1);
      }
    }
    ws[rg][d] = w0;
    ws[rg + 4][d] = w1;
    const double a0 = wave_sum(vo[rg][d] * w0);
    const double a1 = wave_sum(vo[rg + 4][d] * w1);
    if (d == 0) {
      as[rg] = a0;
      as[rg + 4] = a1;
    }
  }

  // ---- phase 3: keys. Thread owns row t/32 and key blocks j0 + t%32.
  const int r = t >> 5;
  const int jj = t & 31;
  const int i = i0 + r;
  for (int j0 = 0; j0 < n; j0 += kJTile) {
    __syncthreads();
    for (int e = t; e < kJTile * kD; e += kThreads) {
      const int kk = e >> 6, dd = e & 63;
      const int j = j0 + kk;
      vt[kk][dd] = (j < n) ? Vh[(size_t)j * kD + dd] : 0.0;
    }
    __syncthreads();
    const int j = j0 + jj;
    if (i < n && j < n) {
      double wv = 0.0;
#pragma unroll 16
      for (int e = 0; e < kD; ++e) wv = fma(ws[r][e], vt[jj][e], wv);
      double q = as[r] - 2.0 * wv + vmv[(size_t)h * n + j];
      q = fmax(q, 0.0);
      const double p = Ph[(size_t)i * n + j];
      key[((size_t)h * n + i) * n + j] = p * sqrt(q) / fmax(1.0 - p, eps);
    }
  }
}

}  // namespace

hipError_t launch_block_map(const double* qpool, const double* kpool,
                            const ress_shape& s, double scale, double* P,
                            hipStream_t st) {
  const int n = s.N_pad / s.B;
  dim3 grid((n + kRows - 1) / kRows, s.H);
  hipLaunchKernelGGL(map_kernel, grid, dim3(kThreads), 0, st, qpool, kpool,
                     scale, n, P);
  return hipGetLastError();
}

hipError_t launch_copy(const double* src, double* dst, size_t count,
                       hipStream_t st) {
  size_t blocks = (count + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                     st, src, dst, count);
  return hipGetLastError();
}

hipError_t launch_vmv(const double* vpool, const double* M,
                      const ress_shape& s, double* vmv, hipStream_t st) {
  const int n = s.N_pad / s.B;
  const int per = kThreads / 64;
  dim3 grid((n + per - 1) / per, s.H);
  hipLaunchKernelGGL(vmv_kernel, grid, dim3(kThreads), 0, st, vpool, M, n,
                     vmv);
  return hipGetLastError();
}

hipError_t launch_drift(const double* P, const double* vpool, const double* M,
                        const double* vmv, const ress_shape& s, double eps,
                        double* key, double* vout, hipStream_t st) {
  const int n = s.N_pad / s.B;
  dim3 grid((n + kRows - 1) / kRows, s.H);
  hipLaunchKernelGGL(drift_kernel, grid, dim3(kThreads), 0, st, P, vpool, M,
                     vmv, n, eps, key, vout);
  return hipGetLastError();
}

}  // namespace ress
