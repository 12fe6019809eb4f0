// Pooled block map and block scores, in float64 on the vector ALUs.
//
// Map ("ReSS: Residual-Restoring Sparse Attention for 3D Vision
// Transformers", §4.1): P_ij = softmax over every key block j of
// scale * qpool_i . kpool_j.
// Drift key (same page, §4.2, Eq. 1, 5-9): vout_i = sum_j P_ij V_j,
// q_ij = vout^T M vout - 2 vout^T M V_j + V_j^T M V_j (the Eq. 9 expansion,
// so no per-pair D-vector is formed), key = P sqrt(max(q,0)) / max(1-P, eps).
//
// Maps are [H][n_q][n_k] (query-block rows, key-block columns; the two
// counts differ when key blocks are smaller than query blocks).
// The three n_q x n_k x 64 products (logits, vout = P V, (M vout) . V_j) run
// as float64 matrix-core products (v_mfma_f64_16x16x4_f64) with their
// elementwise steps in the epilogues; the row softmax is one wave per row.
// Every output element is a fixed sequence of fused multiply-adds and every
// reduction has a fixed order (no atomics), so repeated calls give
// identical bits.
#include "ress_internal.h"
#include "tile_f64.h"

namespace ress {
namespace {

constexpr int kD = 64;
constexpr int kThreads = 256;

__device__ inline double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ inline double wave_max(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o, 64));
  return v;
}

// 8 consecutive float64 of a row (two 16-byte loads per pair).
__device__ inline void load8d(const double* p, double (&x)[8]) {
  const double2* src = reinterpret_cast<const double2*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double2 v = src[e];
    x[2 * e] = v.x;
    x[2 * e + 1] = v.y;
  }
}

// Logits scale * qpool_i . kpool_j of one 64 x 64 tile, written into P.
// Within 128 VGPRs (four workgroups per CU, as its LDS allows): 98 -> 92 us
// per call against the uncapped 132 VGPRs, the same bits.
__global__ __launch_bounds__(kThreads, 4) void logits_kernel(
    const double* __restrict__ qpool, const double* __restrict__ kpool, double scale, int nq,
    int nk, double* __restrict__ P) {
  __shared__ TileF64Smem sm;
  const TileIdx tid3 = xcd_tile_order();
  const int h = tid3.z;
  const int j0 = tid3.x * kTF, i0 = tid3.y * kTF;
  const double* qh = qpool + (size_t)h * nq * kD;
  const double* kh = kpool + (size_t)h * nk * kD;
  f64x4 acc[2][2];
  mfma_tile_f64(
      [&](int r, int d0, double (&x)[8]) { load8d(qh + (size_t)min(i0 + r, nq - 1) * kD + d0, x); },
      [&](int r, int d0, double (&x)[8]) { load8d(kh + (size_t)min(j0 + r, nk - 1) * kD + d0, x); },
      sm, acc);
  const TileF64Map mp;
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + mp.row_of(tr, r);
#pragma unroll
      for (int tc = 0; tc < 2; ++tc) {
        const int j = j0 + mp.col_of(tc);
        if (i < nq && j < nk) P[((size_t)h * nq + i) * nk + j] = scale * acc[tr][tc][r];
      }
    }
}

// Row softmax in place, one wave per row (row i of head h is workgroup
// (i, h)) of n values: max, exponentials and their sum, normalisation.
// KPL > 0: the row (KPL >= ceil(n / 64) values per lane) is held in
// registers; KPL = 0: in LDS (8 n bytes).
template <int KPL>
__global__ __launch_bounds__(64) void softmax_rows_kernel(int n, double* __restrict__ P) {
  extern __shared__ double rowbuf[];
  const int lane = threadIdx.x;
  double* Prow = P + ((size_t)blockIdx.y * gridDim.x + blockIdx.x) * n;
  constexpr int kK = KPL > 0 ? KPL : 1;
  double v[kK];
  double mx = -INFINITY;
  if constexpr (KPL > 0) {
#pragma unroll
    for (int k = 0; k < KPL; ++k) {
      const int j = lane + 64 * k;
      v[k] = j < n ? Prow[j] : -INFINITY;
      mx = fmax(mx, v[k]);
    }
  } else {
    for (int j = lane; j < n; j += 64) {
      const double x = Prow[j];
      rowbuf[j] = x;
      mx = fmax(mx, x);
    }
  }
  mx = wave_max(mx);
  double sum = 0.0;
  if constexpr (KPL > 0) {
#pragma unroll
    for (int k = 0; k < KPL; ++k) {
      const int j = lane + 64 * k;
      v[k] = j < n ? exp(v[k] - mx) : 0.0;
      sum += v[k];
    }
  } else {
    for (int j = lane; j < n; j += 64) {
      const double e = exp(rowbuf[j] - mx);
      rowbuf[j] = e;
      sum += e;
    }
  }
  sum = wave_sum(sum);
  if constexpr (KPL > 0) {
#pragma unroll
    for (int k = 0; k < KPL; ++k) {
      const int j = lane + 64 * k;
      if (j < n) Prow[j] = v[k] / sum;
    }
  } else {
    for (int j = lane; j < n; j += 64) Prow[j] = rowbuf[j] / sum;
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

// vout = P V for 32 rows (all 64 dims) per workgroup on the matrix cores:
// wave w owns rows 16*(w>>1) .. +15 and dims 32*(w&1) .. +31 (two 16 x 16
// tiles); the key blocks stream through LDS 64 at a time, 4 per MFMA step.
// Row padding: 66 doubles for P (a half-wave reads 16 rows x 2 columns) and
// 80 for V (2 rows x 16 columns), so both reads are free of bank conflicts.
__global__ __launch_bounds__(kThreads) void fill_zero_kernel(double* __restrict__ p, size_t n) {
  const size_t e = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (e < n) p[e] = 0.0;
}

constexpr int kVR = 32;  // rows per workgroup
constexpr int kVJ = 32;  // key blocks per LDS stage
constexpr int kVParts = 2;  // key-block halves per row tile (grid z)

__global__ __launch_bounds__(kThreads) void vout_kernel(
    const double* __restrict__ P, const double* __restrict__ vpool, int nq, int nk,
    double* __restrict__ vout) {
  __shared__ double Ps[kVR][kVJ + 2];
  __shared__ double Vs[kVJ][kD + 16];
  const TileIdx tid3 = xcd_tile_order();  // row tiles of a head together
  const int h = tid3.y;
  const int i0 = tid3.x * kVR;
  // this workgroup's share of the key-block chunks
  const int nch = (nk + kVJ - 1) / kVJ;
  const int c_lo = tid3.z * nch / kVParts, c_hi = (tid3.z + 1) * nch / kVParts;
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int rt = 16 * (w >> 1), dt = 32 * (w & 1);
  const double* Ph = P + (size_t)h * nq * nk;
  const double* Vh = vpool + (size_t)h * nk * kD;
  f64x4 acc[2] = {f64x4{0.0, 0.0, 0.0, 0.0}, f64x4{0.0, 0.0, 0.0, 0.0}};
  // chunks of 64 key blocks: P 32 rows x 64 blocks (8 per thread), V 64
  // blocks x 64 dims (16 per thread); the next chunk's loads are in flight
  // in registers while the current chunk's products run
  constexpr int kPE = kVR * kVJ / kThreads, kVE = kVJ * kD / (2 * kThreads);
  double pr[kPE], vx[kVE], vy[kVE];
#define RESS_VOUT_LOAD_CHUNK(JC)                                               \
  do {                                                                         \
    _Pragma("unroll") for (int e = 0; e < kPE; ++e) {                          \
      const int idx = tid + e * kThreads;                                      \
      const int i = min(i0 + idx / kVJ, nq - 1), j = (JC) + idx % kVJ;         \
      const double x = Ph[(size_t)i * nk + min(j, nk - 1)];                    \
      pr[e] = j < nk ? x : 0.0;                                                \
    }                                                                          \
    _Pragma("unroll") for (int e = 0; e < kVE; ++e) {                          \
      const int idx = tid + e * kThreads;                                      \
      const int j = min((JC) + (idx >> 5), nk - 1);                            \
      const double2 v2 = reinterpret_cast<const double2*>(Vh + (size_t)j * kD)[idx & 31]; \
      vx[e] = v2.x;                                                            \
      vy[e] = v2.y;                                                            \
    }                                                                          \
  } while (0)
  RESS_VOUT_LOAD_CHUNK(c_lo * kVJ);
  for (int jc = c_lo * kVJ; jc < c_hi * kVJ; jc += kVJ) {
#pragma unroll
    for (int e = 0; e < kPE; ++e) {
      const int idx = tid + e * kThreads;
      Ps[idx / kVJ][idx % kVJ] = pr[e];
    }
#pragma unroll
    for (int e = 0; e < kVE; ++e) {
      const int idx = tid + e * kThreads;
      *reinterpret_cast<double2*>(&Vs[idx >> 5][2 * (idx & 31)]) = double2{vx[e], vy[e]};
    }
    __syncthreads();
    // (after the last chunk this reloads valid clamped rows, unused)
    RESS_VOUT_LOAD_CHUNK(jc + kVJ);
#pragma unroll 4
    for (int s4 = 0; s4 < kVJ / 4; ++s4) {
      const int k = 4 * s4 + (l >> 4);
      const double a = Ps[rt + (l & 15)][k];
#pragma unroll
      for (int t = 0; t < 2; ++t)
        acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, Vs[k][dt + 16 * t + (l & 15)], acc[t],
                                                      0, 0, 0);
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = i0 + rt + (l >> 4) + 4 * r;
    // the two halves' sums add into the zeroed output; 0 + a + b is the
    // same in either order, so the result does not depend on scheduling
    if (i < nq)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        atomicAdd(&vout[((size_t)h * nq + i) * kD + dt + 16 * t + (l & 15)], acc[t][r]);
  }
}
#undef RESS_VOUT_LOAD_CHUNK

// Drift key of one 64 x 64 tile: w_i = M vout_i (vout_i when M is NULL) is
// formed while staging, a_i = vout_i . w_i, then per (i, j)
// q = a_i - 2 w_i . V_j + vmv_j and key = P sqrt(max(q, 0)) / max(1 - P, eps).
__global__ __launch_bounds__(kThreads) void key_kernel(
    const double* __restrict__ P, const double* __restrict__ vpool,
    const double* __restrict__ M, const double* __restrict__ vmv,
    const double* __restrict__ vout, int nq, int nk, double eps, double* __restrict__ key) {
  __shared__ TileF64Smem sm;
  __shared__ double apart[2][kTF][4];
  const TileIdx tid3 = xcd_tile_order();
  const int h = tid3.z;
  const int j0 = tid3.x * kTF, i0 = tid3.y * kTF;
  const double* voh = vout + (size_t)h * nq * kD;
  const double* vph = vpool + (size_t)h * nk * kD;
  const double* Mh = M ? M + (size_t)h * kD * kD : nullptr;
  // stage w_i dims d0 .. d0+7 of row r; the partial vout . w over those
  // dims goes to apart[half][r][thread's quarter]
  auto stage_w = [&](int r, int d0, double (&x)[8]) {
    const double* vr = voh + (size_t)min(i0 + r, nq - 1) * kD;
    double vo8[8];
    load8d(vr + d0, vo8);
    if (Mh == nullptr) {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = vo8[e];
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double* Mrow = Mh + (size_t)(d0 + e) * kD;
        double wv = 0.0;
#pragma unroll 8
        for (int f = 0; f < kD; ++f) wv = fma(Mrow[f], vr[f], wv);
        x[e] = wv;
      }
    }
    double pa = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) pa = fma(vo8[e], x[e], pa);
    apart[d0 >= kTFHalf][r][(d0 % kTFHalf) / 8] = pa;
  };
  f64x4 acc[2][2];
  mfma_tile_f64(
      stage_w,
      [&](int r, int d0, double (&x)[8]) { load8d(vph + (size_t)min(j0 + r, nk - 1) * kD + d0, x); },
      sm, acc);
  const TileF64Map mp;
#pragma unroll
  for (int tr = 0; tr < 2; ++tr)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rl = mp.row_of(tr, r);
      const int i = i0 + rl;
      double ai = 0.0;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) ai += apart[hh][rl][q4];
#pragma unroll
      for (int tc = 0; tc < 2; ++tc) {
        const int j = j0 + mp.col_of(tc);
        if (i < nq && j < nk) {
          const size_t off = ((size_t)h * nq + i) * nk + j;
          const double q = fmax(ai - 2.0 * acc[tr][tc][r] + vmv[(size_t)h * nk + j], 0.0);
          const double p = P[off];
          key[off] = p * sqrt(q) / fmax(1.0 - p, eps);
        }
      }
    }
}

}  // namespace

hipError_t launch_block_map(const double* qpool, const double* kpool,
                            const ress_shape& s, double scale, double* P,
                            hipStream_t st) {
  const int nq = n_qblocks(s), nk = n_kblocks(s);
  const dim3 tiles((nk + kTF - 1) / kTF, (nq + kTF - 1) / kTF, s.H);
  hipLaunchKernelGGL(logits_kernel, tiles, dim3(kThreads), 0, st, qpool, kpool, scale, nq, nk,
                     P);
  const dim3 rows(nq, s.H);
  if (nk <= 17 * 64)
    hipLaunchKernelGGL((softmax_rows_kernel<17>), rows, dim3(64), 0, st, nk, P);
  else if (nk <= 34 * 64)
    hipLaunchKernelGGL((softmax_rows_kernel<34>), rows, dim3(64), 0, st, nk, P);
  else
    hipLaunchKernelGGL((softmax_rows_kernel<0>), rows, dim3(64), (size_t)nk * 8, st, nk, P);
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
  const int n = n_kblocks(s);
  const int per = kThreads / 64;
  dim3 grid((n + per - 1) / per, s.H);
  hipLaunchKernelGGL(vmv_kernel, grid, dim3(kThreads), 0, st, vpool, M, n,
                     vmv);
  return hipGetLastError();
}

hipError_t launch_drift(const double* P, const double* vpool, const double* M,
                        const double* vmv, const ress_shape& s, double eps,
                        double* key, double* vout, hipStream_t st) {
  const int nq = n_qblocks(s), nk = n_kblocks(s);
  const size_t nv = (size_t)s.H * nq * kD;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((nv + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, vout, nv);
  hipLaunchKernelGGL(vout_kernel, dim3((nq + kVR - 1) / kVR, s.H, kVParts), dim3(kThreads), 0,
                     st, P, vpool, nq, nk, vout);
  const dim3 tiles((nk + kTF - 1) / kTF, (nq + kTF - 1) / kTF, s.H);
  hipLaunchKernelGGL(key_kernel, tiles, dim3(kThreads), 0, st, P, vpool, M, vmv, vout, nq, nk,
                     eps, key);
  return hipGetLastError();
}

}  // namespace ress
