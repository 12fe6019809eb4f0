// Steps of the fused selection on a tile of R consecutive query-block rows
// of one head held in LDS ("ReSS: Residual-Restoring Sparse Attention for 3D
// Vision Transformers", §3 steps (1)-(2), §4.1-§4.2 Eq. 1-9), shared by the
// fused selection kernel and the pooled-input form of the fused
// refinement. Every step is run by all R waves of the workgroup (one wave
// per row, wave w = row w of the tile); a row buffer holds R x ns doubles
// (ns = row_stride(n)).
#pragma once

#include "refine_common.h"
#include "tile_f64.h"

namespace ress {

__host__ __device__ inline int row_stride(int n) { return ((n + 3) & ~3) + 4; }  // doubles

// 1. logits l_rj = scale * qpool_r . kpool_j of the R rows against every key
// block, on the float64 matrix cores (v_mfma_f64_16x16x4f64: the rows
// against 16 key blocks per instruction group, the waves taking the groups
// in turn; with R = 8 the upper half of each row group repeats row 7).
template <int R>
__device__ inline void fused_logits(const double* __restrict__ qh,
                                    const double* __restrict__ kh, int nq, int n, int i0,
                                    double scale, double* rows, int ns) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int ngroups = (n + 15) >> 4;
  // A operand: row l16 (clamped to a valid row), dims 4s + q4
  double qa[16];
  const double* qr = qh + (size_t)min(i0 + min(l16, R - 1), nq - 1) * kD;
#pragma unroll
  for (int s = 0; s < 16; ++s) qa[s] = qr[4 * s + q4];
  for (int g = w; g < ngroups; g += R) {
    const double* kr = kh + (size_t)min(16 * g + l16, n - 1) * kD;
    f64x4 acc = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int s = 0; s < 16; ++s)
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(qa[s], kr[4 * s + q4], acc, 0, 0, 0);
    // element e: row q4 + 4e, key block 16 g + l16
    const int j = 16 * g + l16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = q4 + 4 * e;
      if (r < R && j < n) rows[r * ns + j] = scale * acc[e];
    }
  }
}

// 2. softmax of the wave's row over all j (the map P, normalised over every
// key block, §4.1), in place; the row padding up to ns holds 0.
template <int KPL>
__device__ inline void fused_softmax(double* myrow, int n, int ns) {
  const int lane = threadIdx.x & 63;
  double v[KPL];
  double mx = -INFINITY;
#pragma unroll
  for (int k = 0; k < KPL; ++k) {
    const int j = lane + 64 * k;
    v[k] = j < n ? myrow[j] : -INFINITY;
    mx = fmax(mx, v[k]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, 64));
  double sum = 0.0;
#pragma unroll
  for (int k = 0; k < KPL; ++k) {
    const int j = lane + 64 * k;
    v[k] = j < n ? exp(v[k] - mx) : 0.0;
    sum += v[k];
  }
  sum = wave_sum64(sum);
#pragma unroll
  for (int k = 0; k < KPL; ++k) {
    const int j = lane + 64 * k;
    if (j < ns) myrow[j] = j < n ? v[k] / sum : 0.0;  // P, zero past the row's end
  }
}

// 3a-3b. vout_r = sum_j P_rj V_j (Eq. 1) on the matrix cores, then
// w_r = M vout_r and a_r = vout_r . w_r. Wave w takes dims 16 (w & 3) .. +15
// of the tile and one of R / 4 parts of the key blocks (contiguous runs of
// 4-block steps); A = P (rows l16, blocks 4t + q4), B = V (blocks 4t + q4,
// dims 16 dg + l16). The partial sums go to part [2][R][64] and are added
// in a fixed order ((p0 + p2) + (p1 + p3), or p0 + p1 with two parts).
// Outputs: wv [R][64] (may alias part), av [R], and vout itself in vo
// [R][64] when vo is not null. Contains workgroup barriers.
template <int R>
__device__ inline void fused_vout(const double* rows, int ns, int n,
                                  const double* __restrict__ vh, const double* __restrict__ Mh,
                                  double* part, double* vo, double* wv, double* av) {
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int dg = w & 3, kq = w >> 2;
  constexpr int kParts = R / 4;
  const int steps = (n + 3) >> 2;
  const int t0 = kq * steps / kParts, t1 = (kq + 1) * steps / kParts;
  f64x4 acc = {0.0, 0.0, 0.0, 0.0};
  const double* prow = rows + min(l16, R - 1) * ns;
  for (int t = t0; t < t1; ++t) {
    const int j = 4 * t + q4;  // P is zero for j >= n (row padding)
    const double a = l16 < R ? prow[j] : 0.0;
    const double b = vh[(size_t)min(j, n - 1) * kD + 16 * dg + l16];
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc, 0, 0, 0);
  }
  // parts 0 and 1 store, parts 2 and 3 add
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if ((kq >> 1) == half) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = q4 + 4 * e;
        if (r < R) {
          double* dst = part + ((kq & 1) * R + r) * kD + 16 * dg + l16;
          *dst = half == 0 ? acc[e] : *dst + acc[e];
        }
      }
    }
    __syncthreads();
  }
  // per row: vout, w = M vout, a = vout . w
  const double vout = part[w * kD + lane] + part[(R + w) * kD + lane];
  __syncthreads();  // every row has read its partial sums
  if (vo != nullptr) vo[w * kD + lane] = vout;
  wv[w * kD + lane] = vout;
  wave_lds_sync();
  double x = vout;
  if (Mh != nullptr) {
    const double* Mrow = Mh + (size_t)lane * kD;
    x = 0.0;
#pragma unroll 8
    for (int e = 0; e < kD; ++e) x = fma(Mrow[e], wv[w * kD + e], x);
  }
  const double a = wave_sum64(vout * x);
  wave_lds_sync();
  wv[w * kD + lane] = x;
  if (lane == 0) av[w] = a;
}

// The drift key from P_rj and c_rj = w_r . V_j: q = a_r - 2 c_rj + vmv_j,
// the Eq. 9 expansion of ||vout_r - V_j||_M^2 (clamped at 0 against
// rounding), then P sqrt(q) / max(1 - P, eps) (Eq. 6-7).
__device__ inline double fused_drift_key(double p, double c, double a, double vmj, double eps) {
  const double q = fmax(a - 2.0 * c + vmj, 0.0);
  return p * sqrt(q) / fmax(1.0 - p, eps);
}

// 4. the exact top-c of the wave's row of keys (float64, held at keyrow)
// among the candidates, ties to the lower block index, plus every
// always-kept block: the kept blocks as a per-lane bitmask over k (lane l
// owns blocks l + 64k). whist: the wave's 256-entry histogram.
template <int KPL>
__device__ inline uint64_t fused_topk_bits(const double* keyrow, int n, const SelConfig& cfg,
                                           int c, uint32_t* whist) {
  const int lane = threadIdx.x & 63;
  SelKeys<KPL> keys(reinterpret_cast<const uint64_t*>(keyrow), n, lane);
  uint64_t member = 0, always = 0;
#pragma unroll
  for (int k = 0; k < KPL; ++k) {
    const int j = lane + 64 * k;
    keys.v[k] = j < n ? order_key(__longlong_as_double((long long)keys.v[k])) : 0ull;
    if (j < n) {
      if (sel_always_wave(cfg, j))
        always |= 1ull << k;
      else
        member |= 1ull << k;
    }
  }
  return wave_select<KPL>(keys, member, n, c, whist) | always;
}

}  // namespace ress
