// Fused selection: pooled blocks in, keep lists out, with the block map and
// the ranking key of a row never leaving the chip ("ReSS: Residual-Restoring
// Sparse Attention for 3D Vision Transformers", §3 steps (1)-(2), §4.1-§4.2
// Eq. 1-9; the fused, one-sweep-per-row form of its Appendix E).
//
// One workgroup takes R consecutive query-block rows of one head, one wave
// per row, and keeps those rows in LDS (R x n float64, about 140 KB):
//  1. logits l_rj = scale * qpool_r . kpool_j for every key block j, on the
//     float64 matrix cores (v_mfma_f64_16x16x4f64: the R rows against 16 key
//     blocks per instruction group, the waves taking the groups in turn);
//  2. per row (its wave, the row in registers): the softmax over all j (the
//     map P, normalised over every key block, §4.1);
//  3. drift only: vout_r = sum_j P_rj V_j (Eq. 1) on the matrix cores, the
//     key blocks split in quarters whose partial sums are added in a fixed
//     order; then w_r = M vout_r and a_r = vout_r . w_r; then
//     c_rj = w_r . V_j on the matrix cores, whose epilogue forms
//     q = a_r - 2 c_rj + vmv_j (the Eq. 9 expansion) and the key
//     P sqrt(max(q, 0)) / max(1 - P, eps) (Eq. 6-7) in place of P;
//  4. per row: the exact top-c_h of the keys among the candidates (the
//     radix select of the other selection kernels, ties to the lower block
//     index), plus the always-kept blocks, as an ascending keep list.
// Only the keep lists leave the chip (and vmv, V_j^T M V_j per key block, a
// vector of n_k per head computed before the launch). Rows of up to 2176 key
// blocks: R = 16 rows up to 1088 blocks, R = 8 beyond (half of each
// matrix-core row group then idles).
#include "ress_internal.h"
#include "select_fused_steps.h"

namespace ress {
namespace {

constexpr int kScratch = 16384;  // bytes: vout partials, then w and a, then histograms

__host__ __device__ inline size_t fused_sel_lds(int R, int n) {
  return (size_t)R * row_stride(n) * 8 + kScratch;
}

template <int KPL, int R>
__global__ __launch_bounds__(64 * R) void select_fused_kernel(
    const double* __restrict__ qpool, const double* __restrict__ kpool,
    const double* __restrict__ vpool, const double* __restrict__ M,
    const double* __restrict__ vmv, int nq, int n, double scale, double eps, int drift,
    SelConfig cfg, int k_max, int32_t* __restrict__ kept_idx, int32_t* __restrict__ kept_cnt) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int ns = row_stride(n);
  double* rows = reinterpret_cast<double*>(smem);                       // [R][ns]
  unsigned char* scratch = smem + (size_t)R * ns * 8;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.y, i0 = blockIdx.x * R;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int ngroups = (n + 15) >> 4;  // 16-block groups of key blocks
  const double* qh = qpool + (size_t)h * nq * kD;
  const double* kh = kpool + (size_t)h * n * kD;
  const double* vh = vpool ? vpool + (size_t)h * n * kD : nullptr;

  // ---- 1. logits of the R rows against every key block
  fused_logits<R>(qh, kh, nq, n, i0, scale, rows, ns);
  __syncthreads();

  // ---- 2. softmax of each row (its wave; padding blocks hold 0)
  const bool live = i0 + w < nq;
  double* myrow = rows + w * ns;
  fused_softmax<KPL>(myrow, n, ns);
  __syncthreads();

  if (drift) {
    // ---- 3a-3b. vout, w = M vout and a (w and a then take the place of the
    // partial sums)
    double* part = reinterpret_cast<double*>(scratch);  // [2][R][64]
    double* wv = part;                                  // [R][64]
    double* av = wv + R * kD;                           // [R]
    fused_vout<R>(rows, ns, n, vh, M ? M + (size_t)h * kD * kD : nullptr, part, nullptr, wv,
                  av);
    __syncthreads();
    // ---- 3c. c_rj = w_r . V_j; the key replaces P in the row buffer
    {
      double wa[16];
      const double* wr = wv + min(l16, R - 1) * kD;
#pragma unroll
      for (int s = 0; s < 16; ++s) wa[s] = wr[4 * s + q4];
      const double* vm = vmv + (size_t)h * n;
      for (int g = w; g < ngroups; g += R) {
        const double* vr = vh + (size_t)min(16 * g + l16, n - 1) * kD;
        f64x4 acc2 = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int s = 0; s < 16; ++s)
          acc2 = __builtin_amdgcn_mfma_f64_16x16x4f64(wa[s], vr[4 * s + q4], acc2, 0, 0, 0);
        const int j = 16 * g + l16;
        if (j < n) {
          const double vmj = vm[j];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = q4 + 4 * e;
            if (r < R) rows[r * ns + j] = fused_drift_key(rows[r * ns + j], acc2[e], av[r], vmj, eps);
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- 4. exact top-c_h per row, keep list ascending
  if (!live) return;  // whole wave; no barrier follows
  uint32_t* whist = reinterpret_cast<uint32_t*>(scratch) + 256 * w;
  const uint64_t kept = fused_topk_bits<KPL>(myrow, n, cfg, cfg.keep[h] - cfg.n_always, whist);
  const size_t row = (size_t)h * nq + i0 + w;
  int32_t* out = kept_idx + row * k_max;
  const uint64_t below = (1ull << lane) - 1ull;
  int pos = 0;
  for (int k = 0, j0 = 0; j0 < n; ++k, j0 += 64) {
    const bool b = (kept >> k) & 1ull;
    const uint64_t msk = __ballot(b);
    const int p = pos + __popcll(msk & below);
    if (b && p < k_max) out[p] = j0 + lane;
    pos += __popcll(msk);
  }
  for (int p = pos + lane; p < k_max; p += 64) out[p] = -1;
  if (lane == 0) kept_cnt[row] = pos < k_max ? pos : k_max;
}

template <int KPL, int R>
hipError_t launch_fused_t(const double* qpool, const double* kpool, const double* vpool,
                          const double* M, const double* vmv, const ress_shape& s,
                          double scale, double eps, int drift, const SelConfig& cfg,
                          int32_t k_max, int32_t* kept_idx, int32_t* kept_cnt, hipStream_t st) {
  const int nq = n_qblocks(s), n = n_kblocks(s);
  const size_t lds = fused_sel_lds(R, n);
  const void* fn = reinterpret_cast<const void*>(&select_fused_kernel<KPL, R>);
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((select_fused_kernel<KPL, R>), dim3((nq + R - 1) / R, s.H), dim3(64 * R),
                     lds, st, qpool, kpool, vpool, M, vmv, nq, n, scale, eps, drift, cfg, k_max,
                     kept_idx, kept_cnt);
  return hipGetLastError();
}

}  // namespace

int select_fused_max_blocks() { return 34 * 64; }

hipError_t launch_select_fused(const double* qpool, const double* kpool, const double* vpool,
                               const double* M, const double* vmv, const ress_shape& s,
                               double scale, double eps, int drift, const SelConfig& cfg,
                               int32_t k_max, int32_t* kept_idx, int32_t* kept_cnt,
                               hipStream_t st) {
  const int n = n_kblocks(s);
  if (n <= 17 * 64)
    return launch_fused_t<17, 16>(qpool, kpool, vpool, M, vmv, s, scale, eps, drift, cfg, k_max,
                                  kept_idx, kept_cnt, st);
  return launch_fused_t<34, 8>(qpool, kpool, vpool, M, vmv, s, scale, eps, drift, cfg, k_max,
                               kept_idx, kept_cnt, st);
}

}  // namespace ress
