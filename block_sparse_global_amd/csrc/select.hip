// Per-row selection: top-k keep sets and drop-set refinement.
//
// Top-k ("ReSS: Residual-Restoring Sparse Attention for 3D Vision
// Transformers", §3 step (2), §4.1 Eq. 2, §4.4): per (head, query-block
// row), keep the c_h candidates with the largest key plus every always-kept
// block.
// Refinement (same page, §4.3, Eq. 10-17): budget-neutral restore/drop
// rounds on the drop set with track-best.
//
// One workgroup owns one row; thread t owns the E consecutive key blocks
// [t*E, t*E + E). Selection is exact: an MSB-first radix select over 64-bit
// keys whose unsigned order equals the float64 order, with ties among equal
// keys broken towards the lower block index by a block-wide prefix count.
// No float atomics and fixed-order reductions: results are bit-reproducible.
#include "ress_internal.h"

namespace ress {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kD = 64;

struct SelShared {
  uint32_t hist[256];
  int32_t wave_tot[kWaves];
  double red[kWaves];
  int32_t digit, above, at_digit;
};

__device__ inline uint64_t order_key(double x) {
  if (x == 0.0) x = 0.0;  // -0 and +0 compare equal
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ inline double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Exclusive prefix sum of one int per thread, in thread order; *total gets
// the sum over the workgroup.
__device__ int block_exclusive_scan(int v, SelShared& sh, int* total) {
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh.wave_tot[w] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) {
    if (k < w) base += sh.wave_tot[k];
    tot += sh.wave_tot[k];
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

__device__ inline int block_count(int v, SelShared& sh) {
  int total;
  block_exclusive_scan(v, sh, &total);
  return total;
}

// Sum of one double per thread in a fixed order (waves, then wave totals in
// ascending order); the result is returned to every thread.
__device__ double block_sum(double v, SelShared& sh) {
  const int t = threadIdx.x;
  v = wave_sum(v);
  if ((t & 63) == 0) sh.red[t >> 6] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) s += sh.red[k];
  __syncthreads();
  return s;
}

// Selects the m members with the largest keys (ties: lower element index,
// where thread t's element e has index t*E + e). Requires 0 <= m <= number
// of members. Returns the selected elements of this thread as a bitmask.
template <int E>
__device__ uint32_t select_top(const uint64_t (&u)[E], uint32_t member, int m,
                               SelShared& sh) {
  const int t = threadIdx.x;
  uint32_t selected = 0;
  uint32_t inplay = member;
  if (m <= 0) return 0u;
  int need = m;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int k = t; k < 256; k += kThreads) sh.hist[k] = 0u;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((inplay >> e) & 1u)
        atomicAdd(&sh.hist[(uint32_t)(u[e] >> shift) & 255u], 1u);
    __syncthreads();
    if (t < 64) {
      // lane l covers digits 255-4l .. 252-4l (descending)
      int c[4];
      int s = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        c[k] = (int)sh.hist[255 - 4 * t - k];
        s += c[k];
      }
      int x = s;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (t >= o) x += y;
      }
      const int before = x - s;
      if (before < need && need <= x) {
        int cum = before;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (cum + c[k] >= need) {
            sh.digit = 255 - 4 * t - k;
            sh.above = cum;
            sh.at_digit = c[k];
            break;
          }
          cum += c[k];
        }
      }
    }
    __syncthreads();
    const uint32_t dsel = (uint32_t)sh.digit;
    const int above = sh.above, at_digit = sh.at_digit;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if ((inplay >> e) & 1u) {
        const uint32_t dig = (uint32_t)(u[e] >> shift) & 255u;
        if (dig > dsel) selected |= 1u << e;
        if (dig != dsel) inplay &= ~(1u << e);
      }
    }
    need -= above;
    if (at_digit == need) return selected | inplay;
  }
  // The elements still in play all carry the same key: take the `need`
  // lowest indices.
  int total;
  int rank = block_exclusive_scan(__popc(inplay), sh, &total);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if ((inplay >> e) & 1u) {
      if (rank < need) selected |= 1u << e;
      ++rank;
    }
  }
  return selected;
}

// Writes the ascending list of kept blocks (bitmask per thread) of one row,
// pads it with -1 up to k_max, and stores the count.
template <int E>
__device__ void write_kept(uint32_t kept, int n, int k_max,
                           int32_t* __restrict__ out_idx,
                           int32_t* __restrict__ out_cnt, SelShared& sh) {
  const int t = threadIdx.x;
  int total;
  int pos = block_exclusive_scan(__popc(kept), sh, &total);
#pragma unroll
  for (int e = 0; e < E; ++e)
    if ((kept >> e) & 1u) {
      if (pos < k_max) out_idx[pos] = t * E + e;
      ++pos;
    }
  for (int p = total + t; p < k_max; p += kThreads) out_idx[p] = -1;
  if (t == 0) *out_cnt = total < k_max ? total : k_max;
}

template <int E>
__global__ __launch_bounds__(kThreads) void topk_kernel(
    const double* __restrict__ key, int n, SelConfig cfg, int k_max,
    int32_t* __restrict__ kept_idx, int32_t* __restrict__ kept_cnt) {
  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int t = threadIdx.x;
  __shared__ SelShared sh;
  const double* row = key + ((size_t)h * n + i) * n;
  uint64_t u[E];
  uint32_t member = 0, always = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = t * E + e;
    u[e] = 0;
    if (j < n) {
      u[e] = order_key(row[j]);
      if (sel_always(cfg, j))
        always |= 1u << e;
      else
        member |= 1u << e;
    }
  }
  const int c = cfg.keep[h] - cfg.n_always;
  const uint32_t sel = select_top<E>(u, member, c, sh);
  const size_t r = (size_t)h * n + i;
  write_kept<E>(sel | always, n, k_max, kept_idx + r * k_max, kept_cnt + r,
                sh);
}

// ---------------------------------------------------------------------------
// Refinement
// ---------------------------------------------------------------------------

struct RefineShared {
  SelShared sel;
  double vo[kD];   // vout_i
  double ws[kD];   // M vout_i
  double gs[kD];   // g
  double us[kD];   // M g
  double part[kWaves][kD];
  double scal[2];
  uint8_t flag[RESS_MAX_BLOCKS];  // membership of the current drop set
};

struct State {
  double K, G, J;
};

// g = sum_{j in D} P_j (vout - V_j), K = 1 - sum_{j in D} P_j, u = M g,
// G = g . u, J = G / K^2 (Eq. 10, 12). flag[] holds D.
template <int E>
__device__ State recompute(const double* __restrict__ Prow,
                           const double* __restrict__ Vh,
                           const double* __restrict__ Mh, int n,
                           const double (&p)[E], uint32_t inD,
                           RefineShared& sh) {
  const int t = threadIdx.x;
  const int d = t & 63, sl = t >> 6;
  const int per = (n + kWaves - 1) / kWaves;
  const int j0 = sl * per, j1 = min(n, j0 + per);
  const double vod = sh.vo[d];
  double acc = 0.0;
  for (int j = j0; j < j1; ++j)
    if (sh.flag[j]) acc += Prow[j] * (vod - Vh[(size_t)j * kD + d]);
  sh.part[sl][d] = acc;
  double ks = 0.0;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if ((inD >> e) & 1u) ks += p[e];
  __syncthreads();
  if (t < kD) {
    double g = 0.0;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) g += sh.part[k][t];
    sh.gs[t] = g;
  }
  const double K = 1.0 - block_sum(ks, sh.sel);  // contains barriers
  if (t < kD) {
    double u = sh.gs[t];
    if (Mh != nullptr) {
      const double* Mrow = Mh + (size_t)t * kD;
      u = 0.0;
#pragma unroll 8
      for (int e = 0; e < kD; ++e) u = fma(Mrow[e], sh.gs[e], u);
    }
    sh.us[t] = u;
    const double G = wave_sum(sh.gs[t] * u);
    if (t == 0) sh.scal[0] = G;
  }
  __syncthreads();
  State s;
  s.K = K;
  s.G = sh.scal[0];
  s.J = (K > 0.0) ? s.G / (K * K) : INFINITY;
  __syncthreads();
  return s;
}

template <int E>
__global__ __launch_bounds__(kThreads) void refine_kernel(
    const double* __restrict__ P, const double* __restrict__ vpool,
    const double* __restrict__ vout, const double* __restrict__ vmv,
    const double* __restrict__ M, int n, SelConfig cfg, int rounds,
    double rho, int k_max, int32_t* __restrict__ kept_idx,
    int32_t* __restrict__ kept_cnt, double* __restrict__ J_init,
    double* __restrict__ J_final) {
  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int t = threadIdx.x;
  __shared__ RefineShared sh;
  const size_t row = (size_t)h * n + i;
  const double* Prow = P + row * n;
  const double* Vh = vpool + (size_t)h * n * kD;
  const double* Mh = M ? M + (size_t)h * kD * kD : nullptr;
  const double* vmvh = vmv + (size_t)h * n;
  const int c = cfg.keep[h] - cfg.n_always;

  if (t < kD) sh.vo[t] = vout[row * kD + t];
  for (int j = t; j < n; j += kThreads) sh.flag[j] = 0;
  __syncthreads();
  int cnt = kept_cnt[row];
  cnt = cnt < 0 ? 0 : (cnt > k_max ? k_max : cnt);
  for (int q = t; q < cnt; q += kThreads) {
    const int j = kept_idx[row * k_max + q];
    if (j >= 0 && j < n) sh.flag[j] = 1;
  }
  __syncthreads();

  double p[E];
  uint32_t cand = 0, inD = 0, always = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = t * E + e;
    p[e] = 0.0;
    if (j < n) {
      p[e] = Prow[j];
      if (sel_always(cfg, j)) {
        always |= 1u << e;
      } else {
        cand |= 1u << e;
        if (!sh.flag[j]) inD |= 1u << e;
      }
    }
  }
  // w = M vout and a = vout . w, for s_j^2 = P_j^2 q_j (Eq. 6, 9)
  if (t < kD) {
    double w = sh.vo[t];
    if (Mh != nullptr) {
      const double* Mrow = Mh + (size_t)t * kD;
      w = 0.0;
#pragma unroll 8
      for (int e = 0; e < kD; ++e) w = fma(Mrow[e], sh.vo[e], w);
    }
    sh.ws[t] = w;
    const double a = wave_sum(sh.vo[t] * w);
    if (t == 0) sh.scal[1] = a;
  }
  __syncthreads();
  const double a = sh.scal[1];
  double s2[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    s2[e] = 0.0;
    if ((cand >> e) & 1u) {
      const int j = t * E + e;
      const double2* vj = reinterpret_cast<const double2*>(Vh + (size_t)j * kD);
      double wv = 0.0;
#pragma unroll 8
      for (int k = 0; k < kD / 2; ++k) {
        const double2 x = vj[k];
        wv = fma(sh.ws[2 * k], x.x, wv);
        wv = fma(sh.ws[2 * k + 1], x.y, wv);
      }
      const double q = fmax(a - 2.0 * wv + vmvh[j], 0.0);
      s2[e] = p[e] * p[e] * q;
    }
  }
  // drop-set flags
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = t * E + e;
    if (j < n) sh.flag[j] = (inD >> e) & 1u;
  }
  __syncthreads();
  State st = recompute<E>(Prow, Vh, Mh, n, p, inD, sh);
  const double J0 = st.J;
  double Jbest = st.J;
  uint32_t bestD = inD;

  for (int r = 0; r < rounds; ++r) {
    int m = (int)floor(rho * (double)c / ldexp(1.0, r + 1));
    const int nD = block_count(__popc(inD), sh.sel);
    const int nS = block_count(__popc(cand & ~inD), sh.sel);
    m = min(m, min(nD, nS));
    if (m <= 0) continue;
    const double J = st.G / (st.K * st.K);
    uint64_t gain[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      gain[e] = 0;
      if ((cand >> e) & 1u) {
        const int j = t * E + e;
        const double2* vj =
            reinterpret_cast<const double2*>(Vh + (size_t)j * kD);
        double eu = 0.0;
#pragma unroll 8
        for (int k = 0; k < kD / 2; ++k) {
          const double2 x = vj[k];
          eu = fma(sh.vo[2 * k] - x.x, sh.us[2 * k], eu);
          eu = fma(sh.vo[2 * k + 1] - x.y, sh.us[2 * k + 1], eu);
        }
        const double dMg = p[e] * eu;  // d_j^T M g
        double dJ;
        if ((inD >> e) & 1u) {  // restore: Eq. 14, u = +P_j
          const double dG = -2.0 * dMg + s2[e];
          const double Ku = st.K + p[e];
          dJ = J - (st.G + dG) / (Ku * Ku);
        } else {  // drop: Eq. 15, u = -P_j
          const double dG = 2.0 * dMg + s2[e];
          const double Ku = st.K - p[e];
          dJ = (Ku > 0.0) ? J - (st.G + dG) / (Ku * Ku) : -INFINITY;
        }
        gain[e] = order_key(dJ);
      }
    }
    const uint32_t restore = select_top<E>(gain, inD, m, sh.sel);
    const uint32_t drop = select_top<E>(gain, cand & ~inD, m, sh.sel);
    inD = (inD & ~restore) | drop;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = t * E + e;
      if (j < n) sh.flag[j] = (inD >> e) & 1u;
    }
    __syncthreads();
    st = recompute<E>(Prow, Vh, Mh, n, p, inD, sh);
    if (st.J < Jbest) {
      Jbest = st.J;
      bestD = inD;
    }
  }
  write_kept<E>((cand & ~bestD) | always, n, k_max, kept_idx + row * k_max,
                kept_cnt + row, sh.sel);
  if (t == 0) {
    if (J_init) J_init[row] = J0;
    if (J_final) J_final[row] = Jbest;
  }
}

int pick_e(int n) {
  const int need = (n + kThreads - 1) / kThreads;
  int e = 1;
  while (e < need) e <<= 1;
  return e;
}

}  // namespace

hipError_t launch_topk(const double* key, const ress_shape& s,
                       const SelConfig& cfg, int32_t k_max, int32_t* kept_idx,
                       int32_t* kept_cnt, hipStream_t st) {
  const int n = s.N_pad / s.B;
  dim3 grid(n, s.H);
  switch (pick_e(n)) {
#define RESS_CASE(E)                                                        \
  case E:                                                                   \
    hipLaunchKernelGGL((topk_kernel<E>), grid, dim3(kThreads), 0, st, key, \
                       n, cfg, k_max, kept_idx, kept_cnt);                  \
    break;
    RESS_CASE(1)
    RESS_CASE(2)
    RESS_CASE(4)
    RESS_CASE(8)
    RESS_CASE(16)
#undef RESS_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_refine(const double* P, const double* vpool,
                         const double* vout, const double* vmv,
                         const double* M, const ress_shape& s,
                         const SelConfig& cfg, int32_t rounds, double rho,
                         int32_t k_max, int32_t* kept_idx, int32_t* kept_cnt,
                         double* J_init, double* J_final, hipStream_t st) {
  const int n = s.N_pad / s.B;
  dim3 grid(n, s.H);
  switch (pick_e(n)) {
#define RESS_CASE(E)                                                          \
  case E:                                                                     \
    hipLaunchKernelGGL((refine_kernel<E>), grid, dim3(kThreads), 0, st, P,   \
                       vpool, vout, vmv, M, n, cfg, rounds, rho, k_max,       \
                       kept_idx, kept_cnt, J_init, J_final);                  \
    break;
    RESS_CASE(1)
    RESS_CASE(2)
    RESS_CASE(4)
    RESS_CASE(8)
    RESS_CASE(16)
#undef RESS_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ress
