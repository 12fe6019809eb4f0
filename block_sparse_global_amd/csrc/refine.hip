// Drop-set refinement ("ReSS: Residual-Restoring Sparse Attention for 3D
// Vision Transformers", §4.3 "Iterative Residual Restoration", Eq. 10-17,
// and Appendix E "Fused Kernel Implementation").
//
// One workgroup refines TR consecutive query-block rows of one head, with all
// rounds inside the kernel:
//   * gains: every thread owns one key block j per pass, streams V_j once
//     and forms V_j . (M g_r) for all TR rows, then the exact objective
//     decrease of Eq. 16 for restoring (j in D, Eq. 14) or dropping (j kept,
//     Eq. 15) j; gains are kept in LDS as 64-bit order keys;
//   * selection: wave r selects the m_r best restores and the m_r best drops
//     of row r by an exact radix select (ties: lower block index), with no
//     workgroup barrier;
//   * update: g and K move by the swapped blocks only (Eq. 13); G = g^T M g
//     and J = G / K^2 (Eq. 12) are recomputed; the drop set with the smallest
//     J seen is kept (track-best).
// s_j (Eq. 6) comes from the drift key of Eq. 7: s = key * max(1 - P, eps).
// All reductions have a fixed order, so results are bit-reproducible.
#include "ress_internal.h"

namespace ress {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kD = 64;

struct RowScal {
  double K, G, J, Jbest, J0, vu;  // vu = vout . (M g)
  int nD, nS, nchg, pad;
};

// Exact top-m of one row's gains within one wave. Lane l owns key blocks
// j = l + 64k; bit k of `member` marks membership. Returns the selected
// elements of this lane as a bitmask over k.
__device__ uint64_t wave_select(const uint64_t* __restrict__ g, uint64_t member,
                                int n, int m, uint32_t* __restrict__ whist) {
  const int lane = threadIdx.x & 63;
  uint64_t selected = 0, inplay = member;
  if (m <= 0) return 0;
  int need = m;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int b = lane; b < 256; b += 64) whist[b] = 0u;
    wave_lds_sync();
    for (int k = 0, j = lane; j < n; ++k, j += 64)
      if ((inplay >> k) & 1ull) atomicAdd(&whist[(uint32_t)(g[j] >> shift) & 255u], 1u);
    wave_lds_sync();
    int c[4];
    int s = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] = (int)whist[255 - 4 * lane - q];
      s += c[q];
    }
    int x = s;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    const int before = x - s;
    const bool found = before < need && need <= x;
    int dsel = 0, above = 0, atd = 0;
    if (found) {
      int cum = before;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (cum + c[q] >= need) {
          dsel = 255 - 4 * lane - q;
          above = cum;
          atd = c[q];
          break;
        }
        cum += c[q];
      }
    }
    const int src = __ffsll((unsigned long long)__ballot(found)) - 1;
    dsel = __shfl(dsel, src, 64);
    above = __shfl(above, src, 64);
    atd = __shfl(atd, src, 64);
    wave_lds_sync();
    for (int k = 0, j = lane; j < n; ++k, j += 64) {
      if ((inplay >> k) & 1ull) {
        const int dig = (int)((uint32_t)(g[j] >> shift) & 255u);
        if (dig > dsel) selected |= 1ull << k;
        if (dig != dsel) inplay &= ~(1ull << k);
      }
    }
    need -= above;
    if (atd == need) return selected | inplay;
  }
  // equal keys remain: take the lowest `need` block indices (k-major order)
  const uint64_t below = (1ull << lane) - 1ull;
  int taken = 0;
  for (int k = 0, j0 = 0; j0 < n; ++k, j0 += 64) {
    const bool b = (inplay >> k) & 1ull;
    const uint64_t mask = __ballot(b);
    if (b && taken + __popcll(mask & below) < need) selected |= 1ull << k;
    taken += __popcll(mask);
  }
  return selected;
}

template <int TR>
__global__ __launch_bounds__(kThreads) void refine_kernel(
    const double* __restrict__ P, const double* __restrict__ key,
    const double* __restrict__ vpool, const double* __restrict__ vout,
    const double* __restrict__ M, int n, SelConfig cfg, int rounds, double rho,
    double eps, int k_max, int32_t* __restrict__ kept_idx,
    int32_t* __restrict__ kept_cnt, double* __restrict__ J_init,
    double* __restrict__ J_final) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int n_even = (n + 1) & ~1;  // keeps the regions below 16-byte aligned
  uint64_t* gains = reinterpret_cast<uint64_t*>(smem);    // [TR][n] (stride n)
  double* vo = reinterpret_cast<double*>(gains + TR * n_even);  // [TR][64] vout_r
  double* gv = vo + TR * kD;                               // [TR][64] g_r
  double* uv = gv + TR * kD;                               // [TR][64] M g_r
  RowScal* rs = reinterpret_cast<RowScal*>(uv + TR * kD);  // [TR]
  uint32_t* hist = reinterpret_cast<uint32_t*>(rs + TR);   // [kWaves][256]
  uint8_t* fcur = reinterpret_cast<uint8_t*>(hist + kWaves * 256);  // [TR][n]
  uint8_t* fbest = fcur + TR * n;                                   // [TR][n]

  const int h = blockIdx.y;
  const int i0 = blockIdx.x * TR;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int nrow = min(TR, n - i0);
  const double* Ph = P + (size_t)h * n * n;
  const double* Kh = key + (size_t)h * n * n;
  const double* Vh = vpool + (size_t)h * n * kD;
  const double* Mh = M ? M + (size_t)h * kD * kD : nullptr;
  const int c = cfg.keep[h] - cfg.n_always;

  // ---- initial drop sets D_r = candidates not in the input keep lists
  for (int idx = tid; idx < TR * kD; idx += kThreads) {
    const int r = idx / kD;
    vo[idx] = (r < nrow) ? vout[((size_t)h * n + i0 + r) * kD + idx % kD] : 0.0;
  }
  for (int idx = tid; idx < TR * n; idx += kThreads) {
    const int r = idx / n, j = idx % n;
    fcur[idx] = (r < nrow && !sel_always(cfg, j)) ? 1 : 0;
  }
  __syncthreads();
  for (int idx = tid; idx < TR * k_max; idx += kThreads) {
    const int r = idx / k_max, q = idx % k_max;
    if (r >= nrow) continue;
    const size_t row = (size_t)h * n + i0 + r;
    int cnt = kept_cnt[row];
    cnt = cnt < 0 ? 0 : (cnt > k_max ? k_max : cnt);
    if (q >= cnt) continue;
    const int j = kept_idx[row * k_max + q];
    if (j >= 0 && j < n) fcur[r * n + j] = 0;
  }
  __syncthreads();

  // ---- initial g_r = sum_{j in D_r} P_rj (vout_r - V_j) (Eq. 5, 10).
  // Thread (d, q): row q % TR, slice q / TR of the key blocks; the slices
  // are then added in ascending order.
  {
    double* part = reinterpret_cast<double*>(hist);  // 4 x 64 doubles
    const int d = tid & 63, q = tid >> 6;
    const int r = q % TR, sl = q / TR, nsl = kWaves / TR;
    double acc = 0.0;
    if (r < nrow) {
      const double vod = vo[r * kD + d];
      const double* Prow = Ph + (size_t)(i0 + r) * n;
      const int per = (n + nsl - 1) / nsl;
      const int j0 = sl * per, j1 = min(n, j0 + per);
      // unconditional (predicated) loads so that the unrolled iterations
      // keep many loads in flight; adding +0 for j outside D leaves acc as is
#pragma unroll 16
      for (int j = j0; j < j1; ++j) {
        const double t = Prow[j] * (vod - Vh[(size_t)j * kD + d]);
        acc += fcur[r * n + j] ? t : 0.0;
      }
    }
    part[q * kD + d] = acc;
    __syncthreads();
    if (tid < TR * kD) {
      const int rr = tid / kD, dd = tid % kD;
      double s = 0.0;
      for (int s2 = 0; s2 < nsl; ++s2) s += part[(s2 * TR + rr) * kD + dd];
      gv[tid] = s;
    }
    __syncthreads();
  }

  // ---- per-row scalars: wave r owns row r
  auto row_state = [&](int r, bool first) {
    double u = gv[r * kD + lane];
    if (Mh != nullptr) {
      const double* Mrow = Mh + (size_t)lane * kD;
      u = 0.0;
#pragma unroll 8
      for (int e = 0; e < kD; ++e) u = fma(Mrow[e], gv[r * kD + e], u);
    }
    uv[r * kD + lane] = u;
    const double G = wave_sum64(gv[r * kD + lane] * u);
    const double vu = wave_sum64(vo[r * kD + lane] * u);
    if (lane == 0) {
      RowScal& st = rs[r];
      st.G = G;
      st.vu = vu;
      st.J = (st.K > 0.0) ? G / (st.K * st.K) : INFINITY;
      if (first) {
        st.J0 = st.J;
        st.Jbest = st.J;
      }
    }
  };
  if (wave < nrow) {
    const int r = wave;
    const double* Prow = Ph + (size_t)(i0 + r) * n;
    double ks = 0.0;
    int nD = 0, nS = 0;
    for (int j = lane; j < n; j += 64) {
      const bool cand = !sel_always(cfg, j);
      const bool inD = fcur[r * n + j] != 0;
      if (inD) ks += Prow[j];
      nD += inD;
      nS += cand && !inD;
    }
    const double K = 1.0 - wave_sum64(ks);
    nD = wave_isum64(nD);
    nS = wave_isum64(nS);
    if (lane == 0) {
      rs[r].K = K;
      rs[r].nD = nD;
      rs[r].nS = nS;
    }
    wave_lds_sync();
    row_state(r, true);
    for (int j = lane; j < n; j += 64) fbest[r * n + j] = fcur[r * n + j];
  }
  __syncthreads();

  for (int round = 0; round < rounds; ++round) {
    const int m_base = (int)floor(rho * (double)c / ldexp(1.0, round + 1));
    if (m_base <= 0) continue;  // uniform: every row of the head shares c

    // ---- gains of every (row, key block) from the round-start state
    double sK[TR], sG[TR], sJ[TR], svu[TR];
#pragma unroll
    for (int r = 0; r < TR; ++r) {
      sK[r] = rs[r].K; sG[r] = rs[r].G; sJ[r] = rs[r].J; svu[r] = rs[r].vu;
    }
    for (int jb = 0; jb < n; jb += kThreads) {
      // keeps the (loop-invariant) M g reads below inside the loop: hoisting
      // all TR x 64 of them would not fit in registers
      asm volatile("" ::: "memory");
      const int j = jb + tid;
      if (j >= n || sel_always(cfg, j)) continue;
      double acc[TR];
#pragma unroll
      for (int r = 0; r < TR; ++r) acc[r] = 0.0;
      const double2* vj = reinterpret_cast<const double2*>(Vh + (size_t)j * kD);
#pragma unroll 1
      for (int ch = 0; ch < kD / 16; ++ch) {
        double2 x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = vj[ch * 8 + e];
#pragma unroll
        for (int r = 0; r < TR; ++r) {
          const double2* ur = reinterpret_cast<const double2*>(uv + r * kD) + ch * 8;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const double2 uu = ur[e];
            acc[r] = fma(x[e].x, uu.x, acc[r]);
            acc[r] = fma(x[e].y, uu.y, acc[r]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < TR; ++r) {
        if (r >= nrow) break;
        const size_t off = (size_t)(i0 + r) * n + j;
        const double p = Ph[off];
        const double s = Kh[off] * fmax(1.0 - p, eps);  // s_rj (Eq. 6)
        const double s2 = s * s;
        const double dMg = p * (svu[r] - acc[r]);       // d_j^T M g
        double dJ;
        if (fcur[r * n + j]) {  // restore (Eq. 13-14), u = +P_j
          const double dG = -2.0 * dMg + s2;
          const double Ku = sK[r] + p;
          dJ = sJ[r] - (sG[r] + dG) / (Ku * Ku);
        } else {  // drop (Eq. 15), u = -P_j
          const double dG = 2.0 * dMg + s2;
          const double Ku = sK[r] - p;
          dJ = (Ku > 0.0) ? sJ[r] - (sG[r] + dG) / (Ku * Ku) : -INFINITY;
        }
        gains[r * n + j] = order_key(dJ);
      }
    }
    __syncthreads();

    // ---- selection and set update: wave r owns row r
    if (wave < nrow) {
      const int r = wave;
      RowScal& st = rs[r];
      const int m = min(m_base, min(st.nD, st.nS));
      uint64_t memD = 0, memS = 0;
      for (int k = 0, j = lane; j < n; ++k, j += 64) {
        if (sel_always(cfg, j)) continue;
        if (fcur[r * n + j]) memD |= 1ull << k; else memS |= 1ull << k;
      }
      uint32_t* whist = hist + wave * 256;
      const uint64_t restore = wave_select(gains + r * n, memD, n, m, whist);
      const uint64_t drop = wave_select(gains + r * n, memS, n, m, whist);
      // change list (ascending block index, sign = +1 for a drop), stored
      // over this row's gains, which are no longer needed
      int32_t* chg = reinterpret_cast<int32_t*>(gains + r * n);
      const double* Prow = Ph + (size_t)(i0 + r) * n;
      const uint64_t below = (1ull << lane) - 1ull;
      int pos = 0;
      double dk = 0.0;
      for (int k = 0, j0 = 0; j0 < n; ++k, j0 += 64) {
        const int j = j0 + lane;
        const bool rb = (restore >> k) & 1ull, db = (drop >> k) & 1ull;
        const uint64_t msk = __ballot(rb || db);
        if (rb || db) {
          chg[pos + __popcll(msk & below)] = db ? (j + 1) : -(j + 1);
          fcur[r * n + j] = db ? 1 : 0;
          dk += rb ? Prow[j] : -Prow[j];
        }
        pos += __popcll(msk);
      }
      dk = wave_sum64(dk);
      if (lane == 0) {
        st.K += dk;  // Eq. 13: K moves by +P for a restore, -P for a drop
        st.nchg = pos;
      }
    }
    __syncthreads();

    // ---- g moves by the swapped blocks (Eq. 13), in ascending order
    if (tid < TR * kD) {
      const int r = tid / kD, d = tid % kD;
      if (r < nrow) {
        const int nchg = rs[r].nchg;
        const int32_t* chg = reinterpret_cast<const int32_t*>(gains + r * n);
        const double* Prow = Ph + (size_t)(i0 + r) * n;
        const double vod = vo[r * kD + d];
        double g = gv[r * kD + d];
#pragma unroll 8
        for (int q = 0; q < nchg; ++q) {
          const int e = chg[q];
          const int j = (e > 0 ? e : -e) - 1;
          const double dj = Prow[j] * (vod - Vh[(size_t)j * kD + d]);
          g = (e > 0) ? g + dj : g - dj;
        }
        gv[r * kD + d] = g;
      }
    }
    __syncthreads();
    if (wave < nrow) {
      const int r = wave;
      row_state(r, false);
      wave_lds_sync();
      if (rs[r].J < rs[r].Jbest) {  // track-best, strict
        for (int j = lane; j < n; j += 64) fbest[r * n + j] = fcur[r * n + j];
        wave_lds_sync();
        if (lane == 0) rs[r].Jbest = rs[r].J;
      }
    }
    __syncthreads();
  }

  // ---- keep lists from the best drop sets, ascending, -1 padded
  if (wave < nrow) {
    const int r = wave;
    const size_t row = (size_t)h * n + i0 + r;
    int32_t* out = kept_idx + row * k_max;
    const uint64_t below = (1ull << lane) - 1ull;
    int pos = 0;
    for (int j0 = 0; j0 < n; j0 += 64) {
      const int j = j0 + lane;
      const bool kept = j < n && (sel_always(cfg, j) || !fbest[r * n + j]);
      const uint64_t msk = __ballot(kept);
      const int p = pos + __popcll(msk & below);
      if (kept && p < k_max) out[p] = j;
      pos += __popcll(msk);
    }
    for (int p = pos + lane; p < k_max; p += 64) out[p] = -1;
    if (lane == 0) {
      kept_cnt[row] = pos < k_max ? pos : k_max;
      if (J_init) J_init[row] = rs[r].J0;
      if (J_final) J_final[row] = rs[r].Jbest;
    }
  }
}

size_t lds_bytes(int TR, int n) {
  const size_t n_even = (size_t)((n + 1) & ~1);
  return (size_t)TR * n_even * 8 + 3 * (size_t)TR * kD * 8 + TR * sizeof(RowScal) +
         kWaves * 256 * 4 + 2 * (size_t)TR * n;
}

}  // namespace

hipError_t launch_refine(const double* P, const double* key,
                         const double* vpool, const double* vout,
                         const double* M, const ress_shape& s,
                         const SelConfig& cfg, int32_t rounds, double rho,
                         double eps, int32_t k_max, int32_t* kept_idx,
                         int32_t* kept_cnt, double* J_init, double* J_final,
                         hipStream_t st) {
  const int n = s.N_pad / s.B;
  // rows per workgroup: as many as keep the LDS footprint within 64 KB
  int TR = 4;
  while (TR > 1 && lds_bytes(TR, n) > 65536) TR >>= 1;
  dim3 grid((n + TR - 1) / TR, s.H);
  const size_t lds = lds_bytes(TR, n);
  switch (TR) {
#define RESS_CASE(T)                                                          \
  case T:                                                                     \
    hipLaunchKernelGGL((refine_kernel<T>), grid, dim3(kThreads), lds, st, P,  \
                       key, vpool, vout, M, n, cfg, rounds, rho, eps, k_max,  \
                       kept_idx, kept_cnt, J_init, J_final);                  \
    break;
    RESS_CASE(4)
    RESS_CASE(2)
    RESS_CASE(1)
#undef RESS_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ress
