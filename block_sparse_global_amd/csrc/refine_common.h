// Device helpers shared by the two refinement paths (per-round kernels over
// all rows, and the fused kernel that keeps a tile of rows on chip for every
// round): the swap schedule, the Gram product, and the exact per-wave top-m
// select over 64-bit order keys.
#pragma once

#include <type_traits>

#include "ress_internal.h"

namespace ress {

constexpr int kD = 64;  // head dim

// Row stride of the flag maps: n rounded up to 16 bytes, so that a row is
// read with aligned 16-byte loads.
__host__ __device__ inline int flag_stride(int n) { return (n + 15) & ~15; }

// Swaps of round r for head h: m_r = floor(rho c / 2^(r+1)) (Eq. 17).
__host__ __device__ inline int swaps_of(const SelConfig& cfg, int h, int round, double rho) {
  const int c = cfg.keep[h] - cfg.n_always;
  return (int)floor(rho * (double)c / ldexp(1.0, round + 1));
}

// u = M g (lane d computes dim d; g in LDS), then G = g^T M g and
// vu = vout^T M g, every lane holding the totals.
__device__ inline double gram_apply(const double* __restrict__ Mh, const double* gl,
                                    double gd, double vod, double* G, double* vu) {
  const int d = threadIdx.x & 63;
  double u = gd;
  if (Mh != nullptr) {
    const double* Mrow = Mh + (size_t)d * kD;
    u = 0.0;
#pragma unroll 8
    for (int e = 0; e < kD; ++e) u = fma(Mrow[e], gl[e], u);
  }
  *G = wave_sum64(gd * u);
  *vu = wave_sum64(vod * u);
  return u;
}

// Cancellation guard of the incremental update of g (Eq. 13: each round g
// moves by the d_j of the swapped blocks). When the result is below 2^-20 of
// the magnitudes it was formed from (per dim: |g| before the round plus the
// swapped |d_j|), the update has cancelled most of its bits (a drop set that
// returns to blocks of tiny probability, say), and g is summed again from its
// definition (Eq. 10): over the smaller of D and the kept blocks S (the sum of
// d_j over all blocks is zero), ascending, as the starting state does. Its
// rounding is then relative to g itself. Both refinement paths apply it.
__device__ inline bool g_cancelled(double g, double mag) {
  return wave_sum64(g * g) < 0x1p-40 * wave_sum64(mag * mag);
}

template <typename InD>
__device__ inline double g_from_sets(InD in_drop, int n, int nD, const double* __restrict__ Prow,
                                     const double* __restrict__ Vh, double vod) {
  const int d = threadIdx.x & 63;
  const bool overD = nD < n - nD;
  double acc = 0.0;
  for (int j = 0; j < n; ++j) {
    if (in_drop(j) != overD) continue;  // the same block for every lane
    const double pj = Prow[j];
    const double vj = Vh[(size_t)j * kD + d];
    acc += overD ? pj * (vod - vj) : pj * (vj - vod);
  }
  return acc;
}

// A row's state as the gains epilogue reads it: K (kept mass, Eq. 12), G,
// J = G / K^2 and vu = vout^T M g.
struct RowScalars {
  double K, G, J, vu;
};

// The exact objective decrease of restoring (inD) or dropping block j of a
// row (Eq. 13-16), from p = P_ij, s = s_ij, the product u_i . V_j and the
// row's state.
__device__ inline double swap_gain(const RowScalars& st, double p, double sv, double uv, bool inD) {
  const double s2 = sv * sv;
  const double dMg = p * (st.vu - uv);  // d_j^T M g_i
  if (inD) {  // restore (Eq. 13-14), u = +P_j
    const double dG = -2.0 * dMg + s2;
    const double Ku = st.K + p;
    return st.J - (st.G + dG) / (Ku * Ku);
  }
  // drop (Eq. 15), u = -P_j
  const double dG = 2.0 * dMg + s2;
  const double Ku = st.K - p;
  return (Ku > 0.0) ? st.J - (st.G + dG) / (Ku * Ku) : -INFINITY;
}

// The row's changes chg[0 .. nchg) (+ (j + 1) for a drop, -(j + 1) for a
// restore), in ascending block order, applied to g (lane d: dim d) and to
// the change dk of K, in batches of 8 whose loads are all issued before
// their sums.
__device__ __attribute__((always_inline)) void apply_changes(const int32_t* chg, int nchg, const double* Prow,
                                     const double* Vh, double vod, double& g, double& mag,
                                     double& dk) {
  const int d = threadIdx.x & 63;
  for (int q0 = 0; q0 < nchg; q0 += 8) {
    int ev[8];
    double pv[8], vv[8];
    // lanes 0-7 read the batch's entries in one LDS access; each goes to a
    // scalar register (readlane), so the addresses are scalar work
    const int mine = chg[min(q0 + (d & 7), nchg - 1)];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      ev[t] = __builtin_amdgcn_readlane(mine, t);
      const int j = (ev[t] > 0 ? ev[t] : -ev[t]) - 1;
      pv[t] = Prow[j];
      vv[t] = Vh[(size_t)j * kD + d];
    }
    // a uniform bound instead of a break, so that the loop unrolls and the
    // batch's registers are addressed directly
    const int live = min(8, nchg - q0);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (t < live) {
        const double dj = pv[t] * (vod - vv[t]);
        g = (ev[t] > 0) ? g + dj : g - dj;
        mag += fabs(dj);
        dk = (ev[t] > 0) ? dk - pv[t] : dk + pv[t];  // K: +P for a restore, -P for a drop
      }
    }
  }
}

// Wave-wide AND / OR of a 64-bit value and an inclusive prefix sum of an
// int, on DPP lane moves (vector ALU) and lane reads instead of LDS
// permutes. The results are exact whatever the combination order.
// DPP controls (gfx9 encoding): quad_perm [1,0,3,2] = 0xB1 and
// [2,3,0,1] = 0x4E, row_mirror 0x140, row_half_mirror 0x141,
// row_shr:n 0x110 + n, row_bcast:15 0x142, row_bcast:31 0x143.
template <bool kAnd>
__device__ inline uint32_t wave_bitop32(uint32_t v) {
  auto op = [](uint32_t a, uint32_t b) { return kAnd ? (a & b) : (a | b); };
  // every lane of a 16-lane row ends with its row's value (no lane of these
  // moves reads outside its row)
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xf, 0xf, false));
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xf, 0xf, false));
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return op(op(r0, r1), op(r2, r3));
}
__device__ inline uint64_t wave_and64(uint64_t v) {
  return ((uint64_t)wave_bitop32<true>((uint32_t)(v >> 32)) << 32) |
         wave_bitop32<true>((uint32_t)v);
}
__device__ inline uint64_t wave_or64(uint64_t v) {
  return ((uint64_t)wave_bitop32<false>((uint32_t)(v >> 32)) << 32) |
         wave_bitop32<false>((uint32_t)v);
}
// Lane l gets x_0 + ... + x_l. Row prefixes by shifts of 1, 2, 4 and 8
// lanes (a source outside the row reads 0), then lane 15 of rows 0 and 2 is
// added to rows 1 and 3, and lane 31 (the total of rows 0-1) to rows 2-3.
__device__ inline int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);
  return x;
}

template <int KPL>
struct SelKeys {  // the lane's keys (block j = lane + 64k), in registers
  uint64_t v[KPL];
  __device__ SelKeys(const uint64_t* g, int n, int lane) {
    // every load in bounds and unconditional (no per-key branch), the
    // blocks past the row's end then set to 0
#pragma unroll
    for (int k = 0; k < KPL; ++k) {
      const int j = lane + 64 * k;
      const uint64_t x = g[min(j, n - 1)];
      v[k] = j < n ? x : 0ull;
    }
  }
  __device__ uint64_t operator()(int k) const { return v[k]; }
};
template <>
struct SelKeys<0> {  // long rows: the keys are read from LDS as needed
  const uint64_t* g;
  int lane;
  __device__ SelKeys(const uint64_t* g_, int, int lane_) : g(g_), lane(lane_) {}
  __device__ uint64_t operator()(int k) const { return g[lane + 64 * k]; }
};

// Exact top-m of one row's gains within one wave. Lane l owns key blocks
// j = l + 64k; bit k of `member` marks membership (members have j < n).
// Returns the selected elements of this lane as a bitmask over k. Radix
// select on 8-bit digits. The first digit is taken just below the bits that
// every member shares (the leading bits of the gains are mostly equal), so
// its histogram counts spread over many bins; each later pass takes the next
// 8 bits down, since the keys still in play share every bit above them. The
// per-key update loop is branch-free (integer arithmetic on the membership
// bits), and the wave-wide AND / OR runs once per select, not once per pass.
// KPL > 0: the lane's KPL >= ceil(n / 64) keys are in registers; KPL = 0: up
// to 64 per lane, read from LDS.
template <int KPL>
__device__ __attribute__((always_inline)) uint64_t wave_select(const SelKeys<KPL>& key,
                                                              uint64_t member, int n, int m,
                                uint32_t* __restrict__ whist) {
  const int lane = threadIdx.x & 63;
  if (m <= 0) return 0;
  // keys per lane: KPL, or the row's 64-block words when they are in LDS
  const int kK = KPL > 0 ? KPL : (n + 63) >> 6;
  constexpr int kU = KPL > 0 ? KPL : 4;  // unroll factor of the per-key loops
  // per-lane membership masks over k: 32 bits hold up to 32 keys per lane
  using Mask = typename std::conditional<(KPL > 0 && KPL <= 32), uint32_t, uint64_t>::type;
  Mask selected = 0, inplay = (Mask)member;
  int need = m;
  // AND and OR of the members' keys: their XOR marks the bits that differ
  uint64_t all1 = ~0ull, any1 = 0ull;
#pragma unroll kU
  for (int k = 0; k < kK; ++k) {
    const uint64_t kv = key(k);
    const bool in = (inplay >> k) & 1u;
    all1 &= in ? kv : ~0ull;
    any1 |= in ? kv : 0ull;
  }
  const uint64_t diff = wave_and64(all1) ^ wave_or64(any1);
  if (diff != 0ull) {
    const int top = 63 - __clzll((long long)diff);
    // digit [shift, shift + 8): every key in play shares the bits above it
    int shift = top >= 7 ? top - 7 : 0;
    for (;;) {
      for (int b = lane; b < 256; b += 64) whist[b] = 0u;
      wave_lds_sync();
#pragma unroll kU
      for (int k = 0; k < kK; ++k)
        if ((inplay >> k) & 1u) atomicAdd(&whist[(uint32_t)(key(k) >> shift) & 255u], 1u);
      wave_lds_sync();
      int c[4];
      int s = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = (int)whist[255 - 4 * lane - q];
        s += c[q];
      }
      const int x = wave_incl_scan(s);
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
      // exactly one lane finds the digit (the counts rise along the lanes)
      const int src = __ffsll((unsigned long long)__ballot(found)) - 1;
      dsel = __shfl(dsel, src, 64);
      above = __shfl(above, src, 64);
      atd = __shfl(atd, src, 64);
      wave_lds_sync();
      // keys above the chosen digit are selected; only those at it stay in
      // play (a key already out of play keeps both of its bits). The digits
      // are formed again rather than kept from the histogram loop (the shift
      // passes through readfirstlane, so the compiler does not hold 17 or 34
      // of them live), and the comparisons are integer arithmetic on values
      // below 256, so no lane masks pile up in scalar registers.
      const int sh = __builtin_amdgcn_readfirstlane(shift);
      const uint32_t ds = (uint32_t)dsel;
#pragma unroll kU
      for (int k = 0; k < kK; ++k) {
        const uint32_t dig = (uint32_t)(key(k) >> sh) & 255u;
        const Mask in = (inplay >> k) & 1u;
        const Mask gt = (Mask)((ds - dig) >> 31);         // dig > dsel
        const Mask ne = (Mask)(((dig ^ ds) + 255u) >> 8);  // dig != dsel
        selected |= (gt & in) << k;
        inplay &= ~(ne << k);
      }
      need -= above;
      if (atd == need) return (uint64_t)(selected | inplay);
      if (shift == 0) break;  // every bit decided: the keys in play are equal
      shift = shift >= 8 ? shift - 8 : 0;
    }
  }
  // equal keys remain: take the lowest `need` block indices (k-major order)
  const uint64_t below = (1ull << lane) - 1ull;
  int taken = 0;
  for (int k = 0, j0 = 0; j0 < n; ++k, j0 += 64) {
    const bool b = (inplay >> k) & 1u;
    const uint64_t mask = __ballot(b);
    if (b && taken + __popcll(mask & below) < need) selected |= (Mask)1 << k;
    taken += __popcll(mask);
  }
  return (uint64_t)selected;
}

}  // namespace ress
