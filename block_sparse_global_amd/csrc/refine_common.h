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

// Bitwise AND / OR of a 64-bit value over the wave.
__device__ inline uint64_t wave_and64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v &= (uint64_t)__shfl_xor((long long)v, o, 64);
  return v;
}
__device__ inline uint64_t wave_or64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v |= (uint64_t)__shfl_xor((long long)v, o, 64);
  return v;
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
// select on 8-bit digits; each pass first finds the bits that every key
// still in play shares and takes its digit just below that common prefix,
// so no pass is spent on digits that cannot separate the keys (the leading
// bits of the gains are mostly equal) and the histogram counts spread over
// many bins. KPL > 0: the lane's KPL >= ceil(n / 64) keys are in registers;
// KPL = 0: up to 64 per lane, read from LDS.
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
  // AND and OR of the keys in play; each pass's update loop forms those of
  // the next pass
  uint64_t all1 = ~0ull, any1 = 0ull;
#pragma unroll kU
  for (int k = 0; k < kK; ++k)
    if ((inplay >> k) & 1u) {
      all1 &= key(k);
      any1 |= key(k);
    }
  for (;;) {
    const uint64_t diff = wave_and64(all1) ^ wave_or64(any1);
    if (diff == 0ull) break;  // the keys in play are all equal
    const int top = 63 - __clzll((long long)diff);
    const int shift = top >= 7 ? top - 7 : 0;
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
    all1 = ~0ull;
    any1 = 0ull;
#pragma unroll kU
    for (int k = 0; k < kK; ++k) {
      if ((inplay >> k) & 1u) {
        const uint64_t kv = key(k);
        const int dig = (int)((uint32_t)(kv >> shift) & 255u);
        if (dig > dsel) selected |= (Mask)1 << k;
        if (dig != dsel) {
          inplay &= ~((Mask)1 << k);
        } else {
          all1 &= kv;
          any1 |= kv;
        }
      }
    }
    need -= above;
    if (atd == need) return (uint64_t)(selected | inplay);
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
