// Per-row top-k keep sets.
//
// Top-k ("ReSS: Residual-Restoring Sparse Attention for 3D Vision
// Transformers", §3 step (2), §4.1 Eq. 2, §4.4): per (head, query-block
// row), keep the c_h candidates with the largest key plus every always-kept
// block.
// One workgroup owns one row (workgroup (i, h): query-block row i of head
// h, gridDim.x = n_q rows per head, n key blocks per row); thread t owns the
// E consecutive key blocks [t*E, t*E + E). Selection is exact: an MSB-first radix select over 64-bit
// keys whose unsigned order equals the float64 order, with ties among equal
// keys broken towards the lower block index by a block-wide prefix count.
// No float atomics and fixed-order reductions: results are bit-reproducible.
//
// Cumulative-probability ("CDF", top-p) selection, the probability criterion
// the ReSS page compares against (its related-work section on SparseVGGT's
// top-k and top-p selection, §4.4 and Table 2 "+ CDF threshold"; Appendix F
// two-block floor and sink rule): the always-kept blocks' mass first, then
// candidates by probability descending until the mass reaches tau, at most
// c_h of them, at least enough for two kept blocks. The same radix select
// first finds the c_h best candidates; they are ranked exactly and one lane
// accumulates their probabilities in rank order, one float64 addition at a
// time, so the count matches a sequential scan bit for bit.
#include "ress_internal.h"
#include "refine_common.h"

namespace ress {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
struct SelShared {
  uint32_t hist[256];
  int32_t wave_tot[kWaves];
  double red[kWaves];
  uint64_t and_[kWaves], or_[kWaves];
  int32_t digit, above, at_digit;
};

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
  for (;;) {
    // the bits every key still in play shares: the digit of this pass is
    // the 8 bits just below that common prefix, so no pass is spent on
    // digits that cannot separate the keys (the leading bits of float64
    // keys in a narrow range are all equal)
    uint64_t all1 = ~0ull, any1 = 0ull;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((inplay >> e) & 1u) {
        all1 &= u[e];
        any1 |= u[e];
      }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      all1 &= (uint64_t)__shfl_xor((long long)all1, o, 64);
      any1 |= (uint64_t)__shfl_xor((long long)any1, o, 64);
    }
    if ((t & 63) == 0) {
      sh.and_[t >> 6] = all1;
      sh.or_[t >> 6] = any1;
    }
    for (int k = t; k < 256; k += kThreads) sh.hist[k] = 0u;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
      all1 &= sh.and_[k];
      any1 |= sh.or_[k];
    }
    const uint64_t diff = all1 ^ any1;
    if (diff == 0ull) break;  // the keys in play are all equal
    const int top = 63 - __clzll((long long)diff);
    const int shift = top >= 7 ? top - 7 : 0;
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
  const double* row = key + ((size_t)h * gridDim.x + i) * n;
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
  const size_t r = (size_t)h * gridDim.x + i;
  write_kept<E>(sel | always, n, k_max, kept_idx + r * k_max, kept_cnt + r,
                sh);
}

// One wave per row, four rows per workgroup, for rows of at most 64 KPL key
// blocks: the row's keys as order keys in registers (block j = lane + 64k),
// the exact per-wave radix select of the refinement (same tie rule: the
// lower block index), no workgroup barriers. The keep list is the same as
// topk_kernel's.
template <int KPL>
__global__ __launch_bounds__(256) void topk_wave_kernel(
    const double* __restrict__ key, int nq, int n, SelConfig cfg, int k_max,
    int32_t* __restrict__ kept_idx, int32_t* __restrict__ kept_cnt) {
  __shared__ uint32_t whist[4][256];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + w;
  const int h = blockIdx.y;
  if (i >= nq) return;  // whole wave; nothing below waits on other waves
  const size_t row = (size_t)h * nq + i;
  SelKeys<KPL> keys(reinterpret_cast<const uint64_t*>(key + row * n), n, lane);
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
  const int c = cfg.keep[h] - cfg.n_always;
  const uint64_t kept = wave_select<KPL>(keys, member, n, c, whist[w]) | always;
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

// float64 value of an order key (inverse of order_key)
__device__ inline double order_key_value(uint64_t k) {
  const uint64_t b = (k >> 63) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
  return __longlong_as_double((long long)b);
}

// Dynamic LDS of cdf_kernel for up to `cap` selected candidates: their order
// keys, their probabilities in rank order and their ranks.
__host__ __device__ inline size_t cdf_smem_bytes(int cap) {
  return (size_t)cap * (sizeof(uint64_t) + sizeof(double) + sizeof(int32_t));
}

template <int E>
__global__ __launch_bounds__(kThreads) void cdf_kernel(
    const double* __restrict__ P, int n, SelConfig cfg, double tau, int cap,
    int k_max, int32_t* __restrict__ kept_idx, int32_t* __restrict__ kept_cnt) {
  extern __shared__ __attribute__((aligned(16))) unsigned char cdf_smem[];
  uint64_t* ck = reinterpret_cast<uint64_t*>(cdf_smem);  // [cap] keys, block order
  double* sp = reinterpret_cast<double*>(ck + cap);       // [cap] P in rank order
  int32_t* rk = reinterpret_cast<int32_t*>(sp + cap);     // [cap] rank of ck[a]
  __shared__ SelShared sh;
  __shared__ int s_taken;
  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int t = threadIdx.x;
  const double* row = P + ((size_t)h * gridDim.x + i) * n;
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
  // the c best candidates, compacted in ascending block order
  int total;
  const int pos = block_exclusive_scan(__popc(sel), sh, &total);
  {
    int p = pos;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((sel >> e) & 1u) ck[p++] = u[e];
  }
  __syncthreads();
  // rank by probability descending; equal probabilities by block index,
  // which is the compacted position
  for (int a = t; a < c; a += kThreads) {
    const uint64_t ka = ck[a];
    int r = 0;
    for (int b = 0; b < c; ++b) {
      const uint64_t kb = ck[b];
      r += (kb > ka) || (kb == ka && b < a);
    }
    rk[a] = r;
    sp[r] = order_key_value(ka);
  }
  __syncthreads();
  if (t == 0) {
    double s = 0.0;
    for (int wd = 0; wd * 64 < n; ++wd) {
      uint64_t bits = cfg.always_bits[wd];
      while (bits != 0) {
        const int j = wd * 64 + __builtin_ctzll(bits);
        bits &= bits - 1;
        if (j < n) s += row[j];
      }
    }
    int m = 0;
    while (s < tau && m < c) s += sp[m++];
    m = max(m, 2 - cfg.n_always);
    s_taken = min(m, c);
  }
  __syncthreads();
  const int taken = s_taken;
  uint32_t kept = always;
  {
    int p = pos;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if ((sel >> e) & 1u) {
        if (rk[p] < taken) kept |= 1u << e;
        ++p;
      }
  }
  const size_t r = (size_t)h * gridDim.x + i;
  write_kept<E>(kept, n, k_max, kept_idx + r * k_max, kept_cnt + r, sh);
}

int pick_e(int n) {
  const int need = (n + kThreads - 1) / kThreads;
  int e = 1;
  while (e < need) e <<= 1;
  return e;
}

// LDS of one wave of cdf_wave_kernel: the radix histogram, then the
// candidate tables, rounded up to 16 bytes so that every wave's tables stay
// 8-byte aligned.
__host__ __device__ inline size_t cdf_wave_stride(int cap) {
  return (1024 + cdf_smem_bytes(cap) + 15) & ~(size_t)15;
}

// The cumulative threshold with one wave per row, four rows per workgroup,
// for rows of at most 64 KPL key blocks: the c_h best candidates by the
// per-wave radix select, compacted in ascending block order into the wave's
// LDS, ranked exactly by (P descending, index ascending), and one lane adds
// the always-kept mass and then the ranked probabilities, in the same order
// and with the same float64 additions as cdf_kernel, so the counts agree.
template <int KPL>
__global__ __launch_bounds__(256) void cdf_wave_kernel(
    const double* __restrict__ P, int nq, int n, SelConfig cfg, double tau, int cap,
    int k_max, int32_t* __restrict__ kept_idx, int32_t* __restrict__ kept_cnt) {
  extern __shared__ __attribute__((aligned(16))) unsigned char cdf_smem[];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  unsigned char* mine = cdf_smem + (size_t)w * cdf_wave_stride(cap);
  uint32_t* whist = reinterpret_cast<uint32_t*>(mine);                  // [256]
  uint64_t* ck = reinterpret_cast<uint64_t*>(mine + 1024);              // [cap] keys, block order
  double* sp = reinterpret_cast<double*>(ck + cap);                     // [cap] P in rank order
  int32_t* rk = reinterpret_cast<int32_t*>(sp + cap);                   // [cap] rank of ck[a]
  const int i = blockIdx.x * 4 + w;
  const int h = blockIdx.y;
  if (i >= nq) return;  // whole wave; nothing below waits on other waves
  const size_t row = (size_t)h * nq + i;
  const double* prow = P + row * n;
  SelKeys<KPL> keys(reinterpret_cast<const uint64_t*>(prow), n, lane);
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
  const int c = cfg.keep[h] - cfg.n_always;
  const uint64_t sel = wave_select<KPL>(keys, member, n, c, whist);
  // the c best candidates, compacted in ascending block order
  const uint64_t below = (1ull << lane) - 1ull;
  int pos = 0;
#pragma unroll
  for (int k = 0; k < KPL; ++k) {
    const bool b = (sel >> k) & 1ull;
    const uint64_t msk = __ballot(b);
    if (b) ck[pos + __popcll(msk & below)] = keys.v[k];
    pos += __popcll(msk);
  }
  wave_lds_sync();
  // rank by probability descending; equal probabilities by block index,
  // which is the compacted position
  for (int a = lane; a < c; a += 64) {
    const uint64_t ka = ck[a];
    int r = 0;
    for (int b = 0; b < c; ++b) {
      const uint64_t kb = ck[b];
      r += (kb > ka) || (kb == ka && b < a);
    }
    rk[a] = r;
    sp[r] = order_key_value(ka);
  }
  wave_lds_sync();
  int taken = 0;
  if (lane == 0) {
    double s = 0.0;
    for (int wd = 0; wd * 64 < n; ++wd) {
      uint64_t bits = cfg.always_bits[wd];
      while (bits != 0) {
        const int j = wd * 64 + __builtin_ctzll(bits);
        bits &= bits - 1;
        if (j < n) s += prow[j];
      }
    }
    int m = 0;
    while (s < tau && m < c) s += sp[m++];
    m = max(m, 2 - cfg.n_always);
    taken = min(m, c);
  }
  taken = __shfl(taken, 0, 64);
  uint64_t kept = always;
  pos = 0;
#pragma unroll
  for (int k = 0; k < KPL; ++k) {
    const bool b = (sel >> k) & 1ull;
    const uint64_t msk = __ballot(b);
    if (b && rk[pos + __popcll(msk & below)] < taken) kept |= 1ull << k;
    pos += __popcll(msk);
  }
  int32_t* out = kept_idx + row * k_max;
  pos = 0;
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

template <int KPL>
hipError_t launch_cdf_wave(const double* P, int nq, int n, int H, const SelConfig& cfg,
                           double tau, int cap, int32_t k_max, int32_t* kept_idx,
                           int32_t* kept_cnt, hipStream_t st) {
  const size_t smem = 4 * cdf_wave_stride(cap);
  if (smem > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&cdf_wave_kernel<KPL>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((cdf_wave_kernel<KPL>), dim3((nq + 3) / 4, H), dim3(256), smem, st, P, nq,
                     n, cfg, tau, cap, k_max, kept_idx, kept_cnt);
  return hipGetLastError();
}

template <int E>
hipError_t launch_cdf_e(const double* P, int nq, int n, int H, const SelConfig& cfg,
                        double tau, int cap, int32_t k_max, int32_t* kept_idx,
                        int32_t* kept_cnt, hipStream_t st) {
  const size_t smem = cdf_smem_bytes(cap);
  if (smem > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&cdf_kernel<E>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((cdf_kernel<E>), dim3(nq, H), dim3(kThreads), smem, st, P, n,
                     cfg, tau, cap, k_max, kept_idx, kept_cnt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cdf(const double* P, const ress_shape& s, const SelConfig& cfg,
                      double tau, int32_t k_max, int32_t* kept_idx,
                      int32_t* kept_cnt, hipStream_t st) {
  const int nq = n_qblocks(s), n = n_kblocks(s);
  int cap = 1;
  for (int h = 0; h < s.H; ++h) cap = max(cap, cfg.keep[h] - cfg.n_always);
  // one wave per row for long rows and small budgets (the rank count costs
  // a single wave c^2/64 comparisons per lane, against c^2/256 with four)
  if (n > 512 && cap <= 256 && 4 * cdf_wave_stride(cap) <= 160 * 1024) {
    if (n <= 64 * 17)
      return launch_cdf_wave<17>(P, nq, n, s.H, cfg, tau, cap, k_max, kept_idx, kept_cnt, st);
    if (n <= 64 * 34)
      return launch_cdf_wave<34>(P, nq, n, s.H, cfg, tau, cap, k_max, kept_idx, kept_cnt, st);
  }
  switch (pick_e(n)) {
    case 1: return launch_cdf_e<1>(P, nq, n, s.H, cfg, tau, cap, k_max, kept_idx, kept_cnt, st);
    case 2: return launch_cdf_e<2>(P, nq, n, s.H, cfg, tau, cap, k_max, kept_idx, kept_cnt, st);
    case 4: return launch_cdf_e<4>(P, nq, n, s.H, cfg, tau, cap, k_max, kept_idx, kept_cnt, st);
    case 8: return launch_cdf_e<8>(P, nq, n, s.H, cfg, tau, cap, k_max, kept_idx, kept_cnt, st);
    case 16: return launch_cdf_e<16>(P, nq, n, s.H, cfg, tau, cap, k_max, kept_idx, kept_cnt, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_topk(const double* key, const ress_shape& s,
                       const SelConfig& cfg, int32_t k_max, int32_t* kept_idx,
                       int32_t* kept_cnt, hipStream_t st) {
  const int n = n_kblocks(s), nq = n_qblocks(s);
  if (n <= 64 * 34) {  // one wave per row, the keys in registers
    const dim3 wgrid((nq + 3) / 4, s.H);
    if (n <= 64 * 17)
      hipLaunchKernelGGL((topk_wave_kernel<17>), wgrid, dim3(256), 0, st, key, nq, n, cfg,
                         k_max, kept_idx, kept_cnt);
    else
      hipLaunchKernelGGL((topk_wave_kernel<34>), wgrid, dim3(256), 0, st, key, nq, n, cfg,
                         k_max, kept_idx, kept_cnt);
    return hipGetLastError();
  }
  dim3 grid(nq, s.H);
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

}  // namespace ress
