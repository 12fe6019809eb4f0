// Drop-set refinement with every round on chip ("ReSS: Residual-Restoring
// Sparse Attention for 3D Vision Transformers", §4.3 "Iterative Residual
// Restoration", Eq. 10-17, and Appendix E "Fused Kernel Implementation").
//
// Rows (head h, query block i) are independent across rounds, so one
// workgroup can take a tile of kRows consecutive rows of one head through
// the whole refinement: the starting state from the top-k lists, every
// round, and the final keep lists. Nothing but the lists and J goes back to
// HBM; the gains, the current and best drop sets and the per-row state stay
// in LDS and registers. One wave owns one row for the per-row steps.
// Per round:
//   * gains: C[r][j] = u_r . V_j for the tile's rows r and all key blocks j,
//     with u_r = M g_r, on the float64 matrix cores (v_mfma_f64_16x16x4f64,
//     the tile's 16 rows against 16 key blocks per instruction group, dims
//     in the same order as the per-round kernels), each wave taking every
//     16th group of key blocks; the epilogue turns each product into the
//     exact objective decrease of Eq. 16 and stores its 64-bit order key in
//     LDS;
//   * select: the row's wave selects the m_r best restores and the m_r best
//     drops (exact radix select, ties to the lower block index), moves g and
//     K by the swapped blocks in ascending block order (Eq. 13), recomputes
//     G = g^T M g and J = G / K^2 (Eq. 12) and keeps the set with the
//     smallest J seen.
// Every step repeats the arithmetic of the per-round kernels in the same
// order, so the two paths give identical bits. The gains of a row must fit
// in LDS: n_k <= 1088 key blocks.
//
// On the MI355X this path is slower than the per-round kernels (about
// 1.7 ms against 1.07 ms for 16 heads x 1074 rows x 1074 blocks, 3 rounds): the
// 159 KB of LDS a tile needs leaves one workgroup per CU, so its
// latency-bound per-row steps (the selects, the gathers of the swapped
// blocks) run with nothing to overlap them, while the per-round kernels
// keep many workgroups in flight on every CU. It stays as the workspace-free
// form of the refinement.
#include "ress_internal.h"
#include "refine_common.h"

namespace ress {
namespace {

constexpr int kRows = 16;               // rows per workgroup = waves
constexpr int kFThreads = 64 * kRows;
constexpr int kMaxWords = 17;           // 64-block words per row: n_k <= 1088
constexpr int kSlotBytes = 1024;        // per-wave scratch
// LDS strides padded off multiples of 64 banks: the 16 rows' u vectors (read
// together as matrix operands) and the gains rows (stored four rows at a
// time) then spread over all banks
constexpr int kSlotStride = kSlotBytes + 16;
__host__ __device__ inline int gains_stride(int KW) { return 64 * KW + 16; }  // uint64 words
constexpr int kChgCap = 128;            // change-list entries per flush

typedef double f64x4 __attribute__((ext_vector_type(4)));

// Row scalars read by every wave in the gains epilogue.
struct FusedRow {
  double K, G, J, vu;
};

// LDS layout for KW = ceil(n / 64) words per row, every region 16-byte
// aligned (about 159 KB at KW = 17).
struct FusedLds {
  size_t gains, cur, best, cand, slot, rs, total;
  static __host__ __device__ size_t a16(size_t b) { return (b + 15) & ~(size_t)15; }
  explicit __host__ __device__ FusedLds(int KW) {
    size_t off = 0;
    gains = off; off += a16((size_t)kRows * gains_stride(KW) * 8);  // order keys [kRows][64 KW]
    cur = off;   off += a16((size_t)kRows * KW * 8);  // D bitmask: bit l of word k = block 64k+l
    best = off;  off += a16((size_t)kRows * KW * 8);  // best D bitmask
    cand = off;  off += a16((size_t)KW * 8);          // candidates: not always kept, j < n
    slot = off;  off += (size_t)kRows * kSlotStride;  // per wave: u or g [64] | histogram, changes
    rs = off;    off += (size_t)kRows * sizeof(FusedRow);
    total = off;
  }
};

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
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int q = min(q0 + t, nchg - 1);
      ev[t] = chg[q];
      const int j = (ev[t] > 0 ? ev[t] : -ev[t]) - 1;
      pv[t] = Prow[j];
      vv[t] = Vh[(size_t)j * kD + d];
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (q0 + t >= nchg) break;
      const double dj = pv[t] * (vod - vv[t]);
      g = (ev[t] > 0) ? g + dj : g - dj;
      mag += fabs(dj);
      dk = (ev[t] > 0) ? dk - pv[t] : dk + pv[t];  // K: +P for a restore, -P for a drop
    }
  }
}

__global__ __launch_bounds__(kFThreads) void refine_fused_kernel(
    const double* __restrict__ P, const double* __restrict__ key,
    const double* __restrict__ vpool, const double* __restrict__ vout,
    const double* __restrict__ M, int nq, int n, SelConfig cfg, int rounds, double rho,
    double eps, int k_max, int32_t* __restrict__ kept_idx, int32_t* __restrict__ kept_cnt,
    double* __restrict__ J_init, double* __restrict__ J_final) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int KW = (n + 63) >> 6;
  const FusedLds L(KW);
  uint64_t* gains = reinterpret_cast<uint64_t*>(smem + L.gains);
  uint64_t* curw = reinterpret_cast<uint64_t*>(smem + L.cur);
  uint64_t* bestw = reinterpret_cast<uint64_t*>(smem + L.best);
  FusedRow* rs = reinterpret_cast<FusedRow*>(smem + L.rs);
  uint64_t* candw = reinterpret_cast<uint64_t*>(smem + L.cand);

  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.y;
  const int i0 = blockIdx.x * kRows;
  const int i = i0 + w;  // this wave's row
  const bool live = i < nq;
  const size_t row = (size_t)h * nq + (live ? i : nq - 1);
  const double* Prow = P + row * n;
  const double* Vh = vpool + (size_t)h * n * kD;
  const double* Mh = M ? M + (size_t)h * kD * kD : nullptr;
  unsigned char* slot = smem + L.slot + (size_t)w * kSlotStride;
  double* ul = reinterpret_cast<double*>(slot);                 // u or g of this row [64]
  uint32_t* whist = reinterpret_cast<uint32_t*>(slot);          // histogram [256]
  int32_t* chg = reinterpret_cast<int32_t*>(slot + 512);        // changes [kChgCap]
  uint64_t* myg = gains + (size_t)w * gains_stride(KW);
  uint64_t* mycur = curw + (size_t)w * KW;
  uint64_t* mybest = bestw + (size_t)w * KW;
  const uint64_t below = (1ull << lane) - 1ull;
  const int d = lane;

  for (int k = threadIdx.x; k < KW; k += kFThreads) {
    const int left = n - 64 * k;
    candw[k] = ~cfg.always_bits[k] & (left >= 64 ? ~0ull : ((1ull << left) - 1ull));
  }
  __syncthreads();

  // ---- starting state (the arithmetic of the per-round path's init)
  double g = 0.0, vod = 0.0, Jbest = 0.0, J0 = 0.0, Kc = 1.0;
  int nD = 0, nS = 0;
  if (live) {
    // scratch in this row's gains area: byte flags [fs], then the kept
    // blocks ascending from the front of a list of n, the dropped ones
    // ascending from its back (as the per-round path's init)
    uint8_t* flags = reinterpret_cast<uint8_t*>(myg);
    int32_t* slist = reinterpret_cast<int32_t*>(flags + flag_stride(n));
    for (int j = lane; j < n; j += 64) flags[j] = sel_always(cfg, j) ? 0 : 1;
    wave_lds_sync();
    int cnt = kept_cnt[row];
    cnt = cnt < 0 ? 0 : (cnt > k_max ? k_max : cnt);
    for (int q = lane; q < cnt; q += 64) {
      const int j = kept_idx[row * k_max + q];
      if (j >= 0 && j < n) flags[j] = 0;
    }
    wave_lds_sync();
    double ks = 0.0;
    int pos = 0, dpos = 0;
    for (int k = 0, j0 = 0; j0 < n; ++k, j0 += 64) {
      const int j = j0 + lane;
      const bool in = j < n;
      const uint8_t f = in ? flags[j] : 0;
      const bool inD = in && f != 0, kept = in && f == 0;
      if (inD) ks += Prow[j];
      nD += inD;
      nS += kept && !sel_always(cfg, j);
      const uint64_t dm = __ballot(inD);
      if (lane == 0) {
        mycur[k] = dm;
        mybest[k] = dm;
      }
      const uint64_t msk = __ballot(kept);
      if (kept) slist[pos + __popcll(msk & below)] = j;
      pos += __popcll(msk);
      if (inD) slist[n - 1 - (dpos + __popcll(dm & below))] = j;
      dpos += __popcll(dm);
    }
    Kc = 1.0 - wave_sum64(ks);
    nD = wave_isum64(nD);
    nS = wave_isum64(nS);
    wave_lds_sync();
    vod = vout[row * kD + d];
    double acc = 0.0;
    // g over whichever of D and S has fewer blocks (Eq. 10 over D; over S
    // by the zero total), ascending; batches of 16 blocks, all loads of a
    // batch issued before its sums, which keep the order
    const bool overD = dpos < pos;
    const int len = overD ? dpos : pos;
    for (int q0 = 0; q0 < len; q0 += 16) {
      double pv[16], vv[16];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int qq = min(q0 + t, len - 1);
        const int j = slist[overD ? n - 1 - qq : qq];
        pv[t] = Prow[j];
        vv[t] = Vh[(size_t)j * kD + d];
      }
#pragma unroll
      for (int t = 0; t < 16; ++t)
        if (q0 + t < len) acc += overD ? pv[t] * (vod - vv[t]) : pv[t] * (vv[t] - vod);
    }
    g = acc;  // an empty D: the empty sum of Eq. 10
    ul[d] = g;
    wave_lds_sync();
    double G, vu;
    const double u = gram_apply(Mh, ul, g, vod, &G, &vu);
    const double J = (Kc > 0.0) ? G / (Kc * Kc) : INFINITY;
    J0 = J;
    Jbest = J;
    wave_lds_sync();
    ul[d] = u;
    if (lane == 0) rs[w] = FusedRow{Kc, G, J, vu};
  } else {
    ul[d] = 0.0;  // finite operands for the rows past the last one
    if (lane == 0) rs[w] = FusedRow{1.0, 0.0, 0.0, 0.0};
  }

  // ---- rounds
  const int q4 = lane >> 4, c16 = lane & 15;
  const int n_tiles = (n + 15) >> 4;
  for (int r = 0; r < rounds; ++r) {
    const int m_base = swaps_of(cfg, h, r, rho);
    if (m_base <= 0) continue;  // no swaps for this head in this round
    __syncthreads();            // u and the row scalars of every row are in LDS

    // gains of the tile's rows: A = u (row c16, dims 4s + q4), B = V
    // (block 16t + c16, dims 4s + q4); result rows q4 + 4e, block 16t + c16
    const double* ur = reinterpret_cast<const double*>(smem + L.slot + (size_t)c16 * kSlotStride);
    for (int t = w; t < n_tiles; t += kRows) {
      const int j = 16 * t + c16;
      const int jc = min(j, n - 1);
      const double* vr = Vh + (size_t)jc * kD;
      f64x4 acc = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        double b[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) b[s] = vr[4 * (8 * hf + s) + q4];
#pragma unroll
        for (int s = 0; s < 8; ++s)
          acc = __builtin_amdgcn_mfma_f64_16x16x4f64(ur[4 * (8 * hf + s) + q4], b[s], acc, 0, 0, 0);
      }
      double pv[4], kv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = min(i0 + q4 + 4 * e, nq - 1);
        const size_t rw = (size_t)h * nq + rr;
        pv[e] = P[rw * n + jc];
        kv[e] = key[rw * n + jc];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rl = q4 + 4 * e;  // row within the tile
        const FusedRow st = rs[rl];
        const double p = pv[e];
        const double sv = kv[e] * fmax(1.0 - p, eps);  // s_ij (Eq. 6)
        const double s2 = sv * sv;
        const double dMg = p * (st.vu - acc[e]);  // d_j^T M g_i
        const bool inD = (curw[(size_t)rl * KW + (jc >> 6)] >> (jc & 63)) & 1ull;
        double dJ;
        if (inD) {  // restore (Eq. 13-14), u = +P_j
          const double dG = -2.0 * dMg + s2;
          const double Ku = st.K + p;
          dJ = st.J - (st.G + dG) / (Ku * Ku);
        } else {  // drop (Eq. 15), u = -P_j
          const double dG = 2.0 * dMg + s2;
          const double Ku = st.K - p;
          dJ = (Ku > 0.0) ? st.J - (st.G + dG) / (Ku * Ku) : -INFINITY;
        }
        if (i0 + rl < nq && j < n) gains[(size_t)rl * gains_stride(KW) + j] = order_key(dJ);
      }
    }
    __syncthreads();  // every gain of the tile is in LDS

    if (live) {
      const int m = min(m_base, min(nD, nS));
      uint64_t restore = 0, drop = 0;
      if (m > 0) {
        const SelKeys<0> keys(myg, n, lane);
        // D is a subset of the candidates; the kept candidates are the rest
        uint64_t memD = 0, memS = 0;
#pragma nounroll
        for (int k = 0; k < KW; ++k) {
          const uint64_t dw = mycur[k], cw = candw[k];
          memD |= ((dw >> lane) & 1ull) << k;
          memS |= (((cw & ~dw) >> lane) & 1ull) << k;
        }
        restore = wave_select<0>(keys, memD, n, m, whist);
        drop = wave_select<0>(keys, memS, n, m, whist);
      }
      wave_lds_sync();  // the histogram area becomes the change list
      // changes in ascending block order, flushed kChgCap at a time; the
      // drop set loses the restores and gains the drops
      double dk = 0.0;
      double mag = fabs(g);  // what g is formed from, for the cancellation guard
      int nchg = 0;
      for (int k = 0; k < KW; ++k) {
        const bool rb = (restore >> k) & 1ull, db = (drop >> k) & 1ull;
        const uint64_t rm = __ballot(rb), dm = __ballot(db);
        const uint64_t msk = rm | dm;
        if (msk == 0ull) continue;
        if (nchg + __popcll(msk) > kChgCap) {
          wave_lds_sync();
          apply_changes(chg, nchg, Prow, Vh, vod, g, mag, dk);
          wave_lds_sync();
          nchg = 0;
        }
        const int j = 64 * k + lane;
        if (rb || db) chg[nchg + __popcll(msk & below)] = db ? (j + 1) : -(j + 1);
        nchg += __popcll(msk);
        if (lane == 0) mycur[k] = (mycur[k] & ~rm) | dm;
      }
      wave_lds_sync();
      apply_changes(chg, nchg, Prow, Vh, vod, g, mag, dk);
      if (g_cancelled(g, mag))
        g = g_from_sets([&](int j) { return ((mycur[j >> 6] >> (j & 63)) & 1ull) != 0; }, n, nD,
                        Prow, Vh, vod);
      if (m > 0) {
        wave_lds_sync();
        ul[d] = g;
        wave_lds_sync();
        double G, vu;
        const double u = gram_apply(Mh, ul, g, vod, &G, &vu);
        Kc += dk;
        const double J = (Kc > 0.0) ? G / (Kc * Kc) : INFINITY;
        if (J < Jbest) {  // track-best, strict
          Jbest = J;
          for (int k = lane; k < KW; k += 64) mybest[k] = mycur[k];
        }
        wave_lds_sync();
        ul[d] = u;
        if (lane == 0) rs[w] = FusedRow{Kc, G, J, vu};
      }
      // m = 0: no swap, the row (and its u, which no histogram overwrote)
      // stays as it was
    }
  }
  __syncthreads();

  // ---- the best sets as keep lists, ascending, -1 padded
  if (live) {
    int32_t* out = kept_idx + row * k_max;
    int pos = 0;
    for (int k = 0, j0 = 0; j0 < n; ++k, j0 += 64) {
      const int j = j0 + lane;
      const bool kept = j < n && (sel_always(cfg, j) || !((mybest[k] >> lane) & 1ull));
      const uint64_t msk = __ballot(kept);
      const int p = pos + __popcll(msk & below);
      if (kept && p < k_max) out[p] = j;
      pos += __popcll(msk);
    }
    for (int p = pos + lane; p < k_max; p += 64) out[p] = -1;
    if (lane == 0) {
      kept_cnt[row] = pos < k_max ? pos : k_max;
      if (J_init) J_init[row] = J0;
      if (J_final) J_final[row] = Jbest;
    }
  }
}

}  // namespace

int refine_fused_max_blocks() { return 64 * kMaxWords; }

hipError_t launch_refine_fused(const double* P, const double* key, const double* vpool,
                               const double* vout, const double* M, const ress_shape& s,
                               const SelConfig& cfg, int32_t rounds, double rho, double eps,
                               int32_t k_max, int32_t* kept_idx, int32_t* kept_cnt,
                               double* J_init, double* J_final, hipStream_t st) {
  const int nq = n_qblocks(s), n = n_kblocks(s);
  const size_t lds = FusedLds((n + 63) >> 6).total;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&refine_fused_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(refine_fused_kernel, dim3((nq + kRows - 1) / kRows, s.H), dim3(kFThreads),
                     lds, st, P, key, vpool, vout, M, nq, n, cfg, rounds, rho, eps, k_max,
                     kept_idx, kept_cnt, J_init, J_final);
  return hipGetLastError();
}

}  // namespace ress
