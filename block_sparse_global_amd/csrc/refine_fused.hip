// Drop-set refinement with every round on chip ("ReSS: Residual-Restoring
// Sparse Attention for 3D Vision Transformers", §4.3 "Iterative Residual
// Restoration", Eq. 10-17, and Appendix E "Fused Kernel Implementation").
//
// Rows (head h, query block i) are independent across rounds, so one
// workgroup can take a tile of consecutive rows of one head through the
// whole refinement: the starting state, every round, and the final keep
// lists. Nothing but the lists and J goes back to HBM; the gains, the
// current and best drop sets and the per-row state stay in LDS and
// registers. One wave owns one row for the per-row steps.
// Per round:
//   * gains: C[r][j] = u_r . V_j for the tile's rows r and all key blocks j,
//     with u_r = M g_r, on the float64 matrix cores (v_mfma_f64_16x16x4f64,
//     16 operand rows against 16 key blocks per instruction group, dims in
//     the same order as the per-round kernels), each wave taking every
//     kRows-th group of key blocks; the epilogue turns each product into the
//     exact objective decrease of Eq. 16 and stores its 64-bit order key in
//     LDS;
//   * select: the row's wave selects the m_r best restores and the m_r best
//     drops (exact radix select, ties to the lower block index), moves g and
//     K by the swapped blocks in ascending block order (Eq. 13), recomputes
//     G = g^T M g and J = G / K^2 (Eq. 12) and keeps the set with the
//     smallest J seen.
// The gains of a row must fit in LDS: n_k <= 1088 key blocks.
//
// Two input forms:
//  * kept lists (16 rows a workgroup): the starting drop sets from the
//    top-k lists, P and the drift key read from device memory. Every step
//    repeats the arithmetic of the per-round kernels in the same order, so
//    the two paths give identical bits.
//  * pooled blocks (8 rows a workgroup): the whole selection in one pass,
//    score -> top-k -> refinement, with P and the key never written. The
//    map rows, vout, w = M vout and a = vout . w of the fused selection stay
//    in LDS beside the gains; the drift key of each (row, block), needed by
//    the top-k and by every round's gains, comes from c_rj = w_r . V_j,
//    which shares the gains product's B operand: operand rows 0-7 hold the
//    tile's u, rows 8-15 its w, so every instruction group gives both (the
//    upper half that an 8-row tile would leave idle). The top-k takes the
//    key from the same product rows, so it and the rounds see the same bits.
//
// On the MI355X both forms are slower than the split kernels (the kept-list
// form about 1.7 ms against 1.07 ms for 16 heads x 1074 rows x 1074 blocks,
// 3 rounds): the LDS a tile needs leaves one workgroup per CU, so its
// latency-bound per-row steps (the selects, the gathers of the swapped
// blocks) run with nothing to overlap them, while the per-round kernels
// keep many workgroups in flight on every CU. They stay as the
// workspace-free forms of the selection.
#include "ress_internal.h"
#include "select_fused_steps.h"

namespace ress {
namespace {

// rows per workgroup = waves: 16 from kept lists, 8 from pooled blocks (the
// map rows then share the LDS)
template <bool POOLED>
constexpr int fused_rows() { return POOLED ? 8 : 16; }
constexpr int kMaxWords = 17;           // 64-block words per row: n_k <= 1088
constexpr int kSlotBytes = 1024;        // per-wave scratch
// LDS strides padded off multiples of 64 banks: the 16 operand rows (u, and
// w in the pooled form; read together as matrix operands) and the gains rows (stored four rows at a
// time) then spread over all banks
constexpr int kSlotStride = kSlotBytes + 16;
__host__ __device__ inline int gains_stride(int KW) { return 64 * KW + 16; }  // uint64 words
constexpr int kChgCap = 128;            // change-list entries per flush

// LDS layout of a tile of `rows` rows of n key blocks (KW = ceil(n / 64)
// words per row), every region 16-byte aligned: about 159 KB for 16 rows
// from kept lists and 156 KB for 8 rows from pooled blocks at n = 1088.
struct FusedLds {
  size_t gains, cur, best, cand, slot, rs, prow, vo, wv, av, total;
  static __host__ __device__ size_t a16(size_t b) { return (b + 15) & ~(size_t)15; }
  __host__ __device__ FusedLds(int n, int rows, bool pooled) {
    const int KW = (n + 63) >> 6;
    size_t off = 0;
    // order keys [rows][64 KW]; in the pooled form first the float64 keys
    // of the top-k and, before them, the vout partial sums [2][rows][64]
    // (so at least that large on short rows)
    const size_t gbytes = (size_t)rows * gains_stride(KW) * 8;
    const size_t pbytes = pooled ? (size_t)2 * rows * kD * 8 : 0;
    gains = off; off += a16(gbytes > pbytes ? gbytes : pbytes);
    cur = off;   off += a16((size_t)rows * KW * 8);  // D bitmask: bit l of word k = block 64k+l
    best = off;  off += a16((size_t)rows * KW * 8);  // best D bitmask
    cand = off;  off += a16((size_t)KW * 8);         // candidates: not always kept, j < n
    slot = off;  off += (size_t)rows * kSlotStride;  // per wave: u or g [64] | histogram, changes
    rs = off;    off += a16((size_t)rows * sizeof(RowScalars));
    prow = vo = wv = av = off;
    if (pooled) {
      prow = off; off += a16((size_t)rows * row_stride(n) * 8);  // P [rows][ns]
      vo = off;   off += (size_t)rows * kD * 8;                   // vout [rows][64]
      wv = off;   off += (size_t)rows * kD * 8;                   // w = M vout [rows][64]
      av = off;   off += a16((size_t)rows * 8);                   // a = vout . w [rows]
    }
    total = off;
  }
};

// Products of one group of 16 key blocks (16t .. 16t + 15) with 16 operand
// rows: A = the row at ur (row c16, dims 4s + q4), B = V (block 16t + c16,
// dims 4s + q4); result element e: operand row q4 + 4e, block 16t + c16.
__device__ inline f64x4 group_product(const double* ur, const double* vr, int q4) {
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
  return acc;
}

// Inputs of one launch; the kept-list form reads P, key, vout and the lists,
// the pooled form qpool, kpool, vmv and scale instead.
struct FusedArgs {
  const double* P;
  const double* key;
  const double* vout;
  const double* qpool;
  const double* kpool;
  const double* vmv;
  const double* vpool;
  const double* M;
  int nq, n, rounds, k_max;
  double rho, eps, scale;
  int32_t* kept_idx;
  int32_t* kept_cnt;
  double* J_init;
  double* J_final;
};

template <bool POOLED>
__global__ __launch_bounds__(64 * fused_rows<POOLED>()) void refine_fused_kernel(FusedArgs A,
                                                                                 SelConfig cfg) {
  constexpr int kRows = fused_rows<POOLED>();
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int n = A.n, nq = A.nq;
  const int KW = (n + 63) >> 6;
  const int ns = row_stride(n);
  const FusedLds L(n, kRows, POOLED);
  uint64_t* gains = reinterpret_cast<uint64_t*>(smem + L.gains);
  uint64_t* curw = reinterpret_cast<uint64_t*>(smem + L.cur);
  uint64_t* bestw = reinterpret_cast<uint64_t*>(smem + L.best);
  RowScalars* rs = reinterpret_cast<RowScalars*>(smem + L.rs);
  uint64_t* candw = reinterpret_cast<uint64_t*>(smem + L.cand);
  double* prows = reinterpret_cast<double*>(smem + L.prow);  // pooled form: P [kRows][ns]
  double* vo = reinterpret_cast<double*>(smem + L.vo);
  double* wv = reinterpret_cast<double*>(smem + L.wv);
  double* av = reinterpret_cast<double*>(smem + L.av);

  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.y;
  const int i0 = blockIdx.x * kRows;
  const int i = i0 + w;  // this wave's row
  const bool live = i < nq;
  const size_t row = (size_t)h * nq + (live ? i : nq - 1);
  const double* Prow = POOLED ? prows + (size_t)w * ns : A.P + row * n;
  const double* Vh = A.vpool + (size_t)h * n * kD;
  const double* Mh = A.M ? A.M + (size_t)h * kD * kD : nullptr;
  const double* vm = POOLED ? A.vmv + (size_t)h * n : nullptr;
  unsigned char* slot = smem + L.slot + (size_t)w * kSlotStride;
  double* ul = reinterpret_cast<double*>(slot);                 // u or g of this row [64]
  uint32_t* whist = reinterpret_cast<uint32_t*>(slot);          // histogram [256]
  int32_t* chg = reinterpret_cast<int32_t*>(slot + 512);        // changes [kChgCap]
  uint64_t* myg = gains + (size_t)w * gains_stride(KW);
  uint64_t* mycur = curw + (size_t)w * KW;
  uint64_t* mybest = bestw + (size_t)w * KW;
  const uint64_t below = (1ull << lane) - 1ull;
  const int d = lane;
  const int q4 = lane >> 4, c16 = lane & 15;
  const int n_tiles = (n + 15) >> 4;
  const double eps = A.eps;

  for (int k = threadIdx.x; k < KW; k += 64 * kRows) {
    const int left = n - 64 * k;
    candw[k] = ~cfg.always_bits[k] & (left >= 64 ? ~0ull : ((1ull << left) - 1ull));
  }

  // ---- pooled form: the fused selection's map, drift terms and top-k
  uint64_t kept_bits = 0;
  if constexpr (POOLED) {
    fused_logits<kRows>(A.qpool + (size_t)h * nq * kD, A.kpool + (size_t)h * n * kD, nq, n, i0,
                        A.scale, prows, ns);
    __syncthreads();
    fused_softmax<kMaxWords>(prows + (size_t)w * ns, n, ns);
    __syncthreads();
    // the vout partial sums use the gains area, free until the keys
    fused_vout<kRows>(prows, ns, n, Vh, Mh, reinterpret_cast<double*>(gains), vo, wv, av);
    __syncthreads();
    // the key of every (row, block) into the gains area as float64, from
    // the product rows 8-15 (w, as in the rounds; rows 0-7 repeat them here)
    {
      const double* ur = wv + (size_t)(c16 & 7) * kD;
      for (int t = w; t < n_tiles; t += kRows) {
        const int j = 16 * t + c16;
        const int jc = min(j, n - 1);
        const f64x4 acc = group_product(ur, Vh + (size_t)jc * kD, q4);
        const double vmj = vm[jc];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int rl = q4 + 4 * e;
          const double kv = fused_drift_key(prows[(size_t)rl * ns + jc], acc[e + 2], av[rl], vmj, eps);
          if (j < n) reinterpret_cast<double*>(gains)[(size_t)rl * gains_stride(KW) + j] = kv;
        }
      }
    }
    __syncthreads();
    if (live)
      kept_bits = fused_topk_bits<kMaxWords>(reinterpret_cast<const double*>(myg), n, cfg,
                                             cfg.keep[h] - cfg.n_always, whist);
    wave_lds_sync();  // the keys are in registers: the row's gains area is free
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
    if constexpr (POOLED) {
      // dropped: the candidates outside the top-k
      for (int k = 0, j0 = 0; j0 < n; ++k, j0 += 64) {
        const int j = j0 + lane;
        if (j < n) flags[j] = (sel_always_wave(cfg, j) || ((kept_bits >> k) & 1ull)) ? 0 : 1;
      }
    } else {
      for (int j = lane; j < n; j += 64) flags[j] = sel_always_wave(cfg, j) ? 0 : 1;
      wave_lds_sync();
      int cnt = A.kept_cnt[row];
      cnt = cnt < 0 ? 0 : (cnt > A.k_max ? A.k_max : cnt);
      for (int q = lane; q < cnt; q += 64) {
        const int j = A.kept_idx[row * A.k_max + q];
        if (j >= 0 && j < n) flags[j] = 0;
      }
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
      nS += kept && !sel_always_wave(cfg, j);
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
    vod = POOLED ? vo[(size_t)w * kD + d] : A.vout[row * kD + d];
    double acc = 0.0;
    // g over whichever of D and S has fewer blocks (Eq. 10 over D; over S
    // by the zero total), ascending; batches of 16 blocks, all loads of a
    // batch issued before its sums, which keep the order
    const bool overD = dpos < pos;
    const int len = overD ? dpos : pos;
    for (int q0 = 0; q0 < len; q0 += 16) {
      double pv[16], vv[16];
      // lanes 0-15 read the batch's list entries in one LDS access; each
      // goes to a scalar register, so the addresses are scalar work
      const int qm = min(q0 + (lane & 15), len - 1);
      const int mine = slist[overD ? n - 1 - qm : qm];
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const int j = __builtin_amdgcn_readlane(mine, t);
        pv[t] = Prow[j];
        vv[t] = Vh[(size_t)j * kD + d];
      }
#pragma unroll
      for (int t = 0; t < 16; ++t)
        if (q0 + t < len) acc = fma(pv[t], overD ? vod - vv[t] : vv[t] - vod, acc);
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
    if (lane == 0) rs[w] = RowScalars{Kc, G, J, vu};
  } else {
    ul[d] = 0.0;  // finite operands for the rows past the last one
    for (int k = lane; k < KW; k += 64) mycur[k] = 0ull;
    if (lane == 0) rs[w] = RowScalars{1.0, 0.0, 0.0, 0.0};
  }

  // ---- rounds
  for (int r = 0; r < A.rounds; ++r) {
    const int m_base = swaps_of(cfg, h, r, A.rho);
    if (m_base <= 0) continue;  // no swaps for this head in this round
    __syncthreads();            // u and the row scalars of every row are in LDS

    // gains of the tile's rows: operand row c16 = u of row c16 (kept-list
    // form), or u of row c16 and, for c16 >= 8, w of row c16 - 8 (pooled
    // form); result rows q4 + 4e, block 16t + c16
    const double* ur =
        (POOLED && c16 >= kRows)
            ? wv + (size_t)(c16 - kRows) * kD
            : reinterpret_cast<const double*>(smem + L.slot + (size_t)c16 * kSlotStride);
    for (int t = w; t < n_tiles; t += kRows) {
      const int j = 16 * t + c16;
      const int jc = min(j, n - 1);
      const f64x4 acc = group_product(ur, Vh + (size_t)jc * kD, q4);
      constexpr int kE = POOLED ? 2 : 4;  // result rows that are gains
      double pv[kE], kv[kE];
      if constexpr (POOLED) {
        const double vmj = vm[jc];
#pragma unroll
        for (int e = 0; e < kE; ++e) {
          const int rl = q4 + 4 * e;
          pv[e] = prows[(size_t)rl * ns + jc];
          kv[e] = fused_drift_key(pv[e], acc[e + 2], av[rl], vmj, eps);
        }
      } else {
#pragma unroll
        for (int e = 0; e < kE; ++e) {
          const int rr = min(i0 + q4 + 4 * e, nq - 1);
          const size_t rw = (size_t)h * nq + rr;
          pv[e] = A.P[rw * n + jc];
          kv[e] = A.key[rw * n + jc];
        }
      }
#pragma unroll
      for (int e = 0; e < kE; ++e) {
        const int rl = q4 + 4 * e;  // row within the tile
        const double p = pv[e];
        const double sv = kv[e] * fmax(1.0 - p, eps);  // s_ij (Eq. 6)
        const bool inD = (curw[(size_t)rl * KW + (jc >> 6)] >> (jc & 63)) & 1ull;
        const double dJ = swap_gain(rs[rl], p, sv, acc[e], inD);
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
        if (lane == 0) rs[w] = RowScalars{Kc, G, J, vu};
      }
      // m = 0: no swap, the row (and its u, which no histogram overwrote)
      // stays as it was
    }
  }
  __syncthreads();

  // ---- the best sets as keep lists, ascending, -1 padded
  if (live) {
    int32_t* out = A.kept_idx + row * A.k_max;
    int pos = 0;
    for (int k = 0, j0 = 0; j0 < n; ++k, j0 += 64) {
      const int j = j0 + lane;
      const bool kept = j < n && (sel_always_wave(cfg, j) || !((mybest[k] >> lane) & 1ull));
      const uint64_t msk = __ballot(kept);
      const int p = pos + __popcll(msk & below);
      if (kept && p < A.k_max) out[p] = j;
      pos += __popcll(msk);
    }
    for (int p = pos + lane; p < A.k_max; p += 64) out[p] = -1;
    if (lane == 0) {
      A.kept_cnt[row] = pos < A.k_max ? pos : A.k_max;
      if (A.J_init) A.J_init[row] = J0;
      if (A.J_final) A.J_final[row] = Jbest;
    }
  }
}

template <bool POOLED>
hipError_t launch_fused_form(const FusedArgs& a, const ress_shape& s, const SelConfig& cfg,
                             hipStream_t st) {
  constexpr int kRows = fused_rows<POOLED>();
  const size_t lds = FusedLds(a.n, kRows, POOLED).total;
  if (lds > 64 * 1024) {
    const hipError_t e =
        hipFuncSetAttribute(reinterpret_cast<const void*>(&refine_fused_kernel<POOLED>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(refine_fused_kernel<POOLED>, dim3((a.nq + kRows - 1) / kRows, s.H),
                     dim3(64 * kRows), lds, st, a, cfg);
  return hipGetLastError();
}

}  // namespace

int refine_fused_max_blocks() { return 64 * kMaxWords; }

hipError_t launch_refine_fused(const double* P, const double* key, const double* vpool,
                               const double* vout, const double* M, const ress_shape& s,
                               const SelConfig& cfg, int32_t rounds, double rho, double eps,
                               int32_t k_max, int32_t* kept_idx, int32_t* kept_cnt,
                               double* J_init, double* J_final, hipStream_t st) {
  FusedArgs a{};
  a.P = P;
  a.key = key;
  a.vout = vout;
  a.vpool = vpool;
  a.M = M;
  a.nq = n_qblocks(s);
  a.n = n_kblocks(s);
  a.rounds = rounds;
  a.k_max = k_max;
  a.rho = rho;
  a.eps = eps;
  a.kept_idx = kept_idx;
  a.kept_cnt = kept_cnt;
  a.J_init = J_init;
  a.J_final = J_final;
  return launch_fused_form<false>(a, s, cfg, st);
}

hipError_t launch_select_refine_fused(const double* qpool, const double* kpool,
                                      const double* vpool, const double* M, const double* vmv,
                                      const ress_shape& s, const SelConfig& cfg, double scale,
                                      int32_t rounds, double rho, double eps, int32_t k_max,
                                      int32_t* kept_idx, int32_t* kept_cnt, double* J_init,
                                      double* J_final, hipStream_t st) {
  FusedArgs a{};
  a.qpool = qpool;
  a.kpool = kpool;
  a.vmv = vmv;
  a.vpool = vpool;
  a.M = M;
  a.nq = n_qblocks(s);
  a.n = n_kblocks(s);
  a.rounds = rounds;
  a.k_max = k_max;
  a.rho = rho;
  a.eps = eps;
  a.scale = scale;
  a.kept_idx = kept_idx;
  a.kept_cnt = kept_cnt;
  a.J_init = J_init;
  a.J_final = J_final;
  return launch_fused_form<true>(a, s, cfg, st);
}

}  // namespace ress
