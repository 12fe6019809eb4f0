// Drop-set refinement ("ReSS: Residual-Restoring Sparse Attention for 3D
// Vision Transformers", §4.3 "Iterative Residual Restoration", Eq. 10-17,
// and Appendix E "Fused Kernel Implementation").
//
// The per-row state (g, M g, K, G, J, the current and the best drop set) lives
// in a caller-provided workspace in HBM, and each round is two kernels over
// all rows of all heads:
//   * gains: for every head, the products V_j . (M g_i) of all key blocks j
//     and query-block rows i form one n_q x n_k x 64 float64 product, computed
//     on the matrix cores in 64 x 64 tiles (the dims staged through LDS);
//     its epilogue turns each product into the exact objective
//     decrease of Eq. 16 for restoring (j in D_i, Eq. 14) or dropping (j
//     kept, Eq. 15) j, stored as a 64-bit order key;
//   * select: one wave per row selects the m_r best restores and the m_r
//     best drops by an exact radix select (ties: lower block index), moves g
//     and K by the swapped blocks (Eq. 13), recomputes G = g^T M g and
//     J = G / K^2 (Eq. 12) and keeps the drop set with the smallest J seen
//     (track-best).
// An init kernel builds the starting state from the top-k keep lists and a
// final kernel writes the best sets back as keep lists. Rows are the n_q
// query blocks of every head, each of n = n_k key blocks; the per-row
// kernels run one workgroup per (row i, head h), gridDim.x = n_q.
// s_j (Eq. 6) comes from the drift key of Eq. 7: s = key * max(1 - P, eps).
// Every sum has a fixed order, so results are bit-reproducible.
#include "ress_internal.h"
#include "refine_common.h"
#include "tile_f64.h"

namespace ress {
namespace {


// Per-row scalars of the refinement state.
struct alignas(64) RowState {
  double K, G, J, Jbest, J0, vu;  // vu = vout . (M g)
  int32_t nD, nS;                 // sizes of D and of the kept candidates
};

// Workspace regions (each 256-byte aligned).
struct RefineWs {
  uint64_t* gains;  // [H][n_q][n_k] order keys of the gains
  uint8_t* fcur;    // [H][n_q][fs] 1 = block in the current drop set D
  uint8_t* fbest;   // [H][n_q][fs] 1 = block in the best drop set
  double* g;        // [H][n_q][64]
  double* u;        // [H][n_q][64] M g
  RowState* rs;     // [H][n_q]
};

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

struct WsLayout {
  size_t gains, fcur, fbest, g, u, rs, total;
  explicit WsLayout(const ress_shape& s) {
    const size_t nq = (size_t)n_qblocks(s), nk = (size_t)n_kblocks(s), H = (size_t)s.H;
    size_t off = 0;
    gains = off; off += align256(H * nq * nk * 8);
    const size_t fs = (size_t)flag_stride((int)nk);
    fcur = off;  off += align256(H * nq * fs);
    fbest = off; off += align256(H * nq * fs);
    g = off;     off += align256(H * nq * kD * 8);
    u = off;     off += align256(H * nq * kD * 8);
    rs = off;    off += align256(H * nq * sizeof(RowState));
    total = off;
  }
  RefineWs at(void* base) const {
    unsigned char* b = static_cast<unsigned char*>(base);
    return RefineWs{reinterpret_cast<uint64_t*>(b + gains), b + fcur, b + fbest,
                    reinterpret_cast<double*>(b + g), reinterpret_cast<double*>(b + u),
                    reinterpret_cast<RowState*>(b + rs)};
  }
};



// ---------------------------------------------------------------- init
// One wave per (row i, head h): D_i = candidates not in the keep list,
// K = 1 - sum_{j in D} P_ij, and g_i = sum_{j in D} P_ij (vout_i - V_j)
// (Eq. 5, 10). The sum over all j of P_ij (vout_i - V_j) is zero (the row of
// P sums to one and vout_i is sum_j P_ij V_j), so g_i also equals
// sum_{j in S_i} P_ij (V_j - vout_i) over the kept blocks, up to rounding. g
// is summed over whichever of D and S has fewer blocks: S at high sparsity
// (about a tenth of the terms at 90%), D when few blocks are dropped, where
// the S form would leave a rounding residue of vout (~1e-16 |V|) that can
// dwarf a g of dropped blocks of tiny probability. Both lists ascend.
__global__ __launch_bounds__(64) void refine_init_kernel(
    const double* __restrict__ P, const double* __restrict__ vpool,
    const double* __restrict__ vout, const double* __restrict__ M, int n,
    SelConfig cfg, int k_max, const int32_t* __restrict__ kept_idx,
    const int32_t* __restrict__ kept_cnt, RefineWs ws) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint8_t* flags = smem;                                                 // [n]
  // kept blocks ascending from the front, dropped ones ascending from the
  // back (entry n-1-q is the q-th dropped block)
  int32_t* slist = reinterpret_cast<int32_t*>(smem + ((n + 15) & ~15));  // [n]
  double* gl = reinterpret_cast<double*>(slist + ((n + 3) & ~3));        // [64]
  const int i = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const size_t row = (size_t)h * gridDim.x + i;
  const double* Prow = P + row * n;
  const double* Vh = vpool + (size_t)h * n * kD;

  for (int j = lane; j < n; j += 64) flags[j] = sel_always_wave(cfg, j) ? 0 : 1;
  wave_lds_sync();
  int cnt = kept_cnt[row];
  cnt = cnt < 0 ? 0 : (cnt > k_max ? k_max : cnt);
  for (int q = lane; q < cnt; q += 64) {
    const int j = kept_idx[row * k_max + q];
    if (j >= 0 && j < n) flags[j] = 0;
  }
  wave_lds_sync();

  uint8_t* fc = ws.fcur + row * flag_stride(n);
  uint8_t* fb = ws.fbest + row * flag_stride(n);
  const uint64_t below = (1ull << lane) - 1ull;
  double ks = 0.0;
  int nD = 0, nS = 0, pos = 0, dpos = 0;
  // the P row is read in batches of 8 chunks of 64 blocks (clamped
  // addresses, all loads in flight together); the sum takes the same order
  constexpr int kPre = 8;
  for (int c0 = 0; c0 < n; c0 += 64 * kPre) {
    double pv[kPre];
#pragma unroll
    for (int u = 0; u < kPre; ++u) pv[u] = Prow[min(c0 + 64 * u + lane, n - 1)];
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int j = c0 + 64 * u + lane;
      const bool in = j < n;
      const uint8_t f = in ? flags[j] : 0;
      if (in) {
        fc[j] = f;
        fb[j] = f;
      }
      const bool inD = in && f != 0, kept = in && f == 0;
      if (inD) ks += pv[u];
      nD += inD;
      nS += kept && !sel_always_wave(cfg, j);
      const uint64_t msk = __ballot(kept);
      if (kept) slist[pos + __popcll(msk & below)] = j;
      pos += __popcll(msk);
      const uint64_t dmsk = __ballot(inD);
      if (inD) slist[n - 1 - (dpos + __popcll(dmsk & below))] = j;
      dpos += __popcll(dmsk);
    }
  }
  const double K = 1.0 - wave_sum64(ks);
  nD = wave_isum64(nD);
  nS = wave_isum64(nS);
  wave_lds_sync();

  const int d = lane;
  const double vod = vout[row * kD + d];
  double acc = 0.0;
  if (dpos < pos) {
    // over D, Eq. 10 itself (an empty D: exactly zero)
#pragma unroll 8
    for (int q = 0; q < dpos; ++q) {
      const int j = slist[n - 1 - q];
      acc += Prow[j] * (vod - Vh[(size_t)j * kD + d]);
    }
  } else {
#pragma unroll 8
    for (int q = 0; q < pos; ++q) {
      const int j = slist[q];
      acc += Prow[j] * (Vh[(size_t)j * kD + d] - vod);
    }
  }
  const double g = acc;
  gl[d] = g;
  wave_lds_sync();
  double G, vu;
  const double u = gram_apply(M ? M + (size_t)h * kD * kD : nullptr, gl, g, vod, &G, &vu);
  ws.g[row * kD + d] = g;
  ws.u[row * kD + d] = u;
  if (lane == 0) {
    RowState st;
    st.K = K;
    st.G = G;
    st.J = (K > 0.0) ? G / (K * K) : INFINITY;
    st.J0 = st.J;
    st.Jbest = st.J;
    st.vu = vu;
    st.nD = nD;
    st.nS = nS;
    ws.rs[row] = st;
  }
}

// ---------------------------------------------------------------- gains
// C[i][j] = u_i . V_j over a 64 x 64 tile (rows i < nq, key blocks j < nk)
// of one head on the float64 matrix cores (mfma_tile_f64); the epilogue
// takes the lane's rows two at a time (the loads of a pass, then its gains),
// which keeps the kernel within 128 VGPRs: four workgroups per CU, where the
// latency of its HBM reads needs the extra waves (issuing the epilogue's
// loads ahead of the product measured slower at 240 VGPRs).
__device__ inline void load8d(const double* p, double (&x)[8]) {
  const double2* src = reinterpret_cast<const double2*>(p);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const double2 v = src[e];
    x[2 * e] = v.x;
    x[2 * e + 1] = v.y;
  }
}

__global__ __launch_bounds__(256, 4) void refine_gains_kernel(
    const double* __restrict__ P, const double* __restrict__ key,
    const double* __restrict__ vpool, int nq, int nk, SelConfig cfg, int round, double rho,
    double eps, RefineWs ws) {
  const TileIdx tid3 = xcd_tile_order();
  const int h = tid3.z;
  if (swaps_of(cfg, h, round, rho) <= 0) return;  // no swaps for this head
  __shared__ TileF64Smem sm;
  const int j0 = tid3.x * kTF, i0 = tid3.y * kTF;
  const double* Uh = ws.u + (size_t)h * nq * kD;
  const double* Vh = vpool + (size_t)h * nk * kD;
  f64x4 acc[2][2];
  mfma_tile_f64(
      [&](int r, int d0, double (&x)[8]) { load8d(Uh + (size_t)min(i0 + r, nq - 1) * kD + d0, x); },
      [&](int r, int d0, double (&x)[8]) { load8d(Vh + (size_t)min(j0 + r, nk - 1) * kD + d0, x); },
      sm, acc);

  // epilogue: the exact objective decrease of each swap (Eq. 13-16). Out
  // of range rows and blocks load from a clamped valid address and are not
  // stored. The lane's results cover 8 rows (tr, r) x 2 key blocks (tc),
  // taken in four passes of 2 rows: all loads of a pass, then its gains.
  const TileF64Map mp;
  const int fs = flag_stride(nk);
#pragma unroll
  for (int tr = 0; tr < 2; ++tr) {
#pragma unroll
    for (int rh = 0; rh < 4; rh += 2) {
      double pv[2][2], kv[2][2];
      uint8_t fv[2][2];
      double sK[2], sG[2], sJ[2], svu[2];
#pragma unroll
      for (int r2 = 0; r2 < 2; ++r2) {
        const size_t row = (size_t)h * nq + min(i0 + mp.row_of(tr, rh + r2), nq - 1);
        const RowState* st = ws.rs + row;
        sK[r2] = st->K;
        sG[r2] = st->G;
        sJ[r2] = st->J;
        svu[r2] = st->vu;
#pragma unroll
        for (int tc = 0; tc < 2; ++tc) {
          const int j = min(j0 + mp.col_of(tc), nk - 1);
          pv[r2][tc] = P[row * nk + j];
          kv[r2][tc] = key[row * nk + j];
          fv[r2][tc] = ws.fcur[row * fs + j];
        }
      }
#pragma unroll
      for (int r2 = 0; r2 < 2; ++r2) {
        const int i = i0 + mp.row_of(tr, rh + r2);
        const size_t row = (size_t)h * nq + i;
#pragma unroll
        for (int tc = 0; tc < 2; ++tc) {
          const int j = j0 + mp.col_of(tc);
          const double p = pv[r2][tc];
          const double sv = kv[r2][tc] * fmax(1.0 - p, eps);  // s_ij (Eq. 6)
          const double dJ = swap_gain(RowScalars{sK[r2], sG[r2], sJ[r2], svu[r2]}, p, sv,
                                      acc[tr][tc][rh + r2], fv[r2][tc] != 0);
          if (i < nq && j < nk) ws.gains[row * nk + j] = order_key(dJ);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- select

// One wave per (row i, head h): the swaps of one round and the state update.
template <int KPL>
__global__ __launch_bounds__(64) void refine_select_kernel(
    const double* __restrict__ P, const double* __restrict__ vpool,
    const double* __restrict__ vout, const double* __restrict__ M, int n,
    SelConfig cfg, int round, double rho, RefineWs ws) {
  const int i = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const int m_base = swaps_of(cfg, h, round, rho);
  if (m_base <= 0) return;  // no swaps for this head
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint32_t* whist = reinterpret_cast<uint32_t*>(smem);                      // [256]
  double* gl = reinterpret_cast<double*>(smem + 1024);                      // [64]
  int32_t* chg = reinterpret_cast<int32_t*>(smem + 1536);                   // [n]
  uint8_t* flags = smem + 1536 + 4 * ((n + 3) & ~3);                        // [fs]
  uint64_t* gkeys = reinterpret_cast<uint64_t*>(flags + flag_stride(n));    // [n] (KPL = 0)

  const size_t row = (size_t)h * gridDim.x + i;
  const int fs = flag_stride(n);
  const uint4* fc = reinterpret_cast<const uint4*>(ws.fcur + row * fs);
  const uint64_t* grow = ws.gains + row * n;
  for (int c = lane; c < fs / 16; c += 64) reinterpret_cast<uint4*>(flags)[c] = fc[c];
  if constexpr (KPL == 0)
    for (int j = lane; j < n; j += 64) gkeys[j] = grow[j];
  const SelKeys<KPL> keys(KPL > 0 ? grow : gkeys, n, lane);
  const RowState st = ws.rs[row];
  const int m = min(m_base, min(st.nD, st.nS));
  wave_lds_sync();

  // membership over the candidates (always-kept blocks excluded). With 17
  // keys per lane the loop is branch-free, so all the flag reads and bitmask
  // words are issued together; with more keys that form holds too many of
  // them live (156 VGPRs against 114 at 34 keys per lane), so it stays a
  // loop that tests key by key.
  uint64_t memD = 0, memS = 0;
  constexpr int kU = KPL > 0 ? KPL : 4;
  if constexpr (KPL == 17) {
#pragma unroll
    for (int k = 0; k < KPL; ++k) {
      const int j = lane + 64 * k;
      const bool cand = j < n && !sel_always_wave(cfg, j);
      const bool inD = flags[min(j, n - 1)] != 0;
      memD |= (uint64_t)(cand && inD) << k;
      memS |= (uint64_t)(cand && !inD) << k;
    }
  } else {
#pragma unroll kU
    for (int k = 0; k < (KPL > 0 ? KPL : 64); ++k) {
      const int j = lane + 64 * k;
      if (j >= n) break;
      if (sel_always_wave(cfg, j)) continue;
      if (flags[j]) memD |= 1ull << k; else memS |= 1ull << k;
    }
  }
  const uint64_t restore = wave_select<KPL>(keys, memD, n, m, whist);
  const uint64_t drop = wave_select<KPL>(keys, memS, n, m, whist);
  // change list in ascending block index (sign: +1 for a drop)
  const uint64_t below = (1ull << lane) - 1ull;
  int nchg = 0;
  for (int k = 0, j0 = 0; j0 < n; ++k, j0 += 64) {
    const int j = j0 + lane;
    const bool rb = (restore >> k) & 1ull, db = (drop >> k) & 1ull;
    const uint64_t msk = __ballot(rb || db);
    if (rb || db) {
      chg[nchg + __popcll(msk & below)] = db ? (j + 1) : -(j + 1);
      flags[j] = db ? 1 : 0;
    }
    nchg += __popcll(msk);
  }
  wave_lds_sync();

  // g and K move by the swapped blocks (Eq. 13), in ascending order
  const int d = lane;
  const double* Prow = P + row * n;
  const double* Vh = vpool + (size_t)h * n * kD;
  const double vod = vout[row * kD + d];
  double g = ws.g[row * kD + d];
  double mag = fabs(g);  // what g is formed from, for the cancellation guard
  double dk = 0.0;
  // batches of 16 changes: all loads of a batch are issued before its sums.
  // Lanes 0-15 read the batch's entries from LDS in one access; each entry
  // then goes to a scalar register (readlane), so the block addresses are
  // formed by scalar instructions and the P values come in by scalar loads.
  for (int q0 = 0; q0 < nchg; q0 += 16) {
    int ev[16];
    double pv[16], vv[16];
    const int mine = chg[min(q0 + (lane & 15), nchg - 1)];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      ev[t] = __builtin_amdgcn_readlane(mine, t);
      const int j = (ev[t] > 0 ? ev[t] : -ev[t]) - 1;
      pv[t] = Prow[j];
      vv[t] = Vh[(size_t)j * kD + d];
    }
    // a uniform bound instead of a break, so that the loop unrolls and the
    // batch's registers are addressed directly
    const int live = min(16, nchg - q0);
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      if (t < live) {
        const double dj = pv[t] * (vod - vv[t]);
        g = (ev[t] > 0) ? g + dj : g - dj;
        mag += fabs(dj);
        dk = (ev[t] > 0) ? dk - pv[t] : dk + pv[t];  // K: +P for a restore, -P for a drop
      }
    }
  }
  if (g_cancelled(g, mag))
    g = g_from_sets([&](int j) { return flags[j] != 0; }, n, st.nD, Prow, Vh, vod);
  gl[d] = g;
  wave_lds_sync();
  double G, vu;
  const double u = gram_apply(M ? M + (size_t)h * kD * kD : nullptr, gl, g, vod, &G, &vu);
  const double K = st.K + dk;
  const double J = (K > 0.0) ? G / (K * K) : INFINITY;
  const bool better = J < st.Jbest;  // track-best, strict
  uint8_t* fcw = ws.fcur + row * fs;
  uint8_t* fbw = ws.fbest + row * fs;
  for (int q = lane; q < nchg; q += 64) {
    const int e = chg[q];
    const int j = (e > 0 ? e : -e) - 1;
    fcw[j] = e > 0 ? 1 : 0;
  }
  if (better)
    for (int c = lane; c < fs / 16; c += 64)
      reinterpret_cast<uint4*>(fbw)[c] = reinterpret_cast<const uint4*>(flags)[c];
  ws.g[row * kD + d] = g;
  ws.u[row * kD + d] = u;
  if (lane == 0) {
    RowState s2 = st;
    s2.K = K;
    s2.G = G;
    s2.J = J;
    s2.vu = vu;
    if (better) s2.Jbest = J;
    ws.rs[row] = s2;
  }
}

// ---------------------------------------------------------------- final
// Keep lists from the best drop sets, ascending, -1 padded.
__global__ __launch_bounds__(64) void refine_final_kernel(
    int n, SelConfig cfg, int k_max, RefineWs ws, int32_t* __restrict__ kept_idx,
    int32_t* __restrict__ kept_cnt, double* __restrict__ J_init,
    double* __restrict__ J_final) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int i = blockIdx.x, h = blockIdx.y, lane = threadIdx.x;
  const size_t row = (size_t)h * gridDim.x + i;
  const int fs = flag_stride(n);
  const uint4* fsrc = reinterpret_cast<const uint4*>(ws.fbest + row * fs);
  for (int c = lane; c < fs / 16; c += 64) reinterpret_cast<uint4*>(smem)[c] = fsrc[c];
  wave_lds_sync();
  const uint8_t* fb = smem;
  int32_t* out = kept_idx + row * k_max;
  const uint64_t below = (1ull << lane) - 1ull;
  int pos = 0;
  for (int j0 = 0; j0 < n; j0 += 64) {
    const int j = j0 + lane;
    const bool kept = j < n && (sel_always_wave(cfg, j) || !fb[j]);
    const uint64_t msk = __ballot(kept);
    const int p = pos + __popcll(msk & below);
    if (kept && p < k_max) out[p] = j;
    pos += __popcll(msk);
  }
  for (int p = pos + lane; p < k_max; p += 64) out[p] = -1;
  if (lane == 0) {
    kept_cnt[row] = pos < k_max ? pos : k_max;
    const RowState st = ws.rs[row];
    if (J_init) J_init[row] = st.J0;
    if (J_final) J_final[row] = st.Jbest;
  }
}

}  // namespace

size_t refine_workspace_bytes(const ress_shape& s) { return WsLayout(s).total; }

hipError_t launch_refine(const double* P, const double* key,
                         const double* vpool, const double* vout,
                         const double* M, const ress_shape& s,
                         const SelConfig& cfg, int32_t rounds, double rho,
                         double eps, int32_t k_max, int32_t* kept_idx,
                         int32_t* kept_cnt, double* J_init, double* J_final,
                         void* workspace, hipStream_t st) {
  const int nq = n_qblocks(s), n = n_kblocks(s);
  const RefineWs ws = WsLayout(s).at(workspace);
  const dim3 rows(nq, s.H);
  const size_t lds_init = (size_t)((n + 15) & ~15) + 4 * (size_t)((n + 3) & ~3) + 512;
  hipLaunchKernelGGL(refine_init_kernel, rows, dim3(64), lds_init, st, P, vpool, vout, M, n,
                     cfg, k_max, kept_idx, kept_cnt, ws);
  // the row's keys in registers (17 or 34 per lane) up to 2176 key blocks,
  // in LDS beyond
  const int kpl = n <= 17 * 64 ? 17 : (n <= 34 * 64 ? 34 : 0);
  const size_t lds_sel = 1536 + 4 * (size_t)((n + 3) & ~3) + (size_t)((n + 15) & ~15) +
                         (kpl > 0 ? 0 : 8 * (size_t)n);
  const dim3 tiles((n + kTF - 1) / kTF, (nq + kTF - 1) / kTF, s.H);
  for (int r = 0; r < rounds; ++r) {
    int m_max = 0;
    for (int h = 0; h < s.H; ++h) m_max = max(m_max, swaps_of(cfg, h, r, rho));
    if (m_max <= 0) continue;  // no head swaps in this round
    hipLaunchKernelGGL(refine_gains_kernel, tiles, dim3(256), 0, st, P, key, vpool, nq, n,
                       cfg, r, rho, eps, ws);
    if (kpl == 17)
      hipLaunchKernelGGL((refine_select_kernel<17>), rows, dim3(64), lds_sel, st, P, vpool,
                         vout, M, n, cfg, r, rho, ws);
    else if (kpl == 34)
      hipLaunchKernelGGL((refine_select_kernel<34>), rows, dim3(64), lds_sel, st, P, vpool,
                         vout, M, n, cfg, r, rho, ws);
    else
      hipLaunchKernelGGL((refine_select_kernel<0>), rows, dim3(64), lds_sel, st, P, vpool,
                         vout, M, n, cfg, r, rho, ws);
  }
  hipLaunchKernelGGL(refine_final_kernel, rows, dim3(64), (size_t)flag_stride(n), st, n, cfg,
                     k_max, ws, kept_idx,
                     kept_cnt, J_init, J_final);
  return hipGetLastError();
}

}  // namespace ress
