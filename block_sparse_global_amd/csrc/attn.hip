// Exact attention over the kept key blocks ("ReSS: Residual-Restoring Sparse
// Attention for 3D Vision Transformers", §3 step (3): softmax renormalised
// among the selected blocks; dense global attention when every block is
// kept). Flash-style online softmax, bf16 matrix-core contractions with
// float32 accumulation, for gfx950.
//
// Work decomposition: one workgroup per (query block, head); BLK/32 waves,
// each owning 32 query rows. A tile holds KBLK = BLK keys: one kept key block
// of BLK keys, or, on the grid of 64-key blocks under 128-query blocks, two
// kept key blocks (any two, in list order; the second half is masked when a
// row's count is odd). Per tile the K and V tiles are copied
// straight from HBM into LDS (global_load_lds, double-buffered: the next
// tile streams in while the current one is computed) and every wave computes
//   S^T = K Q^T   (v_mfma_f32_32x32x16_bf16; A = K from LDS, B = Q^T held in
//                  registers for the whole kernel)
//   O^T += V^T P^T (A = V^T read from the row-major V tile with LDS
//                  transpose reads, B = P^T taken directly from the S^T
//                  accumulators after the softmax)
// so that each lane owns one query column: the reference subtracted from the
// logits, the running sum and the rescaling of O are per-lane scalars (the
// two lane halves holding the same query exchange one value when needed).
//
// Softmax in two passes only when needed. The first pass takes the weights
// as p = exp2(scale * log2(e) * S), with no max subtracted at all: O / l
// does not depend on a common offset of the logits, and float32 and bf16
// hold any p in [2^-126, 2^127] to full relative precision. That is valid as
// long as the row sum l stays within [2^-64, 2^64]: then no weight exceeds
// 2^64, and the largest one is at least 2^-64 / (keys in the row), so the
// weights that matter never underflow. A workgroup with any valid row
// outside that range (logits beyond roughly +-44 in natural units) discards
// its result and runs its rows again as a classical online softmax (running
// max, lazy rescaling): the second pass below. The first pass takes its row
// sums on the matrix cores, as the product of the bf16 weights with a 0/1
// selector (v_mfma_f32_16x16x32_bf16, eight per 32 x 128 wave tile), which
// takes 32 vector instructions per tile off the vector ALU.
//
// MFMA 32x32x16 operand convention used here: lane l supplies 8 consecutive
// k-slots of row/column (l % 32); lanes l and l+32 cover the two halves of
// the k range. The result accumulator element r of lane l is
// D[8*(r/4) + 4*(l/32) + r%4][l % 32]. Only this output mapping and the
// equal k-slot mapping of A and B matter for correctness; the parity tests
// check them end to end.
#include <type_traits>

#include "ress_internal.h"

namespace ress {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kD = 64;

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// 8 consecutive input elements as 8 bf16 (16 bytes).
__device__ inline uint4 load_row8(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ inline bf16x8 as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// LDS layout: K and V tiles are both row-major ([key][64 dims], 128-byte
// rows of eight 16-byte chunks), with the chunk index XORed by a
// row-dependent value so that the MFMA operand reads are bank-conflict free.
// gfx950's LDS serves a 128-bit access in passes of 16 lanes over 64
// four-byte banks; the bank group of (row, chunk) is (8 * row + chunk) mod 16.
//  * K (128-bit reads of 16 consecutive rows at one logical chunk):
//    XOR with (row >> 1) & 7 gives 16 distinct groups.
//  * V (transposed 64-bit reads, below): XOR with (row & 3) << 1 makes each
//    32-lane pass hit distinct banks.
__device__ inline int k_swz(int row) { return (row >> 1) & 7; }
__device__ inline int v_swz(int row) { return (row & 3) << 1; }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// ds_read_b64_tr_b16: within each group of 16 lanes, output lane i receives
// element i % 4 of the 8-byte words addressed by source lanes 4k + i / 4,
// k = 0..3. With source lane 4k + q pointing at V[key0 + k][d0 + 4q ..], lane
// i gets V[key0 .. key0 + 3][d0 + i]: four consecutive keys of one dim, the
// k-major operand layout the PV product needs, straight from row-major V.
__device__ inline v4i16 tr_read(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
}

// 16 bytes global -> LDS without registers; lane l of the wave writes the
// 16 bytes at `window` + 16 * l (window is wave-uniform).
__device__ inline void gload_lds16(const uint16_t* g, uint16_t* window) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)window, 16, 0, 0);
}

__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Workgroup barrier for the LDS tiles: waits for this wave's LDS operations
// (not for tile copies still in flight, which wait_vmem covers) and keeps the
// compiler from moving memory accesses across it.
__device__ inline void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// max of a lane's value and the one of lane l ^ 32 (v_permlane32_swap)
__device__ inline float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Range of the row sum accepted from the pass without a max (see the header).
constexpr float kSumMin = 0x1p-64f;
constexpr float kSumMax = 0x1p64f;
// Slack of the online softmax of the second pass (log2 units): a block whose
// max exceeds the one in use by less than this keeps it, so p <= 2^8.
constexpr float kRescaleSlack = 8.0f;

template <int BLK, int KBLK, bool PAIR, typename Tin, typename Tout>
__global__ __launch_bounds__(BLK * 2, 3) void attn_kernel(
    const Tin* __restrict__ Q, const Tin* __restrict__ Kx,
    const Tin* __restrict__ Vx, const int32_t* __restrict__ kept_idx,
    const int32_t* __restrict__ kept_cnt, int k_max, int n, int N, int N_pad,
    float scale, Tout* __restrict__ out, float* __restrict__ lse) {
  // n: key blocks (of kSrc keys, below) per head; gridDim.x: query blocks per head
  static_assert(KBLK <= BLK && BLK % KBLK == 0, "key blocks no larger than query blocks");
  // PAIR: 64-key blocks taken two kept blocks at a time into one 128-key
  // tile (waves 0-1 copy the first block, waves 2-3 the second)
  static_assert(!PAIR || KBLK == 128, "pairs of 64-key blocks fill 128-key tiles");
  constexpr int kSrc = PAIR ? 64 : KBLK;  // keys per key block of the list
  constexpr int kKT = KBLK / 32;     // 32-key tiles per key block
  constexpr int kTile = KBLK * kD;   // elements per K or V tile
  constexpr int kRowsPerWave = KBLK / (BLK / 32);  // tile rows each wave copies
  constexpr int kWin = kRowsPerWave / 8;           // 8-row copy windows per wave
  static_assert(kRowsPerWave % 16 == 0, "the K swizzle repeats every 16 rows");
  // One K buffer and two V buffers (48 KB at KBLK = 128, so three workgroups
  // share a CU): V of the next tile streams in during the whole of the
  // current tile, K of the next tile once every wave has finished its
  // S = K Q^T product.
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kTile];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][kTile];

  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  const size_t head_off = (size_t)h * N_pad * kD;
  const int qrow = i * BLK + 32 * w + l32;

  const float sl2 = scale * 1.4426950408889634f;  // scale * log2(e)
  // Q^T operand: dims 16*ks + 8*half + 0..7 of this lane's query row.
  // Padded query rows (qrow >= N) load row N - 1 instead (their outputs are
  // written as zeros): whatever the padding holds, their scores and weights
  // stay finite, so the first pass's row-sum product (whose zero selector
  // entries meet every query's weights) cannot turn NaN for the valid rows.
  const bool qvalid = qrow < N;
  bf16x8 qb[4];
  {
    const Tin* qp = Q + head_off + (size_t)min(qrow, N - 1) * kD + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qb[ks] = as_bf16x8(load_row8(qp + 16 * ks));
  }

  f32x16 o[2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_use = 0.f;  // running max in use (second pass), scaled log2 units
  float l_run = 0.f;
  const bf16x2 kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
  // row sums of the first pass on the matrix cores: D = Sel P^T with Sel a
  // 16 x 32 0/1 matrix whose row 0 adds the keys of queries 0-15 and row 1
  // those of queries 16-31 (v_mfma_f32_16x16x32_bf16 reads the PV weights'
  // register as 32 keys x 16 columns: column n, key group g = lane / 16
  // holds query n + 16 (g & 1))
  f32x4 lsum = {0.f, 0.f, 0.f, 0.f};
  bf16x8 sel;
  {
    const int m = lane & 15, g = lane >> 4;
    const __bf16 one = (m == 0 && !(g & 1)) || (m == 1 && (g & 1)) ? (__bf16)1.0f : (__bf16)0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) sel[e] = one;
  }

  // The keep list is read through the constant address space so that its
  // (workgroup-uniform) entries come in by scalar loads: vector loads would
  // share the vmcnt counter with the tile copies and a wait for a block index
  // would also wait for the copies in flight.
  typedef const __attribute__((address_space(4))) int32_t* const_i32p;
  int cnt = n;
  const_i32p list = nullptr;
  if (kept_idx != nullptr) {
    const size_t row = (size_t)h * gridDim.x + i;
    cnt = ((const_i32p)kept_cnt)[row];
    cnt = cnt < 0 ? 0 : (cnt > k_max ? k_max : cnt);
    list = (const_i32p)(kept_idx + row * k_max);
  }
  // next list position holding a valid block index (entries outside [0, n)
  // are skipped); uniform across the workgroup
  auto next_valid = [&](int kb) {
    if (list == nullptr) return kb;
    while (kb < cnt) {
      const int j = list[kb];
      if (j >= 0 && j < n) break;
      ++kb;
    }
    return kb;
  };
  auto block_of = [&](int kb) { return list ? list[kb] : kb; };

  // ---- staging of a K or V tile into an LDS buffer. Each wave
  // copies kWin windows of 8 rows; in window it, lane l fills row
  // r = kRowsPerWave*w + 8*it + l/8 at physical chunk l%8, i.e. logical chunk
  // (l%8) ^ swz(r). For V, swz(r) = 2*((l/8)&3) does not depend on it; for
  // K, swz(r) = (l/16) ^ (4*(it&1)) (kRowsPerWave is a multiple of 16). So
  // two per-lane offsets (windows 0 and 1) plus compile-time row steps cover
  // all windows. Rows past N (last key block only) are read from row N-1:
  // finite data whose scores are masked to -inf, so p = 0 multiplies a finite
  // V row; so is the empty second half of a pair tile (block ja again).
  const int row0 = kRowsPerWave * w + (lane >> 3);
  const int kgo0 = row0 * kD + (((lane & 7) ^ (lane >> 4)) * 8);
  const int kgo1 = (row0 + 8) * kD + (((lane & 7) ^ (lane >> 4) ^ 4) * 8);
  const int vgo0 = row0 * kD + (((lane & 7) ^ (((lane >> 3) & 3) << 1)) * 8);
  auto tile_off = [&](int it, bool is_v) {
    return is_v ? vgo0 + 8 * it * kD : ((it & 1) ? kgo1 : kgo0) + 16 * (it >> 1) * kD;
  };
  // the tile of key block ja (and, in pairs, jb): this wave copies its
  // kRowsPerWave tile rows from block src, whose row 0 is tile row hrow
  auto issue_tile = [&](const Tin* X, uint16_t* dst, int ja, int jb, bool is_v) {
    const bool second = PAIR && w >= 2;
    const int src = __builtin_amdgcn_readfirstlane(second ? jb : ja);
    const int hrow = second ? 64 : 0;  // tile row of the source block's row 0
    // block base (uniform) + 32-bit per-lane byte offset: the copies use
    // the scalar-base addressing form
    const char* base = reinterpret_cast<const char*>(X + head_off + (size_t)src * kSrc * kD);
    const bool full = (src + 1) * kSrc <= N;
    if (full) {
#pragma unroll
      for (int it = 0; it < kWin; ++it) {
        const uint32_t off = 2u * (uint32_t)(tile_off(it, is_v) - hrow * kD);
        gload_lds16(reinterpret_cast<const uint16_t*>(base + off), dst + (kWin * w + it) * 512);
      }
    } else {
      const int last = N - 1 - src * kSrc;
#pragma unroll
      for (int it = 0; it < kWin; ++it) {
        const int r = row0 + 8 * it - hrow;  // row within the source block
        const uint32_t off = 2u * (uint32_t)(tile_off(it, is_v) - hrow * kD + (min(r, last) - r) * kD);
        gload_lds16(reinterpret_cast<const uint16_t*>(base + off), dst + (kWin * w + it) * 512);
      }
    }
  };
  // the tile starting at list position kb: its blocks, and where the next
  // tile starts
  struct TileAt { int ja, jb, next; bool has_b; };
  auto tile_at = [&](int kb) {
    TileAt t;
    t.ja = block_of(kb);
    if constexpr (PAIR) {
      const int kb2 = next_valid(kb + 1);
      t.has_b = kb2 < cnt;
      t.jb = t.has_b ? block_of(kb2) : t.ja;
      t.next = t.has_b ? next_valid(kb2 + 1) : cnt;
    } else {
      t.has_b = false;
      t.jb = t.ja;
      t.next = next_valid(kb + 1);
    }
    return t;
  };

  // Per-lane LDS element offsets of the MFMA operands (the buffer, the
  // 32-key tile and the 16-key step only add compile-time constants).
  int koff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    koff[ks] = l32 * kD + (((2 * ks + half) ^ k_swz(l32)) * 8);
  int voff[2];
  {
    const int kk = (lane & 15) >> 2, q = lane & 3, G = (lane & 31) >> 4;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
      voff[dt] = (4 * half + kk) * kD + (((4 * dt + 2 * G + (q >> 1)) ^ (2 * kk)) * 8) +
                 (q & 1) * 4;
  }

  // ---- one tile, cur, with V from buffer B (compile-time, so all LDS
  // offsets are immediates); nxt is the tile after it. ONLINE: the second
  // pass, with a running max. Moves cur and nxt one tile on and returns
  // whether a tile followed.
  auto process = [&](auto bufc, auto onlinec, TileAt& cur, TileAt& nxt) {
    constexpr int B = decltype(bufc)::value;
    constexpr bool ONLINE = decltype(onlinec)::value;
    const bool more = cur.next < cnt;
    // square tiles: the next tile was looked up one block ahead; pairs
    // (whose lookup scans for two valid entries) are looked up here
    if constexpr (PAIR) {
      if (more) nxt = tile_at(cur.next);
    }
    if (more) issue_tile(Vx, Vs[B ^ 1], nxt.ja, nxt.jb, true);

    // S^T = K Q^T; the K operands of tile kt+1 are read while tile kt's
    // MFMAs run
    // wave priorities: the S product at 2, the weights at 0, the PV
    // product at 3 (below)
    __builtin_amdgcn_s_setprio(2);
    f32x16 s[kKT];
    bf16x8 ka[2][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      ka[0][ks] = as_bf16x8(*reinterpret_cast<const uint4*>(&Ks[koff[ks]]));
#pragma unroll
    for (int kt = 0; kt < kKT; ++kt) {
      if (kt + 1 < kKT) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          ka[(kt + 1) & 1][ks] = as_bf16x8(
              *reinterpret_cast<const uint4*>(&Ks[(kt + 1) * 32 * kD + koff[ks]]));
      }
      // keeps those reads ahead of this tile's MFMAs
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kt & 1][ks], qb[ks], s[kt], 0, 0, 0);
    }
    // every wave has read its K operands: the K tile of the next block may
    // replace this one
    lds_barrier();
    if (more) issue_tile(Kx, Ks, nxt.ja, nxt.jb, false);
    // the list entries of the tile after next, looked up now so that the
    // next block issues its copies without waiting for scalar loads
    TileAt nxt2{0, 0, cnt, false};
    if constexpr (!PAIR) {
      if (more && nxt.next < cnt) nxt2 = tile_at(nxt.next);
    }
    // mask padded keys (only the last block has any). Branching on the
    // block's valid-key count, which changes with j, keeps the compiler from
    // hoisting loop-invariant compare masks; the lane-half term is folded
    // into the limit so that the compares use immediate key offsets only.
    if constexpr (PAIR) {
      // per half: the keys of block ja (tile keys 0-63) and of jb (64-127,
      // none when the tile holds one block)
      const int live_a = N - cur.ja * kSrc;
      const int live_b = cur.has_b ? N - cur.jb * kSrc : 0;
      if (live_a < kSrc || live_b < kSrc) {
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt) {
          const int lim = (kt < 2 ? live_a : kSrc + live_b) - 4 * half;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kc = 32 * kt + 8 * (r >> 2) + (r & 3);
            if (kc >= lim) s[kt][r] = -INFINITY;
          }
        }
      }
    } else {
      const int live_keys = N - cur.ja * KBLK;
      if (live_keys < KBLK) {
        const int lim = live_keys - 4 * half;
#pragma unroll
        for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kc = 32 * kt + 8 * (r >> 2) + (r & 3);
            if (kc >= lim) s[kt][r] = -INFINITY;
          }
      }
    }
    if constexpr (ONLINE) {
      // online softmax (per lane = per query), lazy rescaling
      float mb = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mb = fmaxf(mb, s[kt][r]);
      mb = max_halves(mb) * sl2;
      if (__any(mb > m_use + kRescaleSlack)) {
        const float m_new = fmaxf(m_use, mb);
        const float alpha = __builtin_amdgcn_exp2f(m_use - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
        m_use = m_new;
      }
    }
    // per 16-key step: P = exp2(S*scale*log2e - m) as bf16, then
    // O^T += V^T P^T with the V^T operand read transposed from LDS
    float psum = 0.f;
    // V^T operands of 16-key step st (both 32-dim halves); those of step
    // st+1 are read while step st computes
    auto v_operands = [&](int st, bf16x8 (&va)[2]) {
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const uint16_t* vp = &Vs[B][st * 16 * kD + voff[dt]];
        const v4i16 lo = tr_read(vp);           // keys 16*st + 4*half + 0..3
        const v4i16 hi = tr_read(vp + 8 * kD);  // keys 16*st + 8 + 4*half + 0..3
        va[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    // Two phases: first every bf16 weight of the block (exponentials, VALU
    // only; the online pass also sums them here) at wave priority 0, then all
    // PV MFMAs back to back at priority 3, with the first pass's row-sum
    // MFMAs among them; the S product before them runs at priority 2. A
    // wave and its matrix core then alternate in long runs instead of one
    // exponential batch per MFMA pair, and a wave whose P is complete (or
    // whose K tile has landed) gets the matrix core ahead of waves still
    // computing weights. Same bits as any other order; the two-phase order
    // measured 4-5% faster at 100 views than an interleaved one, and these
    // priorities 3% faster than priority 1 for the weights and 0 for S.
    bf16x8 vops[2][2];
    bf16x8 pall[2 * kKT];
    // p = exp2(S * scale * log2 e) (first pass) or exp2(S * scale * log2 e
    // - m) (online pass) as bf16; the online pass sums the very bf16 weights
    // the PV product uses here, two per instruction (bf16 dot product with
    // (1, 1), float32 accumulation), the first pass on the matrix cores
    // below
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int step = 0; step < 2 * kKT; ++step) {
      const int kt = step >> 1, hf = step & 1;
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const float x = ONLINE ? fmaf(s[kt][8 * hf + r], sl2, -m_use) : s[kt][8 * hf + r] * sl2;
        pall[step][r] = (__bf16)__builtin_amdgcn_exp2f(x);
      }
      if constexpr (ONLINE) {
#pragma unroll
        for (int r = 0; r < 8; r += 2) {
          const bf16x2 pp = {pall[step][r], pall[step][r + 1]};
          psum = __builtin_amdgcn_fdot2_f32_bf16(pp, kOnes2, psum, false);
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(3);
    v_operands(0, vops[0]);
#pragma unroll
    for (int step = 0; step < 2 * kKT; ++step) {
      if (step + 1 < 2 * kKT) v_operands(step + 1, vops[(step + 1) & 1]);
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vops[step & 1][dt], pall[step], o[dt], 0, 0, 0);
      if constexpr (!ONLINE) lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sel, pall[step], lsum, 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    l_run += psum;
    wait_vmem();  // this wave's copies of the next block's tiles have landed
    lds_barrier();
    cur = nxt;
    nxt = nxt2;
    return more;
  };

  // ---- the row, first without a max; again with one if any valid row of
  // the workgroup left the accepted range of the row sum
  __shared__ int rerun;
  if (tid == 0) rerun = 0;
  const int kb0 = next_valid(0);
  auto run_row = [&](auto onlinec) {
    TileAt cur{0, 0, cnt, false}, nxt{0, 0, cnt, false};
    if (kb0 < cnt) {
      cur = tile_at(kb0);
      if (!PAIR && cur.next < cnt) nxt = tile_at(cur.next);
      issue_tile(Kx, Ks, cur.ja, cur.jb, false);
      issue_tile(Vx, Vs[0], cur.ja, cur.jb, true);
      wait_vmem();
    }
    lds_barrier();
    if (kb0 < cnt) {
      for (;;) {
        if (!process(std::integral_constant<int, 0>{}, onlinec, cur, nxt)) break;
        if (!process(std::integral_constant<int, 1>{}, onlinec, cur, nxt)) break;
      }
    }
  };
  run_row(std::false_type{});
  float l_fast;
  {
    // query q = lane % 32: D[0][q] (q < 16) or D[1][q - 16], held by lane
    // q % 16 as its accumulator elements 0 and 1
    const int q = lane & 31;
    const float a = __shfl(lsum[0], q & 15, 64), b = __shfl(lsum[1], q & 15, 64);
    l_fast = q < 16 ? a : b;
    const float lt = l_fast;
    const bool bad = qvalid && kb0 < cnt && !(lt >= kSumMin && lt <= kSumMax);
    if (__any(bad) && lane == 0) rerun = 1;
  }
  lds_barrier();
  if (rerun) {
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
    l_run = 0.f;
    m_use = -INFINITY;
    run_row(std::true_type{});
  }

  // ---- epilogue
  const float l_tot = rerun ? l_run + __shfl_xor(l_run, 32, 64) : l_fast;
  const bool valid = qvalid;
  const float inv = (valid && l_tot > 0.f) ? 1.f / l_tot : 0.f;
  Tout* op = out + head_off + (size_t)qrow * kD;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dim = 32 * dt + 8 * g + 4 * half;
      // padded rows may hold garbage (even NaN) in their accumulators:
      // select zero rather than scale by it
      const float x0 = inv != 0.f ? o[dt][4 * g] * inv : 0.f;
      const float x1 = inv != 0.f ? o[dt][4 * g + 1] * inv : 0.f;
      const float x2 = inv != 0.f ? o[dt][4 * g + 2] * inv : 0.f;
      const float x3 = inv != 0.f ? o[dt][4 * g + 3] * inv : 0.f;
      if constexpr (sizeof(Tout) == 2) {
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16_rne(x0) | ((uint32_t)f32_to_bf16_rne(x1) << 16);
        pk.y = (uint32_t)f32_to_bf16_rne(x2) | ((uint32_t)f32_to_bf16_rne(x3) << 16);
        *reinterpret_cast<uint2*>(op + dim) = pk;
      } else {
        *reinterpret_cast<float4*>(op + dim) = make_float4(x0, x1, x2, x3);
      }
    }
  if (lse != nullptr && half == 0) {
    float v = 0.f;
    // m_use is in log2 units of scale*s; ln(2) converts it back
    if (valid) v = (l_tot > 0.f) ? m_use * 0.6931471805599453f + logf(l_tot) : -INFINITY;
    lse[(size_t)h * N_pad + qrow] = v;
  }
}

template <typename Tin>
hipError_t launch_t(const Tin* q, const Tin* k, const Tin* v,
                    const ress_shape& s, const int32_t* kept_idx,
                    const int32_t* kept_cnt, int32_t k_max, float scale,
                    void* out, float* lse, hipStream_t st) {
  const int nk = n_kblocks(s);
  dim3 grid(n_qblocks(s), s.H);
  using Tout = Tin;
  Tout* o = static_cast<Tout*>(out);
  if (s.B == 128 && key_block(s) == 128)
    hipLaunchKernelGGL((attn_kernel<128, 128, false, Tin, Tout>), grid, dim3(256), 0, st,
                       q, k, v, kept_idx, kept_cnt, k_max, nk, s.N, s.N_pad,
                       scale, o, lse);
  else if (s.B == 128)
    hipLaunchKernelGGL((attn_kernel<128, 128, true, Tin, Tout>), grid, dim3(256), 0, st,
                       q, k, v, kept_idx, kept_cnt, k_max, nk, s.N, s.N_pad,
                       scale, o, lse);
  else
    hipLaunchKernelGGL((attn_kernel<64, 64, false, Tin, Tout>), grid, dim3(128), 0, st,
                       q, k, v, kept_idx, kept_cnt, k_max, nk, s.N, s.N_pad,
                       scale, o, lse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const void* q, const void* k, const void* v, int dtype,
                       const ress_shape& s, const int32_t* kept_idx,
                       const int32_t* kept_cnt, int32_t k_max, float scale,
                       void* out, float* lse, hipStream_t st) {
  if (dtype == RESS_DTYPE_BF16)
    return launch_t(static_cast<const uint16_t*>(q),
                    static_cast<const uint16_t*>(k),
                    static_cast<const uint16_t*>(v), s, kept_idx, kept_cnt,
                    k_max, scale, out, lse, st);
  return launch_attn_f32(static_cast<const float*>(q), static_cast<const float*>(k),
                         static_cast<const float*>(v), s, kept_idx, kept_cnt, k_max, scale,
                         static_cast<float*>(out), lse, st);
}

}  // namespace ress
