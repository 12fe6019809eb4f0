// The linear maps on either side of the attention call, as bf16 matrix-core
// GEMMs (gfx950): the QKV projection that produces the per-head Q, K, V
// tensors the path consumes, and the output projection W_O with the residual
// add, which carries the attention output of every head back into the
// residual stream ("ReSS: Residual-Restoring Sparse Attention for 3D Vision
// Transformers", §3: a pre-LN residual sublayer; §4.2 "Mapping to the
// residual space", Eq. 6 and 8: head h's output o^h reaches the residual
// stream as W_O^h o^h).
//
// Both are C[M][Nc] = A[M][K] B[Nc][K]^T with K contiguous in both operands
// (a linear layer's weight is [out][in]), v_mfma_f32_32x32x16_bf16 with
// float32 accumulation, in one of two tile shapes:
//  * 256 x 256 output tiles, eight waves of 128 x 64 (4 x 2 MFMA tiles), one
//    workgroup per CU, for products with at least four such tiles per CU;
//  * 128 x 128 output tiles, four waves of 64 x 64, two workgroups per CU,
//    for smaller ones (the big tile leaves CUs idle there).
// The products are formed as C^T (the weight rows as the MFMA's A operand),
// so each lane ends up with four consecutive output channels of one token
// and stores them with one 8-byte write. k-tiles of 64 alternate between two
// LDS stages, copied straight from global memory (global_load_lds): the next
// k-tile streams in while one is multiplied. The operand loaders and the
// epilogue differ per map:
//  * QKV: A = x [N_pad][d_model]; B = W_qkv [3 H D][d_model]; output channel
//    c = which * H D + h D + d goes to {q,k,v}[which][h][t][d] (the
//    [H][N_pad][D] layout of the path), plus the bias; rows t >= N are
//    written as zeros.
//  * Output: A = the attention output o [H][N_pad][D] read as [N_pad][H D]
//    (k-tile h, 64 wide, is head h's D); B = W_O
//    [d_model][H D]; y[t][c] = residual[t][c] + bias[c] + sum_k A[t][k]
//    W_O[c][k], rounded once to bf16.
#include <type_traits>

#include "ress_internal.h"

namespace ress {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// WGM x WGN waves per workgroup, each wave owning TM x TN sub-tiles of
// 32 x 32 outputs (TM along the tokens, TN along the output channels). A
// copy window is 8 tile rows x 128 bytes (1 KB), one 16-byte copy per lane;
// kWinA / kWinB: windows of each operand per wave.
template <int WGM, int WGN, int TM, int TN>
struct TileCfg {
  static constexpr int kWGM = WGM, kWGN = WGN, kTM = TM, kTN = TN;
  static constexpr int kWaves = WGM * WGN;
  static constexpr int kBM = 32 * WGM * TM, kBN = 32 * WGN * TN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kWinA = kBM / 8 / kWaves, kWinB = kBN / 8 / kWaves;
  static constexpr int kWinPerWave = kWinA + kWinB;
  static_assert(kBM % (8 * kWaves) == 0 && kBN % (8 * kWaves) == 0,
                "whole copy windows of each operand per wave");
};
using BigTile = TileCfg<2, 4, 4, 2>;    // 256 x 256, 8 waves
using SmallTile = TileCfg<2, 2, 2, 2>;  // 128 x 128, 4 waves
constexpr int kBK = 64;

__device__ inline int swz(int row) { return (row >> 1) & 7; }

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// 16 bytes global -> LDS without registers; lane l of the wave writes the
// 16 bytes at `window` + 16 * l (window is wave-uniform). Issued as inline
// assembly, which produces no register and which the compiler does not count
// as an outstanding load: the kernel waits for these copies itself
// (wait_vmem), so that one stage can be read while the copies into the other
// are in flight (the compiler, tracking the copies itself, waits for all of
// them before any LDS read). The compiler's own vmcnt waits stay correct,
// only stricter: the copies complete in issue order with its loads.
__device__ inline void gload_lds16(const uint16_t* g, uint16_t* window) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)window);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(lds)
               : "memory", "m0");
}

// waits until at most N of this wave's vector memory operations are in flight
template <int N>
__device__ inline void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for the LDS stages: waits for this wave's LDS reads (not
// for copies still in flight, which wait_vmem covers) and keeps the compiler
// from moving memory accesses across it.
__device__ inline void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// C[M][Nc] = A B^T over K (a multiple of 64). la.ptr(row, k) / lb.ptr(row,
// k): the address of 8 consecutive k of a row (row < M, resp. < Nc; k a
// multiple of 8; 16-byte aligned). st(m, n, acc[4]): the epilogue of outputs
// (m, n .. n+3) (m < M; n a multiple of 4, n + 3 < Nc, which holds as Nc is a
// multiple of 64).
//
// Operand tiles are row-major in LDS (128-byte rows of eight 16-byte chunks,
// the chunk index XORed by (row >> 1) & 7 so that the operand reads, 16 rows
// at one logical chunk per 16-lane pass, are bank-conflict free). In copy
// window v (rows 8v .. 8v + 7) lane l fills row 8v + l / 8 at physical chunk
// l % 8, i.e. logical chunk (l % 8) ^ ((l / 16 + 4v) % 8). The two stages are
// separate LDS arrays named at compile time.
template <class Cfg, int MINB, class LoadA, class LoadB, class Store>
__global__ __launch_bounds__(Cfg::kThreads, MINB) void gemm_nt_kernel(int M, int Nc, int K,
                                                                     LoadA la, LoadB lb,
                                                                     Store st) {
  constexpr int kTM = Cfg::kTM, kTN = Cfg::kTN, kWGN = Cfg::kWGN, kWaves = Cfg::kWaves;
  constexpr int kBM = Cfg::kBM, kBN = Cfg::kBN;
  constexpr int kWinA = Cfg::kWinA, kWinB = Cfg::kWinB;
  __shared__ __attribute__((aligned(16))) uint16_t As0[kBM * kBK], As1[kBM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs0[kBN * kBK], Bs1[kBN * kBK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, half = lane >> 5;
  const int wm = w / kWGN, wn = w % kWGN;
  // Tile order: workgroups are handed to the eight XCDs in turn, so the ones
  // landing on XCD x (ids x, x + 8, ...) take a contiguous range of tiles,
  // column tiles fastest: the column tiles of one row tile then run on one
  // XCD and share its L2 copy of the A rows.
  const int n_tiles = (Nc + kBN - 1) / kBN;
  int tile;
  {
    const int T = gridDim.x, L = blockIdx.x;
    const int x = L & 7, q = T >> 3, r = T & 7;
    tile = x * q + min(x, r) + (L >> 3);
  }
  const int m0 = (tile / n_tiles) * kBM, n0 = (tile % n_tiles) * kBN;
  const int crow = lane >> 3;

  // the copies of k-tile kt into stage S: A windows w, w + kWaves, ... and
  // B windows likewise
  auto issue = [&](auto stagec, int kt) {
    constexpr int S = decltype(stagec)::value;
    uint16_t* const as = S == 0 ? As0 : As1;
    uint16_t* const bs = S == 0 ? Bs0 : Bs1;
#pragma unroll
    for (int u = 0; u < kWinA; ++u) {
      const int v = w + kWaves * u;  // wave-uniform
      const int c = (lane & 7) ^ (((lane >> 4) + 4 * v) & 7);
      gload_lds16(la.ptr(min(m0 + 8 * v + crow, M - 1), kt * kBK + 8 * c), as + 8 * v * kBK);
    }
#pragma unroll
    for (int u = 0; u < kWinB; ++u) {
      const int v = w + kWaves * u;
      const int c = (lane & 7) ^ (((lane >> 4) + 4 * v) & 7);
      gload_lds16(lb.ptr(min(n0 + 8 * v + crow, Nc - 1), kt * kBK + 8 * c), bs + 8 * v * kBK);
    }
  };

  f32x16 acc[kTM][kTN];
#pragma unroll
  for (int a = 0; a < kTM; ++a)
#pragma unroll
    for (int b = 0; b < kTN; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  // the products of one stage; the operands of 16-k step ks + 1 are read
  // while step ks's MFMAs issue
  auto compute = [&](auto stagec) {
    constexpr int S = decltype(stagec)::value;
    const uint16_t* const as = S == 0 ? As0 : As1;
    const uint16_t* const bs = S == 0 ? Bs0 : Bs1;
    bf16x8 af[2][kTM], bfr[2][kTN];
    auto read = [&](int ks, bf16x8 (&a)[kTM], bf16x8 (&b)[kTN]) {
#pragma unroll
      for (int u = 0; u < kTM; ++u) {
        const int r = 32 * (kTM * wm + u) + l32;
        a[u] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                                              &as[r * kBK + (((2 * ks + half) ^ swz(r)) << 3)]));
      }
#pragma unroll
      for (int u = 0; u < kTN; ++u) {
        const int r = 32 * (kTN * wn + u) + l32;
        b[u] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                                              &bs[r * kBK + (((2 * ks + half) ^ swz(r)) << 3)]));
      }
    };
    read(0, af[0], bfr[0]);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      if (ks + 1 < kBK / 16) read(ks + 1, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);  // keeps those reads ahead of the MFMAs
#pragma unroll
      for (int a = 0; a < kTM; ++a)
#pragma unroll
        for (int b = 0; b < kTN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ks & 1][b], af[ks & 1][a],
                                                             acc[a][b], 0, 0, 0);
    }
  };

  // one k-tile from stage S: wait for its copies, a barrier (every wave's
  // copies have landed, and every wave is done with the other stage), the
  // copies of tile kt + 1 into the other stage, the products
  const int nk = K / kBK;
  auto step = [&](auto stagec, int kt) {
    constexpr int S = decltype(stagec)::value;
    wait_vmem<0>();
    lds_barrier();
    if (kt + 1 < nk) issue(std::integral_constant<int, S ^ 1>{}, kt + 1);
    compute(stagec);
  };

  issue(std::integral_constant<int, 0>{}, 0);
  for (int kt = 0;;) {
    step(std::integral_constant<int, 0>{}, kt);
    if (++kt >= nk) break;
    step(std::integral_constant<int, 1>{}, kt);
    if (++kt >= nk) break;
  }

  // accumulator element r of lane l (C^T): output channel n = 8(r/4) +
  // 4(l/32) + r%4 of the sub-tile, token m = l%32, so r = 4g .. 4g+3 are four
  // consecutive channels of one token
#pragma unroll
  for (int a = 0; a < kTM; ++a) {
    const int m = m0 + 32 * (kTM * wm + a) + l32;
    if (m >= M) continue;
#pragma unroll
    for (int b = 0; b < kTN; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + 32 * (kTN * wn + b) + 8 * g + 4 * half;
        if (n < Nc) {
          const float v[4] = {acc[a][b][4 * g], acc[a][b][4 * g + 1], acc[a][b][4 * g + 2],
                              acc[a][b][4 * g + 3]};
          st(m, n, v);
        }
      }
  }
}

struct RowMajorLoad {  // X[row][k], row stride ld (elements)
  const uint16_t* X;
  int ld;
  __device__ const uint16_t* ptr(int row, int k) const { return X + (size_t)row * ld + k; }
};

struct HeadMajorLoad {  // o[h][t][d] read as A[t][h D + d] (8 k never cross a head)
  const uint16_t* o;
  int N_pad;
  __device__ const uint16_t* ptr(int t, int k) const {
    const int h = k >> 6, d = k & 63;
    return o + ((size_t)h * N_pad + t) * 64 + d;
  }
};

// four consecutive bf16 (8 bytes) to float
__device__ inline void load4(const uint16_t* p, float (&x)[4]) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  x[0] = __uint_as_float(u.x << 16);
  x[1] = __uint_as_float(u.x & 0xFFFF0000u);
  x[2] = __uint_as_float(u.y << 16);
  x[3] = __uint_as_float(u.y & 0xFFFF0000u);
}
__device__ inline void store4(uint16_t* p, const float (&x)[4]) {
  uint2 u;
  u.x = (uint32_t)f32_to_bf16_rne(x[0]) | ((uint32_t)f32_to_bf16_rne(x[1]) << 16);
  u.y = (uint32_t)f32_to_bf16_rne(x[2]) | ((uint32_t)f32_to_bf16_rne(x[3]) << 16);
  *reinterpret_cast<uint2*>(p) = u;
}

struct QkvStore {
  uint16_t* dst[3];
  const uint16_t* bias;  // [3 H D] or null
  int H, N, N_pad;
  __device__ void operator()(int t, int c, const float (&acc)[4]) const {
    const int hd = H * 64;
    const int which = c / hd, h = (c - which * hd) >> 6, d = c & 63;
    float b[4] = {0.f, 0.f, 0.f, 0.f}, v[4];
    if (bias) load4(bias + c, b);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = t < N ? acc[e] + b[e] : 0.f;
    store4(dst[which] + ((size_t)h * N_pad + t) * 64 + d, v);
  }
};

struct OutStore {
  uint16_t* y;
  const uint16_t* bias;      // [d_model] or null
  const uint16_t* residual;  // [N_pad][d_model] or null
  int d_model;
  __device__ void operator()(int t, int c, const float (&acc)[4]) const {
    const size_t at = (size_t)t * d_model + c;
    float v[4] = {acc[0], acc[1], acc[2], acc[3]}, x[4];
    if (bias) {
      load4(bias + c, x);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += x[e];
    }
    if (residual) {
      load4(residual + at, x);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += x[e];
    }
    store4(y + at, v);
  }
};

template <class LA, class LB, class ST>
hipError_t launch_gemm(int M, int Nc, int K, LA la, LB lb, ST st, hipStream_t stream) {
  // the 256 x 256 tile once there are at least four of them per CU
  const int big = ((M + BigTile::kBM - 1) / BigTile::kBM) * ((Nc + BigTile::kBN - 1) / BigTile::kBN);
  if (big >= 4 * 256) {
    hipLaunchKernelGGL((gemm_nt_kernel<BigTile, 1, LA, LB, ST>), dim3(big),
                       dim3(BigTile::kThreads), 0, stream, M, Nc, K, la, lb, st);
  } else {
    const int tiles = ((M + SmallTile::kBM - 1) / SmallTile::kBM) *
                      ((Nc + SmallTile::kBN - 1) / SmallTile::kBN);
    hipLaunchKernelGGL((gemm_nt_kernel<SmallTile, 2, LA, LB, ST>), dim3(tiles),
                       dim3(SmallTile::kThreads), 0, stream, M, Nc, K, la, lb, st);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qkv_project(const uint16_t* x, const uint16_t* w_qkv, const uint16_t* b_qkv,
                              int d_model, const ress_shape& s, uint16_t* q, uint16_t* k,
                              uint16_t* v, hipStream_t st) {
  QkvStore out{{q, k, v}, b_qkv, s.H, s.N, s.N_pad};
  return launch_gemm(s.N_pad, 3 * s.H * 64, d_model, RowMajorLoad{x, d_model},
                     RowMajorLoad{w_qkv, d_model}, out, st);
}

hipError_t launch_out_project(const uint16_t* o, const uint16_t* w_o, const uint16_t* b_o,
                              const uint16_t* residual, int d_model, const ress_shape& s,
                              uint16_t* y, hipStream_t st) {
  OutStore out{y, b_o, residual, d_model};
  return launch_gemm(s.N_pad, d_model, s.H * 64, HeadMajorLoad{o, s.N_pad},
                     RowMajorLoad{w_o, s.H * 64}, out, st);
}

}  // namespace ress
