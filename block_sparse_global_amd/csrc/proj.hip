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
// (a linear layer's weight is [out][in]): 128 x 128 output tiles, k-tiles of
// 32, four waves of 64 x 64 (2 x 2 v_mfma_f32_32x32x16_bf16 tiles each,
// float32 accumulation), four workgroups per CU. The products are formed as
// C^T (the weight rows as the MFMA's A operand), so each lane ends up with
// four consecutive output channels of one token and stores them with one
// 8-byte write. Operand tiles are staged in LDS, double-buffered, row-major
// (64-byte rows of four 16-byte chunks) with the chunk index XORed by
// (row >> 2) & 3, so that the operand reads (16 rows at one logical chunk per
// 16-lane pass) are bank-conflict free; the next k-tile's global loads are in
// flight while the current one is multiplied. The operand loaders and the
// epilogue differ per map:
//  * QKV: A = x [N_pad][d_model]; B = W_qkv [3 H D][d_model]; output channel
//    c = which * H D + h D + d goes to {q,k,v}[which][h][t][d] (the
//    [H][N_pad][D] layout of the path), plus the bias; rows t >= N are
//    written as zeros.
//  * Output: A = the attention output o [H][N_pad][D] read as [N_pad][H D]
//    (the columns of k-tile pair 2h, 2h+1 are head h's D); B = W_O
//    [d_model][H D]; y[t][c] = residual[t][c] + bias[c] + sum_k A[t][k]
//    W_O[c][k], rounded once to bf16.
#include "ress_internal.h"

namespace ress {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128, kBK = 32, kThreads = 256;
constexpr int kChunksPerTile = kBM * kBK / 8;                 // 16-byte chunks
constexpr int kChunksPerThread = kChunksPerTile / kThreads;   // 2
constexpr int kRowChunks = kBK / 8;                          // 16-byte chunks per row

__device__ inline int swz(int row) { return (row >> 2) & 3; }

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ inline float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// C[M][Nc] = A B^T over K (a multiple of 32). la(row, k) / lb(row, k): the
// 16 bytes of 8 consecutive k of a row (row < M, resp. < Nc; k a multiple of
// 8). st(m, n, acc[4]): the epilogue of outputs (m, n .. n+3) (m < M; n a
// multiple of 4, n + 3 < Nc, which holds as Nc is a multiple of 64).
template <class LoadA, class LoadB, class Store>
__global__ __launch_bounds__(kThreads, 4) void gemm_nt_kernel(int M, int Nc, int K, LoadA la,
                                                              LoadB lb, Store st) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][kBM * kBK];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kBN * kBK];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int l32 = lane & 31, half = lane >> 5;
  const int wm = w >> 1, wn = w & 1;
  // column tiles vary fastest: consecutive workgroups share the A rows
  const int n_tiles = (Nc + kBN - 1) / kBN;
  const int m0 = (blockIdx.x / n_tiles) * kBM, n0 = (blockIdx.x % n_tiles) * kBN;

  uint4 ra[kChunksPerThread], rb[kChunksPerThread];
  auto load = [&](int k0) {
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
      const int q = tid + kThreads * u, row = q / kRowChunks, c = q % kRowChunks;
      ra[u] = la(min(m0 + row, M - 1), k0 + 8 * c);
      rb[u] = lb(min(n0 + row, Nc - 1), k0 + 8 * c);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
      const int q = tid + kThreads * u, row = q / kRowChunks, c = q % kRowChunks;
      const int off = row * kBK + ((c ^ swz(row)) << 3);
      *reinterpret_cast<uint4*>(&As[buf][off]) = ra[u];
      *reinterpret_cast<uint4*>(&Bs[buf][off]) = rb[u];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int nk = K / kBK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * kBK);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int ra_row = 64 * wm + 32 * t + l32, rb_row = 64 * wn + 32 * t + l32;
        af[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                                               &As[buf][ra_row * kBK + (((2 * ks + half) ^ swz(ra_row)) << 3)]));
        bfr[t] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                                                &Bs[buf][rb_row * kBK + (((2 * ks + half) ^ swz(rb_row)) << 3)]));
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[b], af[a], acc[a][b], 0, 0, 0);
    }
    if (kt + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }

  // accumulator element r of lane l (C^T): output channel n = 8(r/4) +
  // 4(l/32) + r%4 of the sub-tile, token m = l%32, so r = 4g .. 4g+3 are four
  // consecutive channels of one token
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int m = m0 + 64 * wm + 32 * a + l32;
    if (m >= M) continue;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + 64 * wn + 32 * b + 8 * g + 4 * half;
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
  __device__ uint4 operator()(int row, int k) const {
    return *reinterpret_cast<const uint4*>(X + (size_t)row * ld + k);
  }
};

struct HeadMajorLoad {  // o[h][t][d] read as A[t][h D + d] (8 k never cross a head)
  const uint16_t* o;
  int N_pad;
  __device__ uint4 operator()(int t, int k) const {
    const int h = k >> 6, d = k & 63;
    return *reinterpret_cast<const uint4*>(o + ((size_t)h * N_pad + t) * 64 + d);
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
  const int tiles = ((M + kBM - 1) / kBM) * ((Nc + kBN - 1) / kBN);
  hipLaunchKernelGGL((gemm_nt_kernel<LA, LB, ST>), dim3(tiles), dim3(kThreads), 0, stream, M, Nc,
                     K, la, lb, st);
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
