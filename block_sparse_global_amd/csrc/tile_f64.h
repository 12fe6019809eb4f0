// 64 x 64 tiles of float64 dot products over 64 dims on the matrix cores
// (v_mfma_f64_16x16x4_f64), shared by the block-map, drift-key and
// refinement-gain kernels.
//
// C[i][j] = A_i . B_j for the 64 rows i0 .. i0+63 of A and the 64 rows
// j0 .. j0+63 of B (both [.][64] float64). A workgroup of 256 threads (four
// waves) stages the dims through LDS in two halves of 32; wave w owns the
// 32 x 32 sub-tile at rows 32*(w>>1), columns 32*(w&1) as 2 x 2 MFMA tiles
// of 16 x 16. Operand and result layout of the instruction, per lane l:
// A element [l%16][l/16], B element [l/16][l%16] (k = l/16 of the 4-dim
// step), result element r at [l/16 + 4r][l%16]. The LDS rows are padded to
// 34 doubles, so that the 16 rows x 2 dims a half-wave reads fall in 32
// distinct bank pairs. Each result is a fixed sequence of fused
// multiply-adds over the dims, so repeated calls give identical bits.
#pragma once

#include "ress_internal.h"

namespace ress {

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kTF = 64;      // tile edge
constexpr int kTFHalf = 32;  // dims per LDS stage
constexpr int kTFPad = 34;   // padded LDS row (doubles)

struct TileF64Smem {
  double A[kTF][kTFPad];
  double B[kTF][kTFPad];
};

// Output coordinates of the lane's results: row_of(tr, r), col_of(tc) within
// the 64 x 64 tile.
struct TileF64Map {
  int wr, wc, lr, lc;
  __device__ TileF64Map() {
    const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
    wr = 32 * (w >> 1);
    wc = 32 * (w & 1);
    lr = l >> 4;
    lc = l & 15;
  }
  __device__ int row_of(int tr, int r) const { return wr + 16 * tr + lr + 4 * r; }
  __device__ int col_of(int tc) const { return wc + 16 * tc + lc; }
};

// XCD-aware tile order for a 3-D grid of tiles (x fastest): workgroups go
// round-robin to the 8 XCDs, so the k-th workgroup an XCD receives takes the
// k-th tile of that XCD's contiguous share of the tiles. Neighbouring tiles,
// which read the same operand rows, then run on one XCD and share its L2.
struct TileIdx {
  int x, y, z;
};
__device__ inline TileIdx xcd_tile_order() {
  const int gx = gridDim.x, gy = gridDim.y;
  const int T = gx * gy * gridDim.z;
  const int bid = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const int xcd = bid & 7, k = bid >> 3;
  const int logical = xcd * (T >> 3) + min(xcd, T & 7) + k;
  return TileIdx{logical % gx, (logical / gx) % gy, logical / (gx * gy)};
}

// stage_a(r, d0, x[8]) / stage_b(r, d0, x[8]) return dims d0 .. d0+7 of the
// tile's row r of A / B (callers clamp rows past the end to a valid row).
template <typename StageA, typename StageB>
__device__ inline void mfma_tile_f64(StageA stage_a, StageB stage_b, TileF64Smem& sm,
                                     f64x4 (&acc)[2][2]) {
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int wr = 32 * (w >> 1), wc = 32 * (w & 1);
  const int sr = tid >> 2, sc = (tid & 3) * 8;  // staging: row, first dim
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    double xa[8], xb[8];
    stage_a(sr, kTFHalf * half + sc, xa);
    stage_b(sr, kTFHalf * half + sc, xb);
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      *reinterpret_cast<double2*>(&sm.A[sr][sc + e]) = double2{xa[e], xa[e + 1]};
      *reinterpret_cast<double2*>(&sm.B[sr][sc + e]) = double2{xb[e], xb[e + 1]};
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kTFHalf / 4; ++s) {
      const int k = 4 * s + (l >> 4);
      double av[2], bv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        av[t] = sm.A[wr + 16 * t + (l & 15)][k];
        bv[t] = sm.B[wc + 16 * t + (l & 15)][k];
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[a], bv[b], acc[a][b], 0, 0, 0);
    }
    __syncthreads();
  }
}

}  // namespace ress
