// Exact attention over the kept key blocks ("ReSS: Residual-Restoring Sparse
// Attention for 3D Vision Transformers", §3 step (3): softmax renormalised
// among the selected blocks; dense global attention when every block is
// kept). Flash-style online softmax, bf16 matrix-core contractions with
// float32 accumulation, for gfx950.
//
// Work decomposition: one workgroup per (query block, head); BLK/32 waves,
// each owning 32 query rows. Per kept key block the K tile and the V tile
// are staged in LDS and every wave computes
//   S^T = K Q^T   (v_mfma_f32_32x32x16_bf16; A = K from LDS, B = Q^T held in
//                  registers for the whole kernel)
//   O^T += V^T P^T (A = V^T from LDS, B = P^T taken directly from the S^T
//                  accumulators after the softmax)
// so that each lane owns one query column: the running max, the running sum
// and the rescaling of O are per-lane scalars (the two lane halves holding
// the same query exchange one value per block).
//
// MFMA 32x32x16 operand convention used here: lane l supplies 8 consecutive
// k-slots of row/column (l % 32); lanes l and l+32 cover the two halves of
// the k range. The result accumulator element r of lane l is
// D[8*(r/4) + 4*(l/32) + r%4][l % 32]. Only this output mapping and the
// equal k-slot mapping of A and B matter for correctness; the parity tests
// check them end to end.
#include "ress_internal.h"

namespace ress {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

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
__device__ inline uint4 load_row8(const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  uint4 r;
  r.x = (uint32_t)f32_to_bf16_rne(a.x) | ((uint32_t)f32_to_bf16_rne(a.y) << 16);
  r.y = (uint32_t)f32_to_bf16_rne(a.z) | ((uint32_t)f32_to_bf16_rne(a.w) << 16);
  r.z = (uint32_t)f32_to_bf16_rne(b.x) | ((uint32_t)f32_to_bf16_rne(b.y) << 16);
  r.w = (uint32_t)f32_to_bf16_rne(b.z) | ((uint32_t)f32_to_bf16_rne(b.w) << 16);
  return r;
}

__device__ inline bf16x8 as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Position of key kk (0..15) inside its 16-key group of the V^T tile: the
// 8 keys a lane half feeds to one MFMA k-step are made contiguous
// (lane half 0: keys 0-3, 8-11; lane half 1: keys 4-7, 12-15).
__device__ inline int vt_pos(int kk) {
  return (kk & 3) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

template <int BLK, typename Tin, typename Tout>
__global__ __launch_bounds__(BLK * 2) void attn_kernel(
    const Tin* __restrict__ Q, const Tin* __restrict__ Kx,
    const Tin* __restrict__ Vx, const int32_t* __restrict__ kept_idx,
    const int32_t* __restrict__ kept_cnt, int k_max, int n, int N, int N_pad,
    float scale, Tout* __restrict__ out, float* __restrict__ lse) {
  constexpr int kThreads = BLK * 2;     // BLK/32 waves of 64
  constexpr int kKT = BLK / 32;         // 32-key tiles per block
  constexpr int kChunksPerRowV = BLK / 8;  // 16-byte chunks per V^T row
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BLK * kD];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kD * BLK];

  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  const size_t head_off = (size_t)h * N_pad * kD;
  const int qrow = i * BLK + 32 * w + l32;

  // Q^T operand: dims 16*ks + 8*half + 0..7 of this lane's query row.
  bf16x8 qb[4];
  {
    const Tin* qp = Q + head_off + (size_t)qrow * kD + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qb[ks] = as_bf16x8(load_row8(qp + 16 * ks));
  }

  f32x16 o[2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;
  const float sl2 = scale * 1.4426950408889634f;  // scale * log2(e)

  int cnt = n;
  const int32_t* list = nullptr;
  if (kept_idx != nullptr) {
    const size_t row = (size_t)h * n + i;
    cnt = kept_cnt[row];
    cnt = cnt < 0 ? 0 : (cnt > k_max ? k_max : cnt);
    list = kept_idx + row * k_max;
  }

  for (int kb = 0; kb < cnt; ++kb) {
    const int j = list ? list[kb] : kb;
    if (j < 0 || j >= n) continue;  // uniform across the workgroup
    __syncthreads();  // previous tiles fully consumed
    // ---- stage K (row-major, XOR-swizzled 16-byte chunks) and V^T
    {
      const Tin* kp = Kx + head_off + (size_t)j * BLK * kD;
      const Tin* vp = Vx + head_off + (size_t)j * BLK * kD;
#pragma unroll
      for (int it = 0; it < (BLK * 8) / kThreads; ++it) {
        const int c = tid + it * kThreads;
        const int key = c >> 3, ch = c & 7;
        // padded keys (last block only) are staged as zeros: their scores
        // are masked below, and a zero V row keeps 0 * garbage out of O
        const bool live = j * BLK + key < N;
        uint4 kv = make_uint4(0u, 0u, 0u, 0u), vv = kv;
        if (live) {
          kv = load_row8(kp + (size_t)key * kD + ch * 8);
          vv = load_row8(vp + (size_t)key * kD + ch * 8);
        }
        *reinterpret_cast<uint4*>(&Ks[key * kD + ((ch ^ (key & 7)) * 8)]) = kv;
        const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
        const int pos = (key & ~15) + vt_pos(key & 15);
        const int pch = pos >> 3, pin = pos & 7;
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          const int dim = ch * 8 + dd;
          const int phys = (pch ^ (dim & (kChunksPerRowV - 1))) * 8 + pin;
          Vt[dim * BLK + phys] = (uint16_t)(vw[dd >> 1] >> ((dd & 1) * 16));
        }
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T
    f32x16 s[kKT];
#pragma unroll
    for (int kt = 0; kt < kKT; ++kt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
      const int krow = 32 * kt + l32;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int ch = 2 * ks + half;
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(
            &Ks[krow * kD + ((ch ^ (krow & 7)) * 8)]));
        s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb[ks], s[kt], 0, 0, 0);
      }
    }
    // ---- mask padded keys of the last block
    if (j == n - 1 && N < N_pad) {
      const int base = j * BLK;
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kt + 8 * (r >> 2) + 4 * half + (r & 3);
          if (base + key >= N) s[kt][r] = -INFINITY;
        }
    }
    // ---- online softmax (per lane = per query)
    float mloc = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, s[kt][r]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = exp2f((m_run - m_new) * sl2);
    const float mb = m_new * sl2;
    float psum = 0.f;
    bf16x8 pb[kKT][2];
#pragma unroll
    for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(fmaf(s[kt][r], sl2, -mb));
        psum += p;
        pb[kt][r >> 3][r & 7] = (__bf16)p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    // ---- O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const int dim = 32 * dt + l32;
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const int ch = 2 * (2 * kt + hf) + half;
          const int phys = (ch ^ (dim & (kChunksPerRowV - 1))) * 8;
          const bf16x8 a =
              as_bf16x8(*reinterpret_cast<const uint4*>(&Vt[dim * BLK + phys]));
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kt][hf], o[dt], 0, 0, 0);
        }
    }
  }

  // ---- epilogue
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const bool valid = qrow < N;
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
    if (valid) v = (l_tot > 0.f) ? m_run * scale + logf(l_tot) : -INFINITY;
    lse[(size_t)h * N_pad + qrow] = v;
  }
}

template <typename Tin>
hipError_t launch_t(const Tin* q, const Tin* k, const Tin* v,
                    const ress_shape& s, const int32_t* kept_idx,
                    const int32_t* kept_cnt, int32_t k_max, float scale,
                    void* out, float* lse, hipStream_t st) {
  const int n = s.N_pad / s.B;
  dim3 grid(n, s.H);
  using Tout = Tin;
  Tout* o = static_cast<Tout*>(out);
  if (s.B == 128)
    hipLaunchKernelGGL((attn_kernel<128, Tin, Tout>), grid, dim3(256), 0, st,
                       q, k, v, kept_idx, kept_cnt, k_max, n, s.N, s.N_pad,
                       scale, o, lse);
  else
    hipLaunchKernelGGL((attn_kernel<64, Tin, Tout>), grid, dim3(128), 0, st,
                       q, k, v, kept_idx, kept_cnt, k_max, n, s.N, s.N_pad,
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
  return launch_t(static_cast<const float*>(q), static_cast<const float*>(k),
                  static_cast<const float*>(v), s, kept_idx, kept_cnt, k_max,
                  scale, out, lse, st);
}

}  // namespace ress
