// Exact attention over the kept key blocks for float32 inputs ("ReSS:
// Residual-Restoring Sparse Attention for 3D Vision Transformers", §3 step
// (3): softmax renormalised among the selected blocks; dense when every block
// is kept), on the float32 matrix cores: the products QK^T and PV take the
// float32 values themselves (v_mfma_f32_32x32x2f32), with a float32 online
// softmax, so float32 inputs keep float32 accuracy instead of being rounded
// to bf16. Same contract as the bf16 kernel (attn.hip): one workgroup per
// (query block, head), BLK/32 waves of 32 query rows, key blocks of KBLK
// keys, padded keys masked, padded query rows written as zeros.
//
// MFMA 32x32x2 (float32) operand convention: lane l supplies A[l % 32][l / 32]
// and B[l / 32][l % 32]; accumulator element r of lane l is
// D[8*(r/4) + 4*(l/32) + r%4][l % 32].
//   S^T = K Q^T: A = 32 keys x 2 dims of K (from LDS), B = 2 dims x 32
//   queries of Q^T (registers, the lane's own query row), so lane l ends up
//   with 16 keys of its query column l % 32.
//   O^T += V^T P^T: k-step t pairs key 8*(t/4) + t%4 (lanes 0-31) with the
//   key 4 above it (lanes 32-63), exactly the keys whose weights each lane
//   already holds in its element t, so P^T needs no data movement.
#include "ress_internal.h"

namespace ress {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kD = 64;
// K rows in LDS are padded to 66 floats: a wave's operand read (32 rows at
// dims 2t, 2t+1) then hits 64 distinct banks.
constexpr int kKPad = 66;

__device__ inline float max_halves(float x) {
  return fmaxf(x, __shfl_xor(x, 32, 64));
}

template <int BLK, int KBLK>
__global__ __launch_bounds__(BLK * 2) void attn_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ Kx, const float* __restrict__ Vx,
    const int32_t* __restrict__ kept_idx, const int32_t* __restrict__ kept_cnt, int k_max,
    int n, int N, int N_pad, float scale, float* __restrict__ out, float* __restrict__ lse) {
  constexpr int kThreads = BLK * 2;
  constexpr int kStage = 64;  // key rows staged at a time (34 KB of LDS)
  __shared__ float Ks[kStage * kKPad];
  __shared__ __attribute__((aligned(16))) float Vs[kStage * kD];

  const int i = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l32 = lane & 31, half = lane >> 5;
  const size_t head_off = (size_t)h * N_pad * kD;
  const int qrow = i * BLK + 32 * w + l32;
  const bool qvalid = qrow < N;
  const float sl2 = scale * 1.4426950408889634f;  // scale * log2(e)

  // B operand of S^T = K Q^T: dims 2t + half of this lane's query row
  float qv[32];
  {
    const float* qp = Q + head_off + (size_t)qrow * kD + half;
#pragma unroll
    for (int t = 0; t < 32; ++t) qv[t] = qp[2 * t];
  }
  f32x16 o[2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY;  // running max, scaled log2 units
  float l_run = 0.f;

  int cnt = n;
  const int32_t* list = nullptr;
  if (kept_idx != nullptr) {
    const size_t row = (size_t)h * gridDim.x + i;
    cnt = kept_cnt[row];
    cnt = cnt < 0 ? 0 : (cnt > k_max ? k_max : cnt);
    list = kept_idx + row * k_max;
  }

  for (int kb = 0; kb < cnt; ++kb) {
    const int j = list ? list[kb] : kb;
    if (j < 0 || j >= n) continue;  // invalid entries are skipped (uniform)
#pragma unroll 1
    for (int r0 = 0; r0 < KBLK; r0 += kStage) {
      const int base = j * KBLK + r0;  // first key of this stage
      __syncthreads();                 // the previous stage's tiles are consumed
      // stage 64 key rows of K and V (rows past N read row N-1: finite data
      // whose scores are masked below)
      for (int idx = tid; idx < kStage * (kD / 4); idx += kThreads) {
        const int r = idx / (kD / 4), c = idx % (kD / 4);
        const int rr = min(base + r, N - 1);
        const float4 kv = *reinterpret_cast<const float4*>(Kx + head_off + (size_t)rr * kD + 4 * c);
        const float4 vv = *reinterpret_cast<const float4*>(Vx + head_off + (size_t)rr * kD + 4 * c);
        float* kd = Ks + r * kKPad + 4 * c;
        kd[0] = kv.x; kd[1] = kv.y; kd[2] = kv.z; kd[3] = kv.w;
        *reinterpret_cast<float4*>(Vs + r * kD + 4 * c) = vv;
      }
      __syncthreads();
      const int live_keys = N - base;
#pragma unroll 1
      for (int kt = 0; kt < kStage / 32; ++kt) {
        f32x16 s;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
        const float* ka = Ks + (32 * kt + l32) * kKPad + half;
#pragma unroll
        for (int t = 0; t < 32; ++t)
          s = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[2 * t], qv[t], s, 0, 0, 0);
        // mask padded keys; tile max; online rescale
        float mloc = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * kt + 8 * (r >> 2) + 4 * half + (r & 3);
          if (key >= live_keys) s[r] = -INFINITY;
          mloc = fmaxf(mloc, s[r]);
        }
        mloc = max_halves(mloc) * sl2;
        const float m_new = fmaxf(m_run, mloc);
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
        m_run = m_new;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[r] = m_new == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(fmaf(s[r], sl2, -m_new));
          l_run += s[r];
        }
        // O^T += V^T P^T
#pragma unroll
        for (int t = 0; t < 16; ++t) {
          const int key = 32 * kt + 8 * (t >> 2) + 4 * half + (t & 3);
#pragma unroll
          for (int dt = 0; dt < 2; ++dt)
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(Vs[key * kD + 32 * dt + l32], s[t],
                                                         o[dt], 0, 0, 0);
        }
      }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = (qvalid && l_tot > 0.f) ? 1.f / l_tot : 0.f;
  float* op = out + head_off + (size_t)qrow * kD;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dim = 32 * dt + 8 * g + 4 * half;
      float4 x;
      x.x = inv != 0.f ? o[dt][4 * g] * inv : 0.f;
      x.y = inv != 0.f ? o[dt][4 * g + 1] * inv : 0.f;
      x.z = inv != 0.f ? o[dt][4 * g + 2] * inv : 0.f;
      x.w = inv != 0.f ? o[dt][4 * g + 3] * inv : 0.f;
      *reinterpret_cast<float4*>(op + dim) = x;
    }
  if (lse != nullptr && half == 0) {
    float v = 0.f;
    if (qvalid) v = (l_tot > 0.f) ? m_run * 0.6931471805599453f + logf(l_tot) : -INFINITY;
    lse[(size_t)h * N_pad + qrow] = v;
  }
}

}  // namespace

hipError_t launch_attn_f32(const float* q, const float* k, const float* v, const ress_shape& s,
                           const int32_t* kept_idx, const int32_t* kept_cnt, int32_t k_max,
                           float scale, float* out, float* lse, hipStream_t st) {
  const int nk = n_kblocks(s);
  dim3 grid(n_qblocks(s), s.H);
  if (s.B == 128 && key_block(s) == 128)
    hipLaunchKernelGGL((attn_f32_kernel<128, 128>), grid, dim3(256), 0, st, q, k, v, kept_idx,
                       kept_cnt, k_max, nk, s.N, s.N_pad, scale, out, lse);
  else if (s.B == 128)
    hipLaunchKernelGGL((attn_f32_kernel<128, 64>), grid, dim3(256), 0, st, q, k, v, kept_idx,
                       kept_cnt, k_max, nk, s.N, s.N_pad, scale, out, lse);
  else
    hipLaunchKernelGGL((attn_f32_kernel<64, 64>), grid, dim3(128), 0, st, q, k, v, kept_idx,
                       kept_cnt, k_max, nk, s.N, s.N_pad, scale, out, lse);
  return hipGetLastError();
}

}  // namespace ress
