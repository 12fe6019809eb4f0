// Internal declarations shared by the libress kernels and its host layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ress.h"

namespace ress {

// Block counts of a shape: n_q = N_pad / B query blocks of B tokens and
// n_k = ceil(N / Bk) key blocks of Bk tokens (Bk = 0 means Bk = B).
inline int key_block(const ress_shape& s) { return s.Bk > 0 ? s.Bk : s.B; }
inline int n_qblocks(const ress_shape& s) { return s.N_pad / s.B; }
inline int n_kblocks(const ress_shape& s) {
  const int bk = key_block(s);
  return (s.N + bk - 1) / bk;
}

// Always-kept key blocks as a bitmask (n <= 4096 -> 64 words) and per-head
// keep budgets; small enough to travel in the kernel arguments, so the
// selection kernels need no extra device memory.
struct SelConfig {
  uint64_t always_bits[RESS_MAX_BLOCKS / 64];
  int32_t keep[RESS_MAX_SEL_HEADS];
  int32_t n_always;
};

__host__ __device__ inline bool sel_always(const SelConfig& c, int j) {
  return (c.always_bits[j >> 6] >> (j & 63)) & 1ull;
}
// The same flag where each lane of a wave asks for block j = 64 q + lane, q
// the same in every lane: the bitmask word is read once for the wave (a
// scalar load from the kernel arguments) instead of by a vector load in each
// lane, which a per-key loop would otherwise wait for key by key.
__device__ inline bool sel_always_wave(const SelConfig& c, int j) {
  const int q = __builtin_amdgcn_readfirstlane(j >> 6) & (RESS_MAX_BLOCKS / 64 - 1);
  return (c.always_bits[q] >> (j & 63)) & 1ull;
}

// 64-bit key whose unsigned order is the float64 order (-0 counted as +0).
__device__ inline uint64_t order_key(double x) {
  if (x == 0.0) x = 0.0;
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

// Fixed-order (butterfly) sums over one wave of 64 lanes; every lane gets
// the result.
__device__ inline double wave_sum64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ inline int wave_isum64(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Orders the LDS accesses of one wave (all lanes) before the ones after it.
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Launchers (defined next to their kernels). Each returns hipGetLastError()
// of its launches.
// Pools up to three tensors of one dtype in blocks of `blk` tokens in one
// launch; job a has nb blocks (the last one partial when N is not a
// multiple of blk).
struct PoolJob {
  const void* x;
  double* out;
  int nb;
};
struct PoolJobs {
  PoolJob job[3];
  int count;
};
hipError_t launch_block_pool(const PoolJobs& jobs, int dtype, const ress_shape& s, int blk,
                             hipStream_t st);

hipError_t launch_block_map(const double* qpool, const double* kpool,
                            const ress_shape& s, double scale, double* P,
                            hipStream_t st);

hipError_t launch_copy(const double* src, double* dst, size_t count,
                       hipStream_t st);

hipError_t launch_vmv(const double* vpool, const double* M,
                      const ress_shape& s, double* vmv, hipStream_t st);

hipError_t launch_drift(const double* P, const double* vpool, const double* M,
                        const double* vmv, const ress_shape& s, double eps,
                        double* key, double* vout, hipStream_t st);

hipError_t launch_topk(const double* key, const ress_shape& s,
                       const SelConfig& cfg, int32_t k_max, int32_t* kept_idx,
                       int32_t* kept_cnt, hipStream_t st);

hipError_t launch_cdf(const double* P, const ress_shape& s, const SelConfig& cfg,
                      double tau, int32_t k_max, int32_t* kept_idx,
                      int32_t* kept_cnt, hipStream_t st);

hipError_t launch_refine(const double* P, const double* key,
                         const double* vpool, const double* vout,
                         const double* M, const ress_shape& s,
                         const SelConfig& cfg, int32_t rounds, double rho,
                         double eps, int32_t k_max, int32_t* kept_idx,
                         int32_t* kept_cnt, double* J_init, double* J_final,
                         void* workspace, hipStream_t st);

// Bytes of the refinement workspace for a shape (the per-row state of all
// rows of all heads, in HBM).
size_t refine_workspace_bytes(const ress_shape& s);

// The same refinement with every round of a tile of rows on chip (no
// workspace); rows of at most refine_fused_max_blocks() key blocks.
hipError_t launch_refine_fused(const double* P, const double* key, const double* vpool,
                               const double* vout, const double* M, const ress_shape& s,
                               const SelConfig& cfg, int32_t rounds, double rho, double eps,
                               int32_t k_max, int32_t* kept_idx, int32_t* kept_cnt,
                               double* J_init, double* J_final, hipStream_t st);
int refine_fused_max_blocks();
// Drift scoring, top-k and the refinement in one kernel from the pooled
// blocks (the pooled form of refine_fused.hip); the same row limit. vmv must
// hold V_j^T M V_j already (launch_vmv).
hipError_t launch_select_refine_fused(const double* qpool, const double* kpool,
                                      const double* vpool, const double* M, const double* vmv,
                                      const ress_shape& s, const SelConfig& cfg, double scale,
                                      int32_t rounds, double rho, double eps, int32_t k_max,
                                      int32_t* kept_idx, int32_t* kept_cnt, double* J_init,
                                      double* J_final, hipStream_t st);

hipError_t launch_gram(const void* w_o, int dtype, int d_model, const ress_shape& s, double* M,
                       hipStream_t st);

hipError_t launch_residual_drift(const void* os, const void* od, int dtype, const double* M,
                                 const ress_shape& s, double* drift, hipStream_t st);

// Device address of this GPU's fixed refinement scratch (noalloc.hip),
// RESS_NOALLOC_SCRATCH_BYTES bytes, 256-byte aligned; looked up once per
// device.
hipError_t noalloc_scratch(void** ptr);

// Fused selection, pooled blocks to keep lists (select_fused.hip); rows of
// at most select_fused_max_blocks() key blocks.
int select_fused_max_blocks();
hipError_t launch_select_fused(const double* qpool, const double* kpool, const double* vpool,
                               const double* M, const double* vmv, const ress_shape& s,
                               double scale, double eps, int drift, const SelConfig& cfg,
                               int32_t k_max, int32_t* kept_idx, int32_t* kept_cnt,
                               hipStream_t st);

// QKV projection and output projection with residual add (proj.hip)
hipError_t launch_qkv_project(const uint16_t* x, const uint16_t* w_qkv, const uint16_t* b_qkv,
                              int d_model, const ress_shape& s, uint16_t* q, uint16_t* k,
                              uint16_t* v, hipStream_t st);
hipError_t launch_out_project(const uint16_t* o, const uint16_t* w_o, const uint16_t* b_o,
                              const uint16_t* residual, int d_model, const ress_shape& s,
                              uint16_t* y, hipStream_t st);

// float32 inputs: float32 matrix cores (attn_f32.hip)
hipError_t launch_attn_f32(const float* q, const float* k, const float* v, const ress_shape& s,
                           const int32_t* kept_idx, const int32_t* kept_cnt, int32_t k_max,
                           float scale, float* out, float* lse, hipStream_t st);
hipError_t launch_attn(const void* q, const void* k, const void* v, int dtype,
                       const ress_shape& s, const int32_t* kept_idx,
                       const int32_t* kept_cnt, int32_t k_max, float scale,
                       void* out, float* lse, hipStream_t st);

}  // namespace ress
