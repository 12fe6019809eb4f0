// libress host layer: argument validation, then kernel launches on the
// caller's stream. Validation runs before any HIP call, so every invalid
// argument is reported without touching the device; nothing is launched on
// error. No exception leaves this file.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "ress_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return RESS_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define REQUIRE_PTR(p)                                                   \
  do {                                                                   \
    if ((p) == nullptr) return fail(RESS_ERR_INVALID_ARG, #p " is NULL"); \
    if (!aligned16(p))                                                   \
      return fail(RESS_ERR_INVALID_ARG, #p " is not 16-byte aligned");   \
  } while (0)

#define OPTIONAL_PTR(p)                                                  \
  do {                                                                   \
    if ((p) != nullptr && !aligned16(p))                                 \
      return fail(RESS_ERR_INVALID_ARG, #p " is not 16-byte aligned");   \
  } while (0)

int check_shape(const ress_shape& s) {
  if (s.H < 1) return fail(RESS_ERR_INVALID_ARG, "H=%d must be >= 1", s.H);
  if (s.D != 64)
    return fail(RESS_ERR_UNSUPPORTED, "D=%d: only head dimension 64", s.D);
  if (s.B != 64 && s.B != 128)
    return fail(RESS_ERR_UNSUPPORTED, "B=%d: block size must be 64 or 128",
                s.B);
  if (s.N_pad < 1 || s.N_pad % s.B != 0)
    return fail(RESS_ERR_INVALID_ARG, "N_pad=%d is not a positive multiple of B=%d",
                s.N_pad, s.B);
  if (s.N < 1 || s.N > s.N_pad || s.N_pad - s.N >= s.B)
    return fail(RESS_ERR_INVALID_ARG,
                "N=%d must satisfy N_pad-B < N <= N_pad (N_pad=%d, B=%d)", s.N,
                s.N_pad, s.B);
  if (s.Bk != 0 && ((s.Bk != 64 && s.Bk != 128) || s.Bk > s.B))
    return fail(RESS_ERR_UNSUPPORTED,
                "Bk=%d: key block size must be 0 (= B), or 64 or 128 and at most B=%d",
                s.Bk, s.B);
  const int nq = ress::n_qblocks(s), nk = ress::n_kblocks(s);
  if (nq > RESS_MAX_BLOCKS || nk > RESS_MAX_BLOCKS)
    return fail(RESS_ERR_UNSUPPORTED, "n_q=%d / n_k=%d blocks exceed the cap of %d", nq, nk,
                RESS_MAX_BLOCKS);
  // element counts of the largest tensors must fit the 64-bit offsets used
  // in the kernels; [H][n_q][n_k] maps below 2^40 elements are far inside.
  if ((double)s.H * nq * nk > 1e12)
    return fail(RESS_ERR_UNSUPPORTED, "H*n_q*n_k too large");
  return RESS_OK;
}

int check_dtype(int dtype) {
  if (dtype != RESS_DTYPE_BF16 && dtype != RESS_DTYPE_F32)
    return fail(RESS_ERR_INVALID_ARG, "bad dtype %d", dtype);
  return RESS_OK;
}

// Budgets and always-kept flags (host arrays) -> kernel-argument config.
int make_sel_config(const ress_shape& s, const int32_t* keep,
                    const uint8_t* always_keep, int32_t k_max,
                    ress::SelConfig* cfg) {
  if (keep == nullptr) return fail(RESS_ERR_INVALID_ARG, "keep is NULL");
  if (s.H > RESS_MAX_SEL_HEADS)
    return fail(RESS_ERR_UNSUPPORTED, "H=%d exceeds %d heads for selection",
                s.H, RESS_MAX_SEL_HEADS);
  const int n = ress::n_kblocks(s);  // flags and budgets count key blocks
  memset(cfg, 0, sizeof *cfg);
  int n_always = 0;
  if (always_keep != nullptr) {
    for (int j = 0; j < n; ++j) {
      if (always_keep[j] > 1)
        return fail(RESS_ERR_INVALID_ARG, "always_keep[%d]=%d is not 0 or 1",
                    j, always_keep[j]);
      if (always_keep[j]) {
        cfg->always_bits[j >> 6] |= 1ull << (j & 63);
        ++n_always;
      }
    }
  }
  cfg->n_always = n_always;
  int kmax_needed = 0;
  for (int h = 0; h < s.H; ++h) {
    const int k = keep[h];
    if (k < 2 || k > n)
      return fail(RESS_ERR_INVALID_ARG, "keep[%d]=%d must lie in [2, n_k=%d]", h,
                  k, n);
    if (k <= n_always)
      return fail(RESS_ERR_INVALID_ARG,
                  "keep[%d]=%d must exceed the %d always-kept blocks", h, k,
                  n_always);
    cfg->keep[h] = k;
    if (k > kmax_needed) kmax_needed = k;
  }
  if (k_max < kmax_needed || k_max > n)
    return fail(RESS_ERR_INVALID_ARG, "k_max=%d must lie in [max keep=%d, n_k=%d]",
                k_max, kmax_needed, n);
  return RESS_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(RESS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

int ress_version(void) { return RESS_VERSION; }

const char* ress_last_error(void) { return g_err.c_str(); }

int ress_block_pool(const void* q, const void* k, const void* v, int dtype,
                    ress_shape shape, double* qpool, double* kpool,
                    double* vpool, void* stream) {
  int rc;
  if ((rc = check_shape(shape)) != RESS_OK) return rc;
  if ((rc = check_dtype(dtype)) != RESS_OK) return rc;
  const void* in[3] = {q, k, v};
  double* out[3] = {qpool, kpool, vpool};
  const char* names[3] = {"q/qpool", "k/kpool", "v/vpool"};
  int given = 0;
  for (int a = 0; a < 3; ++a) {
    if ((in[a] == nullptr) != (out[a] == nullptr))
      return fail(RESS_ERR_INVALID_ARG, "%s: input and output must both be given or both be NULL",
                  names[a]);
    if (in[a] != nullptr) {
      if (!aligned16(in[a]) || !aligned16(out[a]))
        return fail(RESS_ERR_INVALID_ARG, "%s: pointer not 16-byte aligned", names[a]);
      ++given;
    }
  }
  if (given == 0) return fail(RESS_ERR_INVALID_ARG, "nothing to pool");
  hipStream_t st = static_cast<hipStream_t>(stream);
  // queries in blocks of B, keys and values in blocks of Bk: one launch per
  // distinct block size (a single one on square grids)
  const int blk[3] = {shape.B, ress::key_block(shape), ress::key_block(shape)};
  const int nb[3] = {ress::n_qblocks(shape), ress::n_kblocks(shape), ress::n_kblocks(shape)};
  for (const int size : {shape.B, ress::key_block(shape)}) {
    ress::PoolJobs jobs{};
    for (int a = 0; a < 3; ++a)
      if (in[a] != nullptr && blk[a] == size) jobs.job[jobs.count++] = {in[a], out[a], nb[a]};
    hipError_t e = ress::launch_block_pool(jobs, dtype, shape, size, st);
    if (e != hipSuccess) return hip_status(e, "block_pool launch");
    if (size == ress::key_block(shape)) break;  // square grid: one size only
  }
  return ok();
}

int ress_block_score(const double* qpool, const double* kpool,
                     const double* vpool, const double* M, ress_shape shape,
                     int mode, double scale, double eps, double* P,
                     double* key, double* vout, double* vmv, void* stream) {
  int rc;
  if ((rc = check_shape(shape)) != RESS_OK) return rc;
  if (mode != RESS_SCORE_PROB && mode != RESS_SCORE_DRIFT)
    return fail(RESS_ERR_INVALID_ARG, "bad score mode %d", mode);
  if (!(scale > 0.0) || !isfinite(scale))
    return fail(RESS_ERR_INVALID_ARG, "scale must be finite and > 0");
  REQUIRE_PTR(qpool);
  REQUIRE_PTR(kpool);
  REQUIRE_PTR(P);
  OPTIONAL_PTR(key);
  if (mode == RESS_SCORE_DRIFT) {
    if (!(eps > 0.0) || !isfinite(eps))
      return fail(RESS_ERR_INVALID_ARG, "eps must be finite and > 0");
    REQUIRE_PTR(vpool);
    REQUIRE_PTR(key);
    REQUIRE_PTR(vout);
    REQUIRE_PTR(vmv);
    OPTIONAL_PTR(M);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = ress::launch_block_map(qpool, kpool, shape, scale, P, st);
  if (e != hipSuccess) return hip_status(e, "block_map launch");
  if (mode == RESS_SCORE_PROB) {
    if (key != nullptr && key != P) {
      e = ress::launch_copy(P, key,
                            (size_t)shape.H * ress::n_qblocks(shape) * ress::n_kblocks(shape), st);
      if (e != hipSuccess) return hip_status(e, "copy launch");
    }
    return ok();
  }
  e = ress::launch_vmv(vpool, M, shape, vmv, st);
  if (e != hipSuccess) return hip_status(e, "vmv launch");
  e = ress::launch_drift(P, vpool, M, vmv, shape, eps, key, vout, st);
  if (e != hipSuccess) return hip_status(e, "drift launch");
  return ok();
}

int ress_select_topk(const double* key, ress_shape shape, const int32_t* keep,
                     const uint8_t* always_keep, int32_t k_max,
                     int32_t* kept_idx, int32_t* kept_cnt, void* stream) {
  int rc;
  if ((rc = check_shape(shape)) != RESS_OK) return rc;
  REQUIRE_PTR(key);
  REQUIRE_PTR(kept_idx);
  REQUIRE_PTR(kept_cnt);
  ress::SelConfig cfg;
  if ((rc = make_sel_config(shape, keep, always_keep, k_max, &cfg)) != RESS_OK)
    return rc;
  hipError_t e = ress::launch_topk(key, shape, cfg, k_max, kept_idx, kept_cnt,
                                   static_cast<hipStream_t>(stream));
  return hip_status(e, "topk launch");
}

int ress_select_cdf(const double* P, ress_shape shape, const int32_t* keep,
                    const uint8_t* always_keep, double tau, int32_t k_max,
                    int32_t* kept_idx, int32_t* kept_cnt, void* stream) {
  int rc;
  if ((rc = check_shape(shape)) != RESS_OK) return rc;
  REQUIRE_PTR(P);
  REQUIRE_PTR(kept_idx);
  REQUIRE_PTR(kept_cnt);
  if (!(tau > 0.0) || !isfinite(tau))
    return fail(RESS_ERR_INVALID_ARG, "tau must be finite and > 0");
  ress::SelConfig cfg;
  if ((rc = make_sel_config(shape, keep, always_keep, k_max, &cfg)) != RESS_OK)
    return rc;
  hipError_t e = ress::launch_cdf(P, shape, cfg, tau, k_max, kept_idx, kept_cnt,
                                  static_cast<hipStream_t>(stream));
  return hip_status(e, "cdf launch");
}

int ress_select_fused(const double* qpool, const double* kpool, const double* vpool,
                      const double* M, ress_shape shape, int mode, double scale, double eps,
                      const int32_t* keep, const uint8_t* always_keep, int32_t k_max,
                      double* vmv, int32_t* kept_idx, int32_t* kept_cnt, void* stream) {
  int rc;
  if ((rc = check_shape(shape)) != RESS_OK) return rc;
  if (mode != RESS_SCORE_PROB && mode != RESS_SCORE_DRIFT)
    return fail(RESS_ERR_INVALID_ARG, "bad score mode %d", mode);
  if (ress::n_kblocks(shape) > ress::select_fused_max_blocks())
    return fail(RESS_ERR_UNSUPPORTED, "n_k=%d key blocks exceed the %d of the fused selection",
                ress::n_kblocks(shape), ress::select_fused_max_blocks());
  REQUIRE_PTR(qpool);
  REQUIRE_PTR(kpool);
  REQUIRE_PTR(kept_idx);
  REQUIRE_PTR(kept_cnt);
  OPTIONAL_PTR(M);
  const bool drift = mode == RESS_SCORE_DRIFT;
  if (drift) {
    REQUIRE_PTR(vpool);
    REQUIRE_PTR(vmv);
  }
  if (!(scale > 0.0) || !isfinite(scale))
    return fail(RESS_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (drift && (!(eps > 0.0) || !isfinite(eps)))
    return fail(RESS_ERR_INVALID_ARG, "eps must be finite and > 0");
  ress::SelConfig cfg;
  if ((rc = make_sel_config(shape, keep, always_keep, k_max, &cfg)) != RESS_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (drift) e = ress::launch_vmv(vpool, M, shape, vmv, st);
  if (e == hipSuccess)
    e = ress::launch_select_fused(qpool, kpool, drift ? vpool : nullptr, M, drift ? vmv : nullptr,
                                  shape, scale, eps, drift ? 1 : 0, cfg, k_max, kept_idx,
                                  kept_cnt, st);
  return hip_status(e, "fused selection launch");
}

int ress_refine_dropset(const double* P, const double* key,
                        const double* vpool, const double* vout,
                        const double* M, ress_shape shape, const int32_t* keep,
                        const uint8_t* always_keep, int32_t rounds, double rho,
                        double eps, int32_t k_max, int32_t* kept_idx,
                        int32_t* kept_cnt, double* J_init, double* J_final,
                        void* workspace, size_t workspace_bytes, void* stream) {
  int rc;
  if ((rc = check_shape(shape)) != RESS_OK) return rc;
  if (workspace == nullptr) return fail(RESS_ERR_INVALID_ARG, "workspace is NULL");
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(RESS_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  if (workspace_bytes < ress::refine_workspace_bytes(shape))
    return fail(RESS_ERR_INVALID_ARG, "workspace of %zu bytes is smaller than the %zu needed",
                workspace_bytes, ress::refine_workspace_bytes(shape));
  REQUIRE_PTR(P);
  REQUIRE_PTR(key);
  REQUIRE_PTR(vpool);
  REQUIRE_PTR(vout);
  OPTIONAL_PTR(M);
  REQUIRE_PTR(kept_idx);
  REQUIRE_PTR(kept_cnt);
  OPTIONAL_PTR(J_init);
  OPTIONAL_PTR(J_final);
  if (rounds < 0) return fail(RESS_ERR_INVALID_ARG, "rounds=%d < 0", rounds);
  if (!(rho > 0.0 && rho <= 1.0))
    return fail(RESS_ERR_INVALID_ARG, "rho must lie in (0, 1]");
  if (!(eps > 0.0) || !isfinite(eps))
    return fail(RESS_ERR_INVALID_ARG, "eps must be finite and > 0");
  ress::SelConfig cfg;
  if ((rc = make_sel_config(shape, keep, always_keep, k_max, &cfg)) != RESS_OK)
    return rc;
  hipError_t e = ress::launch_refine(P, key, vpool, vout, M, shape, cfg, rounds,
                                     rho, eps, k_max, kept_idx, kept_cnt,
                                     J_init, J_final, workspace,
                                     static_cast<hipStream_t>(stream));
  return hip_status(e, "refine launch");
}

int ress_refine_dropset_fused(const double* P, const double* key, const double* vpool,
                              const double* vout, const double* M, ress_shape shape,
                              const int32_t* keep, const uint8_t* always_keep, int32_t rounds,
                              double rho, double eps, int32_t k_max, int32_t* kept_idx,
                              int32_t* kept_cnt, double* J_init, double* J_final,
                              void* stream) {
  int rc;
  if ((rc = check_shape(shape)) != RESS_OK) return rc;
  if (ress::n_kblocks(shape) > ress::refine_fused_max_blocks())
    return fail(RESS_ERR_UNSUPPORTED, "n_k=%d key blocks exceed the %d of the fused refinement",
                ress::n_kblocks(shape), ress::refine_fused_max_blocks());
  REQUIRE_PTR(P);
  REQUIRE_PTR(key);
  REQUIRE_PTR(vpool);
  REQUIRE_PTR(vout);
  OPTIONAL_PTR(M);
  REQUIRE_PTR(kept_idx);
  REQUIRE_PTR(kept_cnt);
  OPTIONAL_PTR(J_init);
  OPTIONAL_PTR(J_final);
  if (rounds < 0) return fail(RESS_ERR_INVALID_ARG, "rounds=%d < 0", rounds);
  if (!(rho > 0.0 && rho <= 1.0))
    return fail(RESS_ERR_INVALID_ARG, "rho must lie in (0, 1]");
  if (!(eps > 0.0) || !isfinite(eps))
    return fail(RESS_ERR_INVALID_ARG, "eps must be finite and > 0");
  ress::SelConfig cfg;
  if ((rc = make_sel_config(shape, keep, always_keep, k_max, &cfg)) != RESS_OK)
    return rc;
  hipError_t e = ress::launch_refine_fused(P, key, vpool, vout, M, shape, cfg, rounds, rho, eps,
                                           k_max, kept_idx, kept_cnt, J_init, J_final,
                                           static_cast<hipStream_t>(stream));
  return hip_status(e, "fused refine launch");
}

int ress_select_refine_fused(const double* qpool, const double* kpool, const double* vpool,
                             const double* M, ress_shape shape, double scale, double eps,
                             const int32_t* keep, const uint8_t* always_keep, int32_t rounds,
                             double rho, int32_t k_max, double* vmv, int32_t* kept_idx,
                             int32_t* kept_cnt, double* J_init, double* J_final, void* stream) {
  int rc;
  if ((rc = check_shape(shape)) != RESS_OK) return rc;
  if (ress::n_kblocks(shape) > ress::refine_fused_max_blocks())
    return fail(RESS_ERR_UNSUPPORTED,
                "n_k=%d key blocks exceed the %d of the fused selection with refinement",
                ress::n_kblocks(shape), ress::refine_fused_max_blocks());
  REQUIRE_PTR(qpool);
  REQUIRE_PTR(kpool);
  REQUIRE_PTR(vpool);
  REQUIRE_PTR(vmv);
  OPTIONAL_PTR(M);
  REQUIRE_PTR(kept_idx);
  REQUIRE_PTR(kept_cnt);
  OPTIONAL_PTR(J_init);
  OPTIONAL_PTR(J_final);
  if (!(scale > 0.0) || !isfinite(scale))
    return fail(RESS_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (!(eps > 0.0) || !isfinite(eps))
    return fail(RESS_ERR_INVALID_ARG, "eps must be finite and > 0");
  if (rounds < 0) return fail(RESS_ERR_INVALID_ARG, "rounds=%d < 0", rounds);
  if (!(rho > 0.0 && rho <= 1.0))
    return fail(RESS_ERR_INVALID_ARG, "rho must lie in (0, 1]");
  ress::SelConfig cfg;
  if ((rc = make_sel_config(shape, keep, always_keep, k_max, &cfg)) != RESS_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = ress::launch_vmv(vpool, M, shape, vmv, st);
  if (e == hipSuccess)
    e = ress::launch_select_refine_fused(qpool, kpool, vpool, M, vmv, shape, cfg, scale, rounds,
                                         rho, eps, k_max, kept_idx, kept_cnt, J_init, J_final,
                                         st);
  return hip_status(e, "fused selection with refinement launch");
}

int ress_refine_dropset_noalloc(const double* P, const double* key, const double* vpool,
                                const double* vout, const double* M, ress_shape shape,
                                const int32_t* keep, const uint8_t* always_keep, int32_t rounds,
                                double rho, double eps, int32_t k_max, int32_t* kept_idx,
                                int32_t* kept_cnt, double* J_init, double* J_final,
                                void* stream) {
  int rc;
  if ((rc = check_shape(shape)) != RESS_OK) return rc;
  REQUIRE_PTR(P);
  REQUIRE_PTR(key);
  REQUIRE_PTR(vpool);
  REQUIRE_PTR(vout);
  OPTIONAL_PTR(M);
  REQUIRE_PTR(kept_idx);
  REQUIRE_PTR(kept_cnt);
  OPTIONAL_PTR(J_init);
  OPTIONAL_PTR(J_final);
  if (rounds < 0) return fail(RESS_ERR_INVALID_ARG, "rounds=%d < 0", rounds);
  if (!(rho > 0.0 && rho <= 1.0))
    return fail(RESS_ERR_INVALID_ARG, "rho must lie in (0, 1]");
  if (!(eps > 0.0) || !isfinite(eps))
    return fail(RESS_ERR_INVALID_ARG, "eps must be finite and > 0");
  ress::SelConfig cfg;
  if ((rc = make_sel_config(shape, keep, always_keep, k_max, &cfg)) != RESS_OK) return rc;
  // heads per group: the most whose refinement state fits the scratch
  const size_t cap = RESS_NOALLOC_SCRATCH_BYTES;
  int group = 0;
  for (int g = shape.H; g >= 1; --g) {
    ress_shape sg = shape;
    sg.H = g;
    if (ress::refine_workspace_bytes(sg) <= cap) {
      group = g;
      break;
    }
  }
  if (group == 0) {
    ress_shape s1 = shape;
    s1.H = 1;
    return fail(RESS_ERR_UNSUPPORTED,
                "one head's refinement state takes %zu bytes, more than the %zu of the scratch",
                ress::refine_workspace_bytes(s1), cap);
  }
  void* scratch = nullptr;
  hipError_t e = ress::noalloc_scratch(&scratch);
  if (e != hipSuccess) return hip_status(e, "scratch address");
  const size_t nq = ress::n_qblocks(shape), nk = ress::n_kblocks(shape), D = shape.D;
  for (int h0 = 0; h0 < shape.H; h0 += group) {
    ress_shape sg = shape;
    sg.H = shape.H - h0 < group ? shape.H - h0 : group;
    ress::SelConfig cg;
    if ((rc = make_sel_config(sg, keep + h0, always_keep, k_max, &cg)) != RESS_OK) return rc;
    const size_t hq = (size_t)h0 * nq;
    e = ress::launch_refine(P + hq * nk, key + hq * nk, vpool + (size_t)h0 * nk * D,
                            vout + hq * D, M ? M + (size_t)h0 * D * D : nullptr, sg, cg, rounds,
                            rho, eps, k_max, kept_idx + hq * k_max, kept_cnt + hq,
                            J_init ? J_init + hq : nullptr, J_final ? J_final + hq : nullptr,
                            scratch, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_status(e, "noalloc refine launch");
  }
  return ok();
}

namespace {

int check_projection(int dtype, int32_t d_model) {
  if (dtype != RESS_DTYPE_BF16)
    return dtype == RESS_DTYPE_F32 ? fail(RESS_ERR_UNSUPPORTED, "projections take bf16 only")
                                   : fail(RESS_ERR_INVALID_ARG, "bad dtype %d", dtype);
  if (d_model < 64 || d_model % 64 != 0 || d_model > 65536)
    return fail(RESS_ERR_INVALID_ARG, "d_model=%d must be a positive multiple of 64, <= 65536",
                d_model);
  return RESS_OK;
}

}  // namespace

int ress_qkv_project(const void* x, const void* w_qkv, const void* b_qkv, int dtype,
                     int32_t d_model, ress_shape shape, void* q, void* k, void* v,
                     void* stream) {
  int rc;
  if ((rc = check_shape(shape)) != RESS_OK) return rc;
  if ((rc = check_projection(dtype, d_model)) != RESS_OK) return rc;
  REQUIRE_PTR(x);
  REQUIRE_PTR(w_qkv);
  OPTIONAL_PTR(b_qkv);
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  hipError_t e = ress::launch_qkv_project(
      static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w_qkv),
      static_cast<const uint16_t*>(b_qkv), d_model, shape, static_cast<uint16_t*>(q),
      static_cast<uint16_t*>(k), static_cast<uint16_t*>(v), static_cast<hipStream_t>(stream));
  return hip_status(e, "qkv projection launch");
}

int ress_out_project(const void* o, const void* w_o, const void* b_o, const void* residual,
                     int dtype, int32_t d_model, ress_shape shape, void* y, void* stream) {
  int rc;
  if ((rc = check_shape(shape)) != RESS_OK) return rc;
  if ((rc = check_projection(dtype, d_model)) != RESS_OK) return rc;
  REQUIRE_PTR(o);
  REQUIRE_PTR(w_o);
  OPTIONAL_PTR(b_o);
  OPTIONAL_PTR(residual);
  REQUIRE_PTR(y);
  if (y == o || y == w_o) return fail(RESS_ERR_INVALID_ARG, "y must not alias o or w_o");
  hipError_t e = ress::launch_out_project(
      static_cast<const uint16_t*>(o), static_cast<const uint16_t*>(w_o),
      static_cast<const uint16_t*>(b_o), static_cast<const uint16_t*>(residual), d_model, shape,
      static_cast<uint16_t*>(y), static_cast<hipStream_t>(stream));
  return hip_status(e, "output projection launch");
}

size_t ress_refine_workspace_size(ress_shape shape) {
  if (check_shape(shape) != RESS_OK) return 0;
  ok();
  return ress::refine_workspace_bytes(shape);
}

int ress_head_budgets(const double* score, int32_t H, int32_t n_k, const uint8_t* always_keep,
                      int64_t total_keep, int32_t* keep) {
  if (H < 1 || H > RESS_MAX_SEL_HEADS)
    return fail(RESS_ERR_INVALID_ARG, "H=%d must lie in [1, %d]", H, RESS_MAX_SEL_HEADS);
  if (n_k < 2 || n_k > RESS_MAX_BLOCKS)
    return fail(RESS_ERR_INVALID_ARG, "n_k=%d must lie in [2, %d]", n_k, RESS_MAX_BLOCKS);
  if (score == nullptr || keep == nullptr)
    return fail(RESS_ERR_INVALID_ARG, "score and keep are required");
  int n_always = 0;
  if (always_keep != nullptr)
    for (int j = 0; j < n_k; ++j) {
      if (always_keep[j] > 1)
        return fail(RESS_ERR_INVALID_ARG, "always_keep[%d]=%d is not 0 or 1", j, always_keep[j]);
      n_always += always_keep[j];
    }
  const int cap = n_k - n_always;                         // candidates per row
  const int floor_c = n_always >= 2 ? 1 : 2 - n_always;   // two kept blocks, one candidate
  if (cap < floor_c)
    return fail(RESS_ERR_INVALID_ARG, "no room for candidates (n_k=%d, %d always kept)", n_k,
                n_always);
  for (int h = 0; h < H; ++h)
    if (!(score[h] >= 0.0) || !isfinite(score[h]))
      return fail(RESS_ERR_INVALID_ARG, "score[%d] must be finite and >= 0", h);
  const int64_t lo = (int64_t)H * (n_always + floor_c), hi = (int64_t)H * n_k;
  if (total_keep < lo || total_keep > hi)
    return fail(RESS_ERR_INVALID_ARG, "total_keep=%lld must lie in [%lld, %lld]",
                (long long)total_keep, (long long)lo, (long long)hi);
  // every head gets the floor; the surplus U goes in proportion to the
  // scores, clipped at cap - floor, the excess of clipped heads spread over
  // the others until no head exceeds the cap
  const double U = (double)(total_keep - lo);
  const double capU = (double)(cap - floor_c);
  double a[RESS_MAX_SEL_HEADS];
  bool clipped[RESS_MAX_SEL_HEADS];
  for (int h = 0; h < H; ++h) clipped[h] = false;
  for (;;) {
    double S = 0.0, R = U;
    int active = 0;
    for (int h = 0; h < H; ++h) {
      if (clipped[h]) {
        R -= capU;
      } else {
        S += score[h];
        ++active;
      }
    }
    bool over = false;
    for (int h = 0; h < H; ++h) {
      if (clipped[h]) continue;
      a[h] = S > 0.0 ? R * score[h] / S : R / (double)active;
      if (a[h] > capU) over = true;
    }
    if (!over) break;
    for (int h = 0; h < H; ++h)
      if (!clipped[h] && a[h] > capU) {
        clipped[h] = true;
        a[h] = capU;
      }
  }
  // integers: floors, then one more unit to the largest fractional parts
  // (equal parts: the lower head index), never beyond the cap
  int64_t b[RESS_MAX_SEL_HEADS], given = 0;
  for (int h = 0; h < H; ++h) {
    b[h] = (int64_t)floor(a[h]);
    if (b[h] > (int64_t)capU) b[h] = (int64_t)capU;
    given += b[h];
  }
  int64_t rem = (int64_t)U - given;
  while (rem > 0) {
    int best = -1;
    double bf = -1.0;
    for (int h = 0; h < H; ++h) {
      if (b[h] >= (int64_t)capU) continue;
      const double f = a[h] - floor(a[h]);
      if (f > bf) {
        bf = f;
        best = h;
      }
    }
    if (best < 0) break;  // cannot happen when total_keep <= H * n_k
    ++b[best];
    a[best] = floor(a[best]);  // its fractional part is used up
    --rem;
  }
  for (int h = 0; h < H; ++h) keep[h] = (int32_t)(n_always + floor_c + b[h]);
  return ok();
}

int ress_gram_from_wo(const void* w_o, int dtype, int32_t d_model, ress_shape shape,
                      double* M, void* stream) {
  int rc;
  if ((rc = check_shape(shape)) != RESS_OK) return rc;
  if ((rc = check_dtype(dtype)) != RESS_OK) return rc;
  REQUIRE_PTR(w_o);
  REQUIRE_PTR(M);
  if (d_model < 1 || d_model > (1 << 20))
    return fail(RESS_ERR_INVALID_ARG, "d_model=%d must lie in [1, 2^20]", d_model);
  hipError_t e = ress::launch_gram(w_o, dtype, d_model, shape, M,
                                   static_cast<hipStream_t>(stream));
  return hip_status(e, "gram launch");
}

int ress_residual_drift(const void* out_sparse, const void* out_dense, int dtype,
                        const double* M, ress_shape shape, double* drift, void* stream) {
  int rc;
  if ((rc = check_shape(shape)) != RESS_OK) return rc;
  if ((rc = check_dtype(dtype)) != RESS_OK) return rc;
  REQUIRE_PTR(out_sparse);
  REQUIRE_PTR(out_dense);
  OPTIONAL_PTR(M);
  REQUIRE_PTR(drift);
  hipError_t e = ress::launch_residual_drift(out_sparse, out_dense, dtype, M, shape, drift,
                                             static_cast<hipStream_t>(stream));
  return hip_status(e, "residual drift launch");
}

int ress_sparse_attn_fwd(const void* q, const void* k, const void* v,
                         int dtype, ress_shape shape, const int32_t* kept_idx,
                         const int32_t* kept_cnt, int32_t k_max, float scale,
                         void* out, float* lse, void* stream) {
  int rc;
  if ((rc = check_shape(shape)) != RESS_OK) return rc;
  if ((rc = check_dtype(dtype)) != RESS_OK) return rc;
  REQUIRE_PTR(q);
  REQUIRE_PTR(k);
  REQUIRE_PTR(v);
  REQUIRE_PTR(out);
  OPTIONAL_PTR(lse);
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(RESS_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (kept_idx != nullptr) {
    REQUIRE_PTR(kept_cnt);
    const int n = ress::n_kblocks(shape);
    if (k_max < 1 || k_max > n)
      return fail(RESS_ERR_INVALID_ARG, "k_max=%d must lie in [1, n_k=%d]", k_max, n);
  }
  hipError_t e = ress::launch_attn(q, k, v, dtype, shape, kept_idx, kept_cnt,
                                   k_max, scale, out, lse,
                                   static_cast<hipStream_t>(stream));
  return hip_status(e, "attention launch");
}

}  // extern "C"
