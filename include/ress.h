/*
 * ress.h — C ABI of libress, block-sparse global attention for MI355X (gfx950).
 *
 * The operation is the three-step block-sparse attention of multi-view
 * geometry transformers as described in "ReSS: Residual-Restoring Sparse
 * Attention for 3D Vision Transformers", §3 "Block-Sparse Attention for 3D
 * ViTs": (1) Q and K are mean pooled per block into a coarse block-level
 * attention map; (2) per (query block, head) key blocks are selected up to a
 * per-head budget, blocks holding special tokens always kept; (3) exact
 * attention runs over the selected blocks only, with the softmax
 * renormalised among them. The subject of those pages, "Block-Sparse Global
 * Attention for Efficient Multi-View Geometry Transformers" (abstract), is
 * the training-free form of this with probability-based selection; the ReSS
 * page adds the drift score (§4.2) and drop-set refinement (§4.3).
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Blocks: queries are grouped in blocks of B tokens, keys (and values)
 *    in blocks of Bk tokens (Bk = 0 means Bk = B). There are n_q = N_pad / B
 *    query blocks and n_k = ceil(N / Bk) key blocks; the last block of
 *    either kind may be partial. Square blocks (Bk = B) are the common case;
 *    ReSS Appendix F uses query blocks of 128 and key blocks of 64.
 *  - Tensor layout: head-major, row-major, contiguous. Token tensors are
 *    [H][N_pad][D]; pooled query blocks [H][n_q][D], pooled key and value
 *    blocks [H][n_k][D]; block maps [H][n_q][n_k] (row i: query block i,
 *    column j: key block j). Tokens t >= N are padding (ignored as keys,
 *    written as zero rows of the attention output).
 *  - D must be 64; B must be 64 or 128; Bk must be 0, 64 or 128 and at most
 *    B; n_q and n_k must be <= 4096.
 *  - Pointers named "device" are caller-owned device memory on the current
 *    HIP device, 16-byte aligned, and must not alias one another. Arrays
 *    named "host" are read on the host during the call and not retained.
 *  - stream: a hipStream_t (NULL = the null stream). Every call only
 *    enqueues work on it and returns; outputs are valid once the stream has
 *    been synchronised. The library never synchronises and allocates no
 *    memory; it keeps no state between calls except a cached record of the
 *    device properties.
 *  - Errors: every argument is validated on the host before any HIP call.
 *    On error nothing is launched, a negative status is returned and a
 *    message is available from ress_last_error() (thread-local). No C++
 *    exception crosses this interface. NaN or Inf inputs give unspecified
 *    (but memory-safe) outputs.
 */
#ifndef RESS_H
#define RESS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RESS_VERSION 5

/* Status codes. */
#define RESS_OK 0
#define RESS_ERR_INVALID_ARG -1 /* a bad pointer, size, budget or enum   */
#define RESS_ERR_UNSUPPORTED -2 /* valid but outside what is implemented */
#define RESS_ERR_HIP -3         /* a HIP runtime or launch error         */

/* Element types of Q, K, V (and of the attention output). */
#define RESS_DTYPE_BF16 0
#define RESS_DTYPE_F32 1

/* Block scores. */
#define RESS_SCORE_PROB 0  /* pooled attention probability             */
#define RESS_SCORE_DRIFT 1 /* ReSS drift key, Eq. 7 of the ReSS page   */

/* Largest supported number of query blocks or key blocks (n_q, n_k). */
#define RESS_MAX_BLOCKS 4096
/* Largest number of heads accepted by the selection calls, whose per-head
 * budgets travel in the kernel arguments. */
#define RESS_MAX_SEL_HEADS 64

typedef struct ress_shape {
  int32_t H;     /* heads                                     */
  int32_t N;     /* valid tokens, 1 <= N <= N_pad             */
  int32_t N_pad; /* padded length, a multiple of B, N_pad-N<B */
  int32_t D;     /* head dimension, must be 64                */
  int32_t B;     /* query block size, 64 or 128               */
  int32_t Bk;    /* key block size: 0 (= B), or 64 / 128 <= B */
} ress_shape;

/*
 * ress_block_pool — mean pooling per block ("ReSS" page, §3 step (1)).
 *
 *   xpool[h][b][:] = mean of x[h][t][:] over the valid tokens t < N of block b
 *
 * with blocks of B tokens for q and of Bk tokens for k and v. q, k, v:
 * device [H][N_pad][D] of `dtype`. Each of the three (input, output) pairs
 * is either both non-NULL or both NULL; at least one pair is given. qpool:
 * device float64 [H][n_q][D]; kpool, vpool: [H][n_k][D]. Accumulation is in
 * float64.
 */
int ress_block_pool(const void* q, const void* k, const void* v, int dtype,
                    ress_shape shape, double* qpool, double* kpool,
                    double* vpool, void* stream);

/*
 * ress_block_score — pooled block map and per-block ranking key.
 *
 *   P[h][i][j] = softmax over all j of scale * qpool[h][i] . kpool[h][j]
 *     ("ReSS" page §4.1: the map is normalised over all key blocks).
 *
 * mode RESS_SCORE_PROB: the ranking key is P itself (SparseVGGT/HeSS as
 *   described on the ReSS page, §3). `key` may be NULL (then rank by P);
 *   vpool, M, vout and vmv are ignored.
 * mode RESS_SCORE_DRIFT (ReSS page §4.2, Eq. 1 and 5-9):
 *   vout[h][i]  = sum_j P[h][i][j] vpool[h][j]                      (Eq. 1)
 *   vmv[h][j]   = vpool[h][j]^T M_h vpool[h][j]  (Eq. 9's last term)
 *   q_ij        = vout_i^T M vout_i - 2 vout_i^T M V_j + vmv_j      (Eq. 9)
 *   key[h][i][j] = P_ij sqrt(max(q_ij, 0)) / max(1 - P_ij, eps)     (Eq. 6-7)
 *   with M_h = I when M is NULL, else M: device float64 [H][D][D], symmetric
 *   (a Gram matrix W_O^T W_O, Eq. 8). vpool, key, vout, vmv are required.
 *
 * qpool: device float64 [H][n_q][D]; kpool, vpool: [H][n_k][D]. P, key:
 * device float64 [H][n_q][n_k]. vout: device float64 [H][n_q][D]. vmv:
 * device float64 [H][n_k].
 * scale > 0 (1/sqrt(D) is the usual value); eps > 0 (1e-4 on the page).
 */
int ress_block_score(const double* qpool, const double* kpool,
                     const double* vpool, const double* M, ress_shape shape,
                     int mode, double scale, double eps, double* P,
                     double* key, double* vout, double* vmv, void* stream);

/*
 * ress_select_topk — per (head, query-block row) keep set (ReSS page §3 step
 * (2), §4.1 Eq. 2 with |S| = c_h, §4.4 "Sparsity control").
 *
 * Candidates are the key blocks j with always_keep[j] == 0. Per row of head
 * h, the c_h = keep[h] - |always| candidates with the largest key are kept
 * (equal keys: the lower block index wins), together with every always-kept
 * block. kept_idx[h][i][0 .. keep[h]-1] receives the kept block indices in
 * ascending order and the rest of the row (up to k_max) is set to -1;
 * kept_cnt[h][i] = keep[h].
 *
 * key: device float64 [H][n_q][n_k]. keep: HOST int32 [H], each
 * 2 <= keep[h] <= n_k and keep[h] > |always|. always_keep: HOST uint8 [n_k]
 * (one flag per key block) or NULL (no always-kept blocks).
 * max_h keep[h] <= k_max <= n_k. kept_idx: device int32 [H][n_q][k_max].
 * kept_cnt: device int32 [H][n_q]. H <= 64.
 */
int ress_select_topk(const double* key, ress_shape shape, const int32_t* keep,
                     const uint8_t* always_keep, int32_t k_max,
                     int32_t* kept_idx, int32_t* kept_cnt, void* stream);

/*
 * ress_select_fused — ress_block_score followed by ress_select_topk as one
 * pass per tile of query-block rows, the block map and the key of a row
 * never leaving the chip (the fused, one-sweep-per-row selection of the ReSS
 * page's Appendix E; §3 steps (1)-(2), §4.1-§4.2 Eq. 1-9). The same keep
 * sets as the two calls (equal up to ties whose keys differ by float64
 * rounding: the sums are taken in another fixed order).
 *
 * qpool, kpool, vpool, M, mode, scale, eps: as for ress_block_score (vpool
 * and vmv required in drift mode, ignored in probability mode). keep,
 * always_keep, k_max, kept_idx, kept_cnt: as for ress_select_topk. vmv:
 * device float64 [H][n_k], written first with V_j^T M_h V_j (Eq. 9's last
 * term, a vector per head; the only other buffer the call writes). Rows of
 * at most 2176 key blocks (RESS_ERR_UNSUPPORTED beyond: use the two calls).
 * Each workgroup keeps up to 156 KB of LDS.
 */
int ress_select_fused(const double* qpool, const double* kpool, const double* vpool,
                      const double* M, ress_shape shape, int mode, double scale, double eps,
                      const int32_t* keep, const uint8_t* always_keep, int32_t k_max,
                      double* vmv, int32_t* kept_idx, int32_t* kept_cnt, void* stream);

/*
 * ress_select_refine_fused — the whole selection with refinement in one
 * pass per tile of query-block rows: ress_block_score in drift mode,
 * ress_select_topk and ress_refine_dropset, with the block map P and the
 * drift key never leaving the chip (the fused selection of the ReSS page's
 * Appendix E, whose kernel sweeps each row once and writes only the new
 * drop set; §4.1-§4.3, Eq. 1-17). A workgroup takes 8 consecutive rows of
 * one head: their map rows stay in LDS next to the refinement's gains,
 * and the drift key of each (row, block), which the top-k and every
 * round's gains need, is re-formed from the product w_r . V_j (Eq. 9
 * expansion) in the same matrix-core instructions as the gains. The keep
 * sets match the three calls up to ties whose keys or gains differ by
 * float64 rounding (vout is summed in another fixed order, as in
 * ress_select_fused); J_init and J_final agree to float64 rounding.
 *
 * qpool, kpool, vpool, M, scale, eps: as for ress_block_score in drift mode
 * (vpool required). keep, always_keep, rounds, rho, k_max: as for
 * ress_refine_dropset. vmv: device float64 [H][n_k], written first with
 * V_j^T M_h V_j (as ress_select_fused). kept_idx [H][n_q][k_max], kept_cnt
 * [H][n_q]: the refined keep lists (ascending, -1 padded). J_init, J_final
 * (optional, float64 [H][n_q]): J of the top-k set and of the best set.
 * Rows of at most 1088 key blocks (RESS_ERR_UNSUPPORTED beyond: use the
 * separate calls). Each workgroup keeps about 156 KB of LDS. No workspace.
 */
int ress_select_refine_fused(const double* qpool, const double* kpool, const double* vpool,
                             const double* M, ress_shape shape, double scale, double eps,
                             const int32_t* keep, const uint8_t* always_keep, int32_t rounds,
                             double rho, int32_t k_max, double* vmv, int32_t* kept_idx,
                             int32_t* kept_cnt, double* J_init, double* J_final, void* stream);

/*
 * ress_select_cdf — per (head, query-block row) keep set under a cumulative
 * probability (top-p, "CDF") threshold, with the per-head budget as a cap:
 * the probability selection the ReSS page compares against (related work on
 * SparseVGGT's top-k and top-p selection; §4.4 and Table 2 "+ CDF
 * threshold"; Appendix F: special blocks always kept, at least two key
 * blocks per query row).
 *
 * Per row of head h: s starts as the sum of P over the always-kept blocks
 * (ascending block order); candidates (always_keep[j] == 0) are then taken
 * by P descending (equal P: the lower block index first), each adding its P
 * to s, one float64 addition at a time in that order, while s < tau and
 * fewer than c_h = keep[h] - |always| are taken; the count is finally raised
 * so that the row keeps at least two blocks. The kept blocks (the taken
 * candidates and every always-kept block) go to kept_idx[h][i] in ascending
 * order, the rest of the row (up to k_max) is set to -1, and kept_cnt[h][i]
 * receives the row's count, which varies with the data (at most keep[h]).
 * tau >= 1 (or above the row's total mass) keeps c_h candidates, the top-k
 * rule on P.
 *
 * P: device float64 [H][n_q][n_k] (ress_block_score's map). tau: finite,
 * > 0.
 * keep, always_keep, k_max, kept_idx, kept_cnt: as for ress_select_topk.
 * Uses cap * 20 bytes of LDS per workgroup, cap = max_h c_h.
 */
int ress_select_cdf(const double* P, ress_shape shape, const int32_t* keep,
                    const uint8_t* always_keep, double tau, int32_t k_max,
                    int32_t* kept_idx, int32_t* kept_cnt, void* stream);

/*
 * ress_refine_dropset — ReSS iterative residual restoration (ReSS page
 * §4.3, Eq. 10-17, Appendix E), applied to the keep sets from
 * ress_select_topk.
 *
 * Per row, with D = candidates not kept, d_j = P_j (vout - V_j) (Eq. 5):
 * g = sum_{j in D} d_j, K = 1 - sum_{j in D} P_j, G = g^T M g, J = G / K^2
 * (Eq. 10, 12). Round r (r < rounds) swaps m_r = floor(rho c / 2^(r+1))
 * blocks (Eq. 17), clamped to |D| and to the kept candidates: from the
 * round-start g, K, G it computes the exact objective decrease (Eq. 16) of
 * restoring each k in D (Eq. 13-14) and of dropping each kept candidate
 * (Eq. 15; a drop with K + u <= 0 counts as -inf), with s_k^2 = (key_k *
 * max(1 - P_k, eps))^2 (Eq. 6-7); restores the m_r best restores and drops
 * the m_r best drops (ties: lower index); then moves g and K by the swapped
 * blocks (Eq. 13) and recomputes G and J. The set with the smallest J seen
 * (strictly smaller replaces) is written back to kept_idx / kept_cnt in the
 * same format as the top-k call.
 *
 * P, key: device float64 [H][n_q][n_k] (key = the drift key of
 * ress_block_score with the same eps and M). vpool: device float64
 * [H][n_k][D] and vout: [H][n_q][D], as written by ress_block_score in drift
 * mode. M: device float64 [H][D][D] or NULL
 * (= I). keep, always_keep: HOST, as for ress_select_topk. rounds >= 0,
 * 0 < rho <= 1, eps > 0. kept_idx, kept_cnt: device, in/out. J_init,
 * J_final: device float64 [H][n_q] or NULL. H <= 64. workspace: device,
 * workspace_bytes >= ress_refine_workspace_size(shape), 256-byte aligned;
 * calls that share one workspace must not overlap. The rounds run as
 * kernels on `stream` (an init kernel, then a gains and a selection kernel
 * per round with swaps, then a final kernel).
 */
int ress_refine_dropset(const double* P, const double* key,
                        const double* vpool, const double* vout,
                        const double* M, ress_shape shape, const int32_t* keep,
                        const uint8_t* always_keep, int32_t rounds, double rho,
                        double eps, int32_t k_max, int32_t* kept_idx,
                        int32_t* kept_cnt, double* J_init, double* J_final,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * ress_refine_dropset_fused — the same refinement as ress_refine_dropset
 * (same arguments apart from the workspace, same results bit for bit),
 * with the whole of it in one kernel: a workgroup takes 16 consecutive
 * query-block rows of one head through the starting state, every round and
 * the final keep lists, holding the gains, the current and best drop sets
 * and the row state on chip (the fused restoration kernel of ReSS Appendix
 * E). Only the keep lists and J_init / J_final are written to device memory;
 * no workspace. Returns RESS_ERR_UNSUPPORTED when n_k > 1088 (a row's gains
 * must fit in the workgroup's LDS); ress_refine_dropset covers those shapes.
 * On the MI355X the per-round call is the faster of the two (one such
 * workgroup fills a CU's LDS, which leaves its latency-bound per-row steps
 * nothing to overlap with); this one needs no workspace.
 */
int ress_refine_dropset_fused(const double* P, const double* key, const double* vpool,
                              const double* vout, const double* M, ress_shape shape,
                              const int32_t* keep, const uint8_t* always_keep, int32_t rounds,
                              double rho, double eps, int32_t k_max, int32_t* kept_idx,
                              int32_t* kept_cnt, double* J_init, double* J_final,
                              void* stream);

/* Bytes of the fixed device scratch of ress_refine_dropset_noalloc (64 MiB;
 * each GPU that loads the library holds one such array). */
#define RESS_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * ress_refine_dropset_noalloc — ress_refine_dropset (same arguments apart
 * from the workspace, same results bit for bit) for callers that cannot
 * allocate device memory: code under graph capture, tight serving loops,
 * harnesses that forbid allocation. Its refinement state lives in a fixed
 * array of RESS_NOALLOC_SCRATCH_BYTES bytes inside the library, one per GPU;
 * the call allocates nothing and calls no allocating routine. The heads are
 * refined in groups of as many heads as the scratch holds (the state of g
 * heads takes ress_refine_workspace_size of the shape with H = g), one group
 * after another on `stream`. RESS_ERR_UNSUPPORTED when a single head's state
 * exceeds the scratch (about 10 n_q n_k + 1100 n_q bytes: square grids up to
 * n = 2535 blocks fit; the 128 x 64 grid at 100 views takes 23 MB a head).
 * Every call on one GPU uses that GPU's one array, which keeps the last
 * call's contents (nothing in it needs to start at zero): calls that overlap
 * on one GPU (other streams, other threads) race and give undefined results.
 */
int ress_refine_dropset_noalloc(const double* P, const double* key, const double* vpool,
                                const double* vout, const double* M, ress_shape shape,
                                const int32_t* keep, const uint8_t* always_keep, int32_t rounds,
                                double rho, double eps, int32_t k_max, int32_t* kept_idx,
                                int32_t* kept_cnt, double* J_init, double* J_final,
                                void* stream);

/*
 * ress_refine_workspace_size — bytes of device workspace that
 * ress_refine_dropset needs for `shape`: the refinement state of every
 * (head, query-block) row, about 10 n_q n_k H + 1100 n_q H bytes (the gains, the
 * current and best drop sets, g and M g per row). 0 for an invalid shape
 * (ress_last_error says why). The caller allocates it (256-byte aligned, as
 * hipMalloc returns) and may reuse it across calls on one stream; its
 * contents need no initialisation and are garbage after a call.
 */
size_t ress_refine_workspace_size(ress_shape shape);

/*
 * ress_head_budgets — per-head keep budgets from head importance scores, the
 * allocation ReSS adopts from HeSS (ReSS page §4.4 and Appendix D:
 * proportional allocation with iterative clipping at the cap). Host only;
 * no device memory is touched.
 *
 * Every head first gets the floor f (at least two kept blocks per row and at
 * least one candidate: f = max(1, 2 - |always|) candidates). The surplus
 * U = total_keep - H (|always| + f) is split in proportion to score[h]
 * (equally when every score is 0); a head whose share exceeds the cap
 * (all n_k - |always| candidates, less f) is fixed at the cap and the rest
 * of U is split again among the others, until no share exceeds the cap.
 * Integer budgets: each share rounded down, then the units still missing go
 * one each to the largest fractional parts (equal parts: the lower head),
 * never beyond the cap. keep[h] = |always| + f + that integer, so
 * sum_h keep[h] = total_keep, ready for ress_select_topk.
 *
 * score: HOST float64 [H], finite, >= 0. H: 1 .. 64. n_k: key blocks per
 * row, 2 .. 4096. always_keep: HOST uint8 [n_k] or NULL. total_keep: in
 * [H (|always| + f), H n_k]. keep: HOST int32 [H], written.
 */
int ress_head_budgets(const double* score, int32_t H, int32_t n_k, const uint8_t* always_keep,
                      int64_t total_keep, int32_t* keep);

/*
 * ress_gram_from_wo — per-head Gram matrices of the output projection
 * (ReSS page §4.2, Eq. 8): M[h] = (W_O^h)^T W_O^h, where W_O^h is the slice
 * of the output projection that maps head h's D outputs into the residual
 * stream, so that e^T M[h] e = ||W_O^h e||^2 (Eq. 6, 9). The result feeds
 * the M argument of ress_block_score and ress_refine_dropset, making the
 * drift score and the refinement objective residual-space exact.
 *
 * w_o: device [d_model][H*D] row-major of `dtype` (the layout of a linear
 * layer's weight from H*D inputs to d_model outputs; W_O^h is columns
 * h*D .. h*D+D-1). d_model: 1 .. 2^20. M: device float64 [H][D][D]; each
 * entry is a fixed-order float64 sum over the d_model rows (products of
 * bf16 or float32 values are exact in float64).
 */
int ress_gram_from_wo(const void* w_o, int dtype, int32_t d_model, ress_shape shape,
                      double* M, void* stream);

/*
 * ress_sparse_attn_fwd — exact attention over the kept key blocks (ReSS page
 * §3 step (3): softmax renormalised among the selected blocks alone, the
 * unselected blocks contributing nothing; dense global attention when kept_idx is
 * NULL).
 *
 *   out[h][t] = sum_u softmax_u(scale q[h][t] . k[h][u]) v[h][u]
 *
 * over the valid keys u < N of the blocks kept_idx[h][i][0 .. kept_cnt-1]
 * of t's query block i. bf16 inputs: QK^T and PV run on bf16 matrix cores
 * with float32 accumulation, the weights rounded to bf16 for PV (the row sum
 * is taken over those same weights); a first pass takes the weights without
 * subtracting a running max and is kept when every row sum lies in
 * [2^-64, 2^64], else the workgroup reruns as a classical online softmax
 * (same accuracy either way). float32 inputs: QK^T and PV on float32 matrix
 * cores with float32 weights (float32 accuracy). Rows t >= N are written as
 * zeros.
 *
 * Query block i holds tokens i*B .. i*B+B-1 and key block j tokens
 * j*Bk .. j*Bk+Bk-1. q, k, v: device [H][N_pad][D] of `dtype`. kept_idx:
 * device int32 [H][n_q][k_max] or NULL (dense: all n_k key blocks); entries
 * outside [0, n_k) are skipped. kept_cnt: device int32 [H][n_q], required
 * with kept_idx (values are clamped
 * to [0, k_max]; a row with nothing kept is written as zeros). out: device
 * [H][N_pad][D] of `dtype`. lse: device float32 [H][N_pad] or NULL; it
 * receives log sum_u exp(scale q . k_u) (natural log; -inf for an empty
 * row, 0 for padded rows). scale > 0.
 */
int ress_sparse_attn_fwd(const void* q, const void* k, const void* v,
                         int dtype, ress_shape shape, const int32_t* kept_idx,
                         const int32_t* kept_cnt, int32_t k_max, float scale,
                         void* out, float* lse, void* stream);

/*
 * ress_residual_drift — the drift a sparse attention output leaves in the
 * residual stream, measured against the dense output (ReSS page §4.2,
 * Eq. 6 and 9 at token level; the quantity the page argues governs the cost
 * of sparsification, §6):
 *
 *   drift[h][i] = mean over the valid tokens t of query block i of
 *                 e^T M[h] e,   e = out_sparse[h][t] - out_dense[h][t],
 *
 * = ||W_O^h e||^2 averaged over the block when M[h] = (W_O^h)^T W_O^h
 * (ress_gram_from_wo); ||e||^2 when M is NULL.
 *
 * out_sparse, out_dense: device [H][N_pad][D] of `dtype` (outputs of
 * ress_sparse_attn_fwd with and without kept_idx). M: device float64
 * [H][D][D], symmetric, or NULL. drift: device float64 [H][n_q].
 */
int ress_residual_drift(const void* out_sparse, const void* out_dense, int dtype,
                        const double* M, ress_shape shape, double* drift, void* stream);

/*
 * ress_qkv_project — the QKV projection in front of the attention call: the
 * per-head queries, keys and values the path consumes, from the token
 * features of the attention sublayer (ReSS page §3, a pre-LN residual
 * sublayer; §4.2 names the per-head Q, K, V). A linear layer y = x W^T + b
 * with W = w_qkv, split by output channel c = which * H*D + h*D + d into
 * q, k, v (which = 0, 1, 2) in the path's layout:
 *
 *   {q,k,v}[h][t][d] = b_qkv[c] + sum_e x[t][e] w_qkv[c][e]   (t < N)
 *
 * bf16 matrix cores with float32 accumulation, each output rounded once to
 * bf16 (nearest even). Rows t >= N of q, k, v are written as zeros.
 *
 * x: device bf16 [N_pad][d_model]. w_qkv: device bf16 [3*H*D][d_model] (a
 * linear layer's weight, [out][in]). b_qkv: device bf16 [3*H*D] or NULL.
 * q, k, v: device bf16 [H][N_pad][D]. dtype: RESS_DTYPE_BF16 only.
 * d_model: a positive multiple of 64, at most 65536.
 */
int ress_qkv_project(const void* x, const void* w_qkv, const void* b_qkv, int dtype,
                     int32_t d_model, ress_shape shape, void* q, void* k, void* v,
                     void* stream);

/*
 * ress_out_project — the output projection with the residual add behind the
 * attention call: every head's output o^h enters the residual stream as
 * W_O^h o^h (ReSS page §4.2 "Mapping to the residual space", Eq. 6 and 8;
 * W_O^h is the slice of W_O that ress_gram_from_wo turns into M_h):
 *
 *   y[t][c] = residual[t][c] + b_o[c] + sum_{h,d} o[h][t][d] w_o[c][h*D + d]
 *
 * bf16 matrix cores with float32 accumulation; the sum, the bias and the
 * residual are added in float32 and rounded once to bf16 (nearest even).
 * Every row t < N_pad is computed (the attention call writes padded rows of
 * o as zeros).
 *
 * o: device bf16 [H][N_pad][D] (ress_sparse_attn_fwd's output). w_o: device
 * bf16 [d_model][H*D] (a linear layer's weight). b_o: device bf16 [d_model]
 * or NULL. residual: device bf16 [N_pad][d_model] or NULL (then no residual
 * is added). y: device bf16 [N_pad][d_model]; y may be the residual buffer
 * itself (an in-place residual add: each element is read and then written by
 * the same thread), but must not alias o or w_o. dtype: RESS_DTYPE_BF16
 * only. d_model: a positive multiple of 64, at most 65536.
 */
int ress_out_project(const void* o, const void* w_o, const void* b_o, const void* residual,
                     int dtype, int32_t d_model, ress_shape shape, void* y, void* stream);

/* Message of the last failed call on this thread ("" if none). */
const char* ress_last_error(void);

/* RESS_VERSION of the built library. */
int ress_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RESS_H */
