"""The whole block-sparse global-attention step over the C ABI.

``BlockSparseGlobalAttention`` owns the device buffers of one workload shape
(allocated once with torch) and runs pool -> score -> top-k (or the cumulative-probability
threshold) -> [refine] -> sparse attention as library calls on one stream. It only allocates and
sequences; every step is a libress kernel.
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch

from ._lib import (
    REFINE_FUSED_MAX_BLOCKS,
    SELECT_FUSED_MAX_BLOCKS,
    RESS_SCORE_DRIFT,
    RESS_SCORE_PROB,
    SELECT_REFINE_FUSED_MAX_BLOCKS,
    Shape,
    ress_block_pool,
    ress_block_score,
    ress_refine_dropset,
    ress_refine_dropset_fused,
    ress_refine_workspace_size,
    ress_select_cdf,
    ress_select_fused,
    ress_select_refine_fused,
    ress_select_topk,
    ress_sparse_attn_fwd,
)


# Rows up to this many key blocks take the fused selection under
# select_impl="auto". Measured on the MI355X (score and top-k together):
# 0.020 against 0.030 ms for the unfused calls at 86 key blocks (8 views),
# 0.110 against 0.081 ms at 344 (32 views); longer rows stream more pooled
# blocks through each row tile than the split kernels read.
SELECT_FUSED_AUTO_MAX_BLOCKS = 128


def select_path(shape: Shape, select_impl: str, rounds: int, tau) -> str:
    """The selection calls used for ``select_impl`` on ``shape``: "fused" is
    one pass per row tile with the block map and key never written:
    ress_select_fused (score and top-k) on rows of at most
    SELECT_FUSED_MAX_BLOCKS key blocks, or, with refinement rounds,
    ress_select_refine_fused (score, top-k and refinement) on rows of at
    most SELECT_REFINE_FUSED_MAX_BLOCKS; otherwise (and for the cumulative
    threshold) ress_block_score + ress_select_topk / _cdf [+ the
    refinement call]. "auto" takes the fused pass for top-k without
    refinement on rows of at most SELECT_FUSED_AUTO_MAX_BLOCKS key blocks,
    where it measured faster, else the unfused calls."""
    if select_impl not in ("fused", "unfused", "auto"):
        raise ValueError(select_impl)
    limit = SELECT_FUSED_MAX_BLOCKS if rounds == 0 else SELECT_REFINE_FUSED_MAX_BLOCKS
    applies = tau is None and shape.nk <= limit
    if select_impl == "auto":
        return ("fused" if applies and rounds == 0 and shape.nk <= SELECT_FUSED_AUTO_MAX_BLOCKS
                else "unfused")
    if select_impl == "fused" and not applies:
        return "unfused"
    return select_impl


def refine_path(shape: Shape, refine_impl: str) -> str:
    """The refinement call used for ``refine_impl`` on ``shape``: "fused" rows
    longer than REFINE_FUSED_MAX_BLOCKS key blocks take the per-round kernels
    (the same results, bit for bit)."""
    if refine_impl not in ("fused", "rounds"):
        raise ValueError(refine_impl)
    if refine_impl == "fused" and shape.nk > REFINE_FUSED_MAX_BLOCKS:
        return "rounds"
    return refine_impl


class BlockSparseGlobalAttention:
    def __init__(self, shape: Shape, keep, always_keep, mode: str = "prob",
                 rounds: int = 0, rho: float = 0.5, eps: float = 1e-4,
                 scale: Optional[float] = None, M: Optional[torch.Tensor] = None,
                 device="cuda", with_lse: bool = False, tau: Optional[float] = None,
                 refine_impl: str = "rounds", select_impl: str = "auto"):
        """``tau`` switches the selection from top-k to the cumulative
        probability threshold (ress_select_cdf, probability scoring only; the
        budget ``keep`` is then the cap). ``refine_impl``: "rounds"
        (ress_refine_dropset, kernels per round and a workspace; the faster
        one on the MI355X) or "fused" (ress_refine_dropset_fused, one kernel,
        no workspace, rows of at most REFINE_FUSED_MAX_BLOCKS key blocks;
        longer rows fall back to the per-round kernels, as the fused
        restoration kernel of ReSS Appendix E falls back to its unfused path
        outside its limits); both give the same bits. ``select_impl``:
        "unfused" (ress_block_score then ress_select_topk), "fused"
        (ress_select_fused, or ress_select_refine_fused with refinement
        rounds, which then also refines: one pass per row tile, the map and
        key never written, within the row limits of select_path, else the
        unfused calls) or "auto" (the fused pass for top-k without
        refinement on rows of at most SELECT_FUSED_AUTO_MAX_BLOCKS key
        blocks, where it measured faster, else the unfused calls); all give
        the same lists up to near-ties."""
        refine_impl = refine_path(shape, refine_impl)
        self.select_impl = select_path(shape, select_impl, int(rounds), tau)
        if mode not in ("prob", "drift"):
            raise ValueError(mode)
        if rounds > 0 and mode != "drift":
            raise ValueError("refinement rounds need the drift-mode score outputs")
        if tau is not None and mode != "prob":
            raise ValueError("the cumulative threshold ranks by probability: mode='prob'")
        self.tau = None if tau is None else float(tau)
        self.shape = shape
        self.keep = np.ascontiguousarray(np.asarray(keep, dtype=np.int32))
        self.always = (None if always_keep is None
                       else np.ascontiguousarray(np.asarray(always_keep, dtype=np.uint8)))
        self.mode = mode
        self.rounds = int(rounds)
        self.rho = float(rho)
        self.eps = float(eps)
        self.scale = float(scale if scale is not None else 1.0 / math.sqrt(shape.D))
        self.M = M
        self.k_max = int(self.keep.max())
        H, nq, nk, D, Np = shape.H, shape.nq, shape.nk, shape.D, shape.N_pad
        f64 = dict(dtype=torch.float64, device=device)
        self.qpool = torch.empty((H, nq, D), **f64)
        self.kpool = torch.empty((H, nk, D), **f64)
        need_v = mode == "drift"
        self.vpool = torch.empty((H, nk, D), **f64) if need_v else None
        fused = self.select_impl == "fused"
        self.P = None if fused else torch.empty((H, nq, nk), **f64)
        self.key = torch.empty((H, nq, nk), **f64) if mode == "drift" and not fused else None
        self.vout = torch.empty((H, nq, D), **f64) if need_v and not fused else None
        self.vmv = torch.empty((H, nk), **f64) if need_v else None
        self.kept_idx = torch.empty((H, nq, self.k_max), dtype=torch.int32, device=device)
        self.kept_cnt = torch.empty((H, nq), dtype=torch.int32, device=device)
        self.J_init = torch.empty((H, nq), **f64) if rounds > 0 else None
        self.J_final = torch.empty((H, nq), **f64) if rounds > 0 else None
        self.refine_impl = refine_impl
        self.workspace = (torch.empty(ress_refine_workspace_size(shape), dtype=torch.uint8,
                                      device=device)
                          if rounds > 0 and refine_impl == "rounds" and not fused else None)
        self.lse = (torch.empty((H, Np), dtype=torch.float32, device=device)
                    if with_lse else None)
        self.out = None

    # -- the steps ------------------------------------------------------------
    def pool(self, q, k, v, stream=None):
        ress_block_pool(q, k, v if self.vpool is not None else None, self.shape,
                        self.qpool, self.kpool, self.vpool, stream)

    def score(self, stream=None):
        if self.select_impl == "fused":
            return  # the fused selection scores on chip
        mode = RESS_SCORE_DRIFT if self.mode == "drift" else RESS_SCORE_PROB
        ress_block_score(self.qpool, self.kpool, self.vpool, self.M, self.shape, mode,
                         self.scale, self.eps, self.P, self.key, self.vout, self.vmv,
                         stream)

    def select(self, stream=None):
        if self.select_impl == "fused" and self.rounds > 0:
            ress_select_refine_fused(self.qpool, self.kpool, self.vpool, self.M, self.shape,
                                     self.scale, self.eps, self.keep, self.always, self.rounds,
                                     self.rho, self.k_max, self.vmv, self.kept_idx,
                                     self.kept_cnt, self.J_init, self.J_final, stream)
            return
        if self.select_impl == "fused":
            mode = RESS_SCORE_DRIFT if self.mode == "drift" else RESS_SCORE_PROB
            ress_select_fused(self.qpool, self.kpool, self.vpool, self.M, self.shape, mode,
                              self.scale, self.eps, self.keep, self.always, self.k_max,
                              self.vmv, self.kept_idx, self.kept_cnt, stream)
            return
        if self.tau is not None:
            ress_select_cdf(self.P, self.shape, self.keep, self.always, self.tau,
                            self.k_max, self.kept_idx, self.kept_cnt, stream)
            return
        key = self.key if self.key is not None else self.P
        ress_select_topk(key, self.shape, self.keep, self.always, self.k_max,
                         self.kept_idx, self.kept_cnt, stream)

    def refine(self, stream=None):
        if self.rounds <= 0 or self.select_impl == "fused":
            return  # the fused pass refines on chip
        if self.refine_impl == "fused":
            ress_refine_dropset_fused(self.P, self.key, self.vpool, self.vout, self.M,
                                      self.shape, self.keep, self.always, self.rounds,
                                      self.rho, self.eps, self.k_max, self.kept_idx,
                                      self.kept_cnt, self.J_init, self.J_final, stream)
            return
        ress_refine_dropset(self.P, self.key, self.vpool, self.vout, self.M, self.shape,
                            self.keep, self.always, self.rounds, self.rho, self.eps,
                            self.k_max, self.kept_idx, self.kept_cnt, self.J_init,
                            self.J_final, self.workspace, stream)

    def attend(self, q, k, v, out, stream=None):
        ress_sparse_attn_fwd(q, k, v, self.shape, self.kept_idx, self.kept_cnt,
                             self.k_max, self.scale, out, self.lse, stream)

    def __call__(self, q, k, v, out=None, stream=None):
        if out is None:
            if self.out is None or self.out.dtype != q.dtype:
                self.out = torch.empty_like(q)
            out = self.out
        self.pool(q, k, v, stream)
        self.score(stream)
        self.select(stream)
        self.refine(stream)
        self.attend(q, k, v, out, stream)
        return out


def dense_attention(q, k, v, shape: Shape, out, scale: Optional[float] = None,
                    lse=None, stream=None):
    """Dense global attention through the same kernel (every block kept)."""
    s = float(scale if scale is not None else 1.0 / math.sqrt(shape.D))
    ress_sparse_attn_fwd(q, k, v, shape, None, None, 1, s, out, lse, stream)
    return out
