"""libress: block-sparse global attention for MI355X (gfx950).

Python side of the C-ABI library built from ``csrc/``: the entry points
under their C names, plus ``BlockSparseGlobalAttention`` which sequences them
for one workload shape. Importing this package loads ``libress.so`` and
raises if it has not been built (``python block_sparse_global_amd/build.py``
or ``python __graft_entry__.py build``).
"""

from ._lib import (  # noqa: F401
    ENTRY_POINTS,
    LIB_PATH,
    RESS_DTYPE_BF16,
    RESS_DTYPE_F32,
    RESS_ERR_HIP,
    RESS_ERR_INVALID_ARG,
    RESS_ERR_UNSUPPORTED,
    RESS_MAX_BLOCKS,
    RESS_OK,
    RESS_SCORE_DRIFT,
    RESS_SCORE_PROB,
    LIB,
    RessError,
    Shape,
    ress_block_pool,
    ress_block_score,
    ress_gram_from_wo,
    ress_head_budgets,
    ress_last_error,
    ress_refine_dropset,
    ress_refine_dropset_fused,
    ress_refine_dropset_noalloc,
    REFINE_FUSED_MAX_BLOCKS,
    RESS_NOALLOC_SCRATCH_BYTES,
    ress_refine_workspace_size,
    ress_residual_drift,
    ress_qkv_project,
    ress_out_project,
    ress_select_topk,
    ress_select_cdf,
    ress_select_fused,
    SELECT_FUSED_MAX_BLOCKS,
    ress_select_refine_fused,
    SELECT_REFINE_FUSED_MAX_BLOCKS,
    ress_sparse_attn_fwd,
    ress_version,
)
from .layer import BlockSparseGlobalAttention, dense_attention  # noqa: F401
