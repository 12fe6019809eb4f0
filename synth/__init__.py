"""Seeded synthetic inputs for block-sparse global attention.

This package is the only code shared by the CPU oracle (``oracle/``) and the
GPU path (``block_sparse_global_amd``). It holds workload shapes, the token
layout, the integer keep budgets and the random tensors, and none of the
method's arithmetic: no pooling, no attention map, no scoring, no selection.

Workloads stand in for the multi-view scenes the pages evaluate on (at most
100 views per scene for the ReSS benchmark, "ReSS: Residual-Restoring Sparse
Attention for 3D Vision Transformers", §5.1 "Benchmarks"), which are not
available here; only their shapes are reproduced.
"""

from .workloads import WORKLOADS, Workload, get_workload  # noqa: F401
from .layout import always_keep_blocks, keep_budgets, token_views  # noqa: F401
from .gen import (  # noqa: F401
    GEN_VERSION,
    as_f64,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_inputs,
    make_gram,
    make_head_scores,
    make_sublayer,
    make_wo,
)
