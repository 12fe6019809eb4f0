"""CPU oracle for block-sparse global attention (test infrastructure).

A plain, slow, float64 numpy restatement of what the method computes, used
only to check the GPU library. Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import it; the product path never does.
It shares no code with the GPU library: both sides receive the same inputs
from ``synth`` and nothing else.
"""

from .ress_oracle import (  # noqa: F401
    block_pool,
    block_map,
    pooled_output,
    drift_key,
    gram_from_wo,
    select_topk,
    select_cdf,
    kept_lists,
    head_budgets,
    swap_schedule,
    drop_objective,
    swap_gains,
    refine_dropset,
    masked_attention,
    dense_attention,
    residual_drift,
    qkv_project,
    out_project,
    run_selection,
)
