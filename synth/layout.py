"""Token layout, always-kept blocks and integer keep budgets.

Layout (a reading: the pages do not fix the order). The patch tokens of all
views come first, view after view; then the special tokens (1 camera + 4
register per view), view after view; then zero padding up to a whole block.
Special tokens therefore sit at the tail, which matches the "sink rule" of
"ReSS: Residual-Restoring Sparse Attention for 3D Vision Transformers",
Appendix F ("Common conditions"): the trailing block that holds the special
tokens is always kept. A key block is always kept when it holds any special
token (same page, §3 and §4.1: blocks containing special tokens are always
kept; the rest form the candidate set P).

Budgets: "keep X% of key blocks per query-block row" is read as a total of
k_h = max(2, floor((1 - s_h) * n + 0.5)) kept key blocks per row, always-kept
blocks included; the floor of two blocks per row is the one stated in
Appendix F of the same page. The candidate budget c_h of §4.1 (Eq. 2) is
k_h minus the number of always-kept blocks. The integers are computed here
once, so both sides of every comparison use the same ones.
"""

from __future__ import annotations

import math

import numpy as np

from .workloads import Workload


def token_views(w: Workload):
    """Per valid token: (view index, is_special) as two int arrays of length N."""
    P = w.patches_per_view
    S = w.specials_per_view
    V = w.views
    view = np.empty(w.N, dtype=np.int64)
    special = np.zeros(w.N, dtype=bool)
    view[: V * P] = np.repeat(np.arange(V), P)
    if S:
        view[V * P:] = np.repeat(np.arange(V), S)
        special[V * P:] = True
    return view, special


def always_keep_blocks(w: Workload) -> np.ndarray:
    """uint8 flags [n_k]: 1 where the key block holds a special token."""
    flags = np.zeros(w.n_kblocks, dtype=np.uint8)
    if w.specials_per_view:
        first = w.views * w.patches_per_view
        last = w.N - 1
        flags[first // w.kblock: last // w.kblock + 1] = 1
    return flags


def keep_budgets(w: Workload) -> np.ndarray:
    """int32 [H]: total kept key blocks per query-block row, per head."""
    n = w.n_kblocks
    k = []
    for h in range(w.heads):
        s = w.head_sparsity(h)
        k.append(max(2, int(math.floor((1.0 - s) * n + 0.5))))
    k = np.asarray(k, dtype=np.int32)
    n_always = int(always_keep_blocks(w).sum())
    if np.any(k <= n_always) or np.any(k > n):
        raise ValueError(f"{w.name}: budgets {k} do not fit n={n}, always={n_always}")
    return k

