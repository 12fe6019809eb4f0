"""The synthetic workloads of block-sparse global attention.

Each workload is one global-attention call of a VGGT-style multi-view
transformer: the tokens of all views are concatenated into one bidirectional
sequence ("ReSS: Residual-Restoring Sparse Attention for 3D Vision
Transformers", §1 and §3 "Block-Sparse Attention for 3D ViTs"). A view of the
large workloads carries 1369 patch tokens, 1 camera token and 4 register
tokens; camera and register tokens are the special tokens whose blocks are
never dropped (same page, §3 and §4.1).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    views: int
    patches_per_view: int
    specials_per_view: int
    heads: int
    head_dim: int
    block: int
    dtype: str  # "f32" or "bf16": the element type of Q, K, V
    # Target sparsity per head: a single value for every head, or the two
    # endpoints of a linear schedule over heads 0..H-1.
    sparsity: Tuple[float, float]
    score: str  # "prob", "drift" or "both" (both scorings timed)
    rounds: int  # drop-set refinement rounds (0 = none)
    rho: float  # total swap fraction of the keep budget
    generator: str  # "shared_vector" or "low_rank"
    # Key block size (0: the same as `block`, square blocks). ReSS Appendix F
    # uses query blocks of 128 and key blocks of 64.
    key_block: int = 0
    seed: int = 0
    notes: str = field(default="", compare=False)

    @property
    def tokens_per_view(self) -> int:
        return self.patches_per_view + self.specials_per_view

    @property
    def N(self) -> int:
        """Number of valid tokens in the concatenated sequence."""
        return self.views * self.tokens_per_view

    @property
    def N_pad(self) -> int:
        """Sequence length rounded up to a whole number of blocks."""
        return -(-self.N // self.block) * self.block

    @property
    def n_blocks(self) -> int:
        """Query blocks (rows of the block maps)."""
        return self.N_pad // self.block

    @property
    def kblock(self) -> int:
        return self.key_block if self.key_block else self.block

    @property
    def n_kblocks(self) -> int:
        """Key blocks (columns of the block maps); the last one may be partial."""
        return -(-self.N // self.kblock)

    def head_sparsity(self, h: int) -> float:
        s0, s1 = self.sparsity
        if self.heads == 1 or s0 == s1:
            return s0
        return s0 + (s1 - s0) * h / (self.heads - 1)

    def dense_flop(self) -> float:
        """4*D*N_pad^2*H: QK^T and PV over every block pair."""
        return 4.0 * self.head_dim * self.N_pad * self.N_pad * self.heads

    def shape_args(self):
        """(H, N, N_pad, D, B, Bk) of the library's shape."""
        return (self.heads, self.N, self.N_pad, self.head_dim, self.block, self.key_block)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload(
            name="tiny",
            views=2, patches_per_view=128, specials_per_view=0,
            heads=2, head_dim=64, block=64, dtype="f32",
            sparsity=(0.5, 0.5), score="prob", rounds=0, rho=0.5,
            generator="shared_vector",
            notes="2 views x 128 tokens, fp32, 4x4 block map",
        ),
        Workload(
            name="views8",
            views=8, patches_per_view=1369, specials_per_view=5,
            heads=16, head_dim=64, block=128, dtype="bf16",
            sparsity=(0.5, 0.5), score="prob", rounds=0, rho=0.5,
            generator="low_rank",
            notes="VGGT-L global layer, 8 views",
        ),
        Workload(
            name="views32",
            views=32, patches_per_view=1369, specials_per_view=5,
            heads=16, head_dim=64, block=128, dtype="bf16",
            sparsity=(0.75, 0.75), score="drift", rounds=0, rho=0.5,
            generator="low_rank",
            notes="32 views, drift score, special-token blocks kept",
        ),
        Workload(
            name="views100",
            views=100, patches_per_view=1369, specials_per_view=5,
            heads=16, head_dim=64, block=128, dtype="bf16",
            sparsity=(0.9, 0.9), score="drift", rounds=3, rho=0.5,
            generator="low_rank",
            notes="100 views, drift score + 3 refinement rounds",
        ),
        Workload(
            name="views8-k64",
            views=8, patches_per_view=1369, specials_per_view=5,
            heads=16, head_dim=64, block=128, dtype="bf16",
            sparsity=(0.5, 0.5), score="drift", rounds=2, rho=0.5,
            generator="low_rank", key_block=64,
            notes="8 views on ReSS Appendix F's grid: query blocks 128, key blocks 64",
        ),
        Workload(
            name="views100-k64",
            views=100, patches_per_view=1369, specials_per_view=5,
            heads=16, head_dim=64, block=128, dtype="bf16",
            sparsity=(0.9, 0.9), score="drift", rounds=3, rho=0.5,
            generator="low_rank", key_block=64,
            notes="100 views, drift + 3 rounds, query blocks 128, key blocks 64",
        ),
        Workload(
            name="views200",
            views=200, patches_per_view=1369, specials_per_view=5,
            heads=16, head_dim=64, block=128, dtype="bf16",
            sparsity=(0.70, 0.95), score="both", rounds=0, rho=0.5,
            generator="low_rank",
            notes="200 views, per-head sparsity 70%..95% linear in h",
        ),
    ]
}

# The workloads in the order small -> large.
ORDER = ["tiny", "views8", "views32", "views100", "views200", "views8-k64", "views100-k64"]


def get_workload(name: str) -> Workload:
    try:
        return WORKLOADS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {ORDER}") from None


def custom(name: str = "custom", **kw) -> Workload:
    """A workload with explicit fields (for edge-case tests)."""
    base = dict(
        views=1, patches_per_view=128, specials_per_view=0, heads=1,
        head_dim=64, block=64, dtype="bf16", sparsity=(0.5, 0.5),
        score="prob", rounds=0, rho=0.5, generator="low_rank", seed=0,
    )
    base.update(kw)
    return Workload(name=name, **base)


def _check():
    for w in WORKLOADS.values():
        assert w.N_pad % w.block == 0
        assert 0 <= w.N_pad - w.N < w.block
        assert w.kblock <= w.block and w.block % w.kblock == 0
        assert math.isfinite(w.dense_flop())


_check()
