"""The fused selection (ress_select_fused: pooled blocks to keep lists in one
pass per row tile, the block map and key never written) against the oracle's
top-k on the oracle's own keys (equal up to near-ties below 1e-6 relative)
and against the unfused GPU calls, on every row: 8/32/200 views with either
score, the 128 x 64 grid, the float32 tiny workload, a Gram matrix, and
seeded ragged shapes on both sides of the 1088-block register limit."""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import synth
from synth.workloads import custom
from tests.helpers import (
    check_lists_wellformed,
    compare_masks,
    f64,
    kept_mask_from_lists,
    to_torch_tokens,
)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _run(w, x, mode, impl, M=None):
    import block_sparse_global_amd as b
    shape = b.Shape(*w.shape_args())
    Mt = torch.from_numpy(M).cuda() if M is not None else None
    layer = b.BlockSparseGlobalAttention(shape, x["keep"], x["always"], mode=mode, M=Mt,
                                         select_impl=impl)
    assert layer.select_impl == impl
    q, k, v = (to_torch_tokens(x[t], w.dtype) for t in ("q", "k", "v"))
    layer.pool(q, k, v)
    layer.score()
    layer.select()
    torch.cuda.synchronize()
    return layer.kept_idx.cpu().numpy(), layer.kept_cnt.cpu().numpy()


def _oracle_keys(w, x, mode, M=None):
    qp = oracle.block_pool(f64(x["q"], w), w.N, w.block)
    kp = oracle.block_pool(f64(x["k"], w), w.N, w.kblock)
    P = oracle.block_map(qp, kp, 1.0 / math.sqrt(w.head_dim))
    if mode == "prob":
        return P
    vp = oracle.block_pool(f64(x["v"], w), w.N, w.kblock)
    return oracle.drift_key(P, vp, M, 1e-4)[0]


def _check(w, x, mode, M=None):
    n = w.n_kblocks
    gi, gc = _run(w, x, mode, "fused", M)
    check_lists_wellformed(gi, gc, x["keep"], x["always"], n)
    key = _oracle_keys(w, x, mode, M)
    kept, _ = oracle.select_topk(key, x["keep"], x["always"])
    nd = compare_masks(kept_mask_from_lists(gi, gc, n), kept, key, x["always"], x["keep"])
    ui, uc = _run(w, x, mode, "unfused", M)
    same = np.all(kept_mask_from_lists(gi, gc, n) == kept_mask_from_lists(ui, uc, n), axis=-1)
    print(f"\n[select-fused] {w.name}/{mode}: {nd} near-tie rows vs the oracle, "
          f"{int((~same).sum())} rows differ from the unfused calls, of {gc.size}")
    return nd


@pytest.mark.parametrize("name,mode", [("tiny", "prob"), ("views8", "prob"), ("views8", "drift"),
                                       ("views32", "drift"), ("views8-k64", "drift"),
                                       ("views200", "prob"), ("views200", "drift")])
def test_fused_selection_matches_oracle(name, mode):
    w = synth.get_workload(name)
    _check(w, synth.make_inputs(w), mode)


def test_fused_selection_with_gram_matrix():
    w = custom(name="fg", views=4, patches_per_view=300, specials_per_view=5, heads=3, block=64,
               sparsity=(0.5, 0.8), score="drift")
    _check(w, synth.make_inputs(w), "drift", synth.make_gram(w.heads, w.head_dim, seed=4))


@pytest.mark.parametrize("idx", range(12))
def test_fused_selection_random_shapes(idx):
    rng = np.random.default_rng(500 + idx)
    for _ in range(100):
        block = int(rng.choice([64, 128]))
        # around the 1088-block boundary of the register-resident rows too
        ppv = int(rng.choice([int(rng.integers(20, 700)), 1088 * 64 - 37, 1090 * 64]))
        w = custom(name=f"sf{idx}", views=1 if ppv > 10000 else int(rng.integers(1, 4)),
                   patches_per_view=ppv, specials_per_view=int(rng.choice([0, 5])),
                   heads=int(rng.integers(1, 3)), block=block if ppv < 10000 else 64,
                   key_block=int(rng.choice([0, 64])) if block == 128 and ppv < 10000 else 0,
                   dtype=str(rng.choice(["bf16", "f32"])),
                   sparsity=tuple(sorted(float(s) for s in rng.uniform(0.3, 0.97, 2))),
                   score="drift", seed=int(rng.integers(1 << 30)))
        if w.n_kblocks < 3:
            continue
        try:
            x = synth.make_inputs(w)
        except ValueError:
            continue
        break
    print(f"\n[select-fused random {idx}] N={w.N} B={w.block} Bk={w.kblock} H={w.heads} "
          f"n_k={w.n_kblocks} dtype={w.dtype}", flush=True)
    _check(w, x, str(rng.choice(["prob", "drift"])))
