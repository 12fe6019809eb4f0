"""Exact ties among selection keys on the GPU.

Every selection call breaks ties toward the lower key-block index (reading
R9, the oracle's rule). These cases make most keys exactly equal, including
-0.0 against +0.0, so that the radix selects have to break ties on every row.
They run at the three row lengths of the per-wave select: 17 and 34 keys per
lane, and the 256-thread top-k kernel above 2176 key blocks. Keep sets must
equal the oracle's bit for bit: the ties are exact, so no near-tie allowance
is needed.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import check_lists_wellformed, kept_mask_from_lists

pytestmark = pytest.mark.gpu

H = 2


def _lib():
    import block_sparse_global_amd as b
    return b


def _setup(n: int):
    """Square grid of n blocks of 128 tokens (ragged last block), blocks 3
    and n - 1 always kept, budgets of about a seventh and a third of n."""
    b = _lib()
    shape = b.Shape(H=H, N=n * 128 - 37, N_pad=n * 128, D=64, B=128)
    always = np.zeros(n, np.uint8)
    always[[3, n - 1]] = 1
    keep = np.array([2 + max(1, n // 7), 2 + max(1, n // 3)], np.int32)
    return b, shape, keep, always


def _outputs(shape, k_max):
    idx = torch.full((H, shape.nq, k_max), 7, dtype=torch.int32, device="cuda")
    cnt = torch.full((H, shape.nq), -5, dtype=torch.int32, device="cuda")
    return idx, cnt


def _tie_keys(n: int, seed: int, values) -> np.ndarray:
    rng = np.random.default_rng(seed)
    key = np.asarray(values, np.float64)[rng.integers(0, len(values), size=(H, n, n))]
    key[:, ::5, :] = values[-1]  # every fifth row: one value throughout
    return key


@pytest.mark.parametrize("n", [86, 1100, 2300])
def test_topk_exact_ties_take_the_lower_index(n):
    b, shape, keep, always = _setup(n)
    key = _tie_keys(n, 100 + n, [-0.0, 0.0, 0.25, 0.5])
    k_max = int(keep.max())
    idx, cnt = _outputs(shape, k_max)
    print(f"\n[ties topk] n={n} keep={keep.tolist()}", flush=True)
    b.ress_select_topk(torch.from_numpy(key).cuda(), shape, keep, always, k_max, idx, cnt)
    torch.cuda.synchronize()
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    check_lists_wellformed(gi, gc, keep, always, n)
    kept, _ = oracle.select_topk(key, keep, always)
    assert np.array_equal(kept_mask_from_lists(gi, gc, n), kept)


@pytest.mark.parametrize("n", [86, 1100])
def test_cdf_exact_ties_take_the_lower_index(n):
    b, shape, keep, always = _setup(n)
    raw = _tie_keys(n, 200 + n, [0.25, 0.5, 0.75, 1.0])
    P = raw / raw.sum(axis=-1, keepdims=True)  # equal values stay exactly equal
    k_max = int(keep.max())
    idx, cnt = _outputs(shape, k_max)
    tau = 0.3
    print(f"\n[ties cdf] n={n} tau={tau}", flush=True)
    b.ress_select_cdf(torch.from_numpy(P).cuda(), shape, keep, always, tau, k_max, idx, cnt)
    torch.cuda.synchronize()
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    kept, taken, _ = oracle.select_cdf(P, keep, always, tau)
    assert np.array_equal(gc, taken + int(always.sum()))
    for h in range(H):
        for i in range(shape.nq):
            lst = gi[h, i, : gc[h, i]]
            assert np.all(np.diff(lst) > 0) and np.all(gi[h, i, gc[h, i]:] == -1)
    assert np.array_equal(kept_mask_from_lists(gi, gc, n), kept)


@pytest.mark.parametrize("n", [86, 1100])
@pytest.mark.parametrize("mode", ["prob", "drift"])
def test_fused_selection_uniform_map_takes_the_lowest_indices(n, mode):
    """Zero pooled queries give a uniform block map, and identical pooled
    values give equal drift keys: every candidate ties, so each row keeps the
    always-kept blocks and the c_h candidates of lowest index."""
    b, shape, keep, always = _setup(n)
    rng = np.random.default_rng(300 + n)
    qpool = torch.zeros((H, shape.nq, 64), dtype=torch.float64, device="cuda")
    kpool = torch.from_numpy(rng.standard_normal((H, n, 64))).cuda()
    vrow = rng.standard_normal((H, 1, 64))
    vpool = torch.from_numpy(np.repeat(vrow, n, axis=1)).cuda()
    vmv = torch.empty((H, n), dtype=torch.float64, device="cuda")
    k_max = int(keep.max())
    idx, cnt = _outputs(shape, k_max)
    md = b.RESS_SCORE_PROB if mode == "prob" else b.RESS_SCORE_DRIFT
    print(f"\n[ties fused] n={n} mode={mode}", flush=True)
    b.ress_select_fused(qpool, kpool, vpool, None, shape, md, 0.125, 1e-4, keep, always,
                        k_max, vmv, idx, cnt)
    torch.cuda.synchronize()
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    check_lists_wellformed(gi, gc, keep, always, n)
    cand = np.nonzero(always == 0)[0]
    for h in range(H):
        want = np.sort(np.concatenate([cand[: keep[h] - int(always.sum())],
                                       np.nonzero(always)[0]]))
        assert np.all(gi[h, :, : keep[h]] == want[None, :]), f"head {h}"
