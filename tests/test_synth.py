"""Synthetic inputs: bf16 rounding, layout, budgets, seed stability."""

import hashlib

import numpy as np
import pytest
import torch

import synth
from synth.workloads import ORDER, custom


def test_bf16_rounding_matches_torch_cpu_cast():
    r = np.random.default_rng(0)
    x = np.concatenate([
        r.standard_normal(500_000).astype(np.float32),
        (r.standard_normal(200_000) * 1e-39).astype(np.float32),       # subnormals
        (r.standard_normal(200_000) * 1e38).astype(np.float32),        # near overflow
        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38], np.float32),
    ])
    # exact ties: values whose low 16 bits are 0x8000
    u = r.integers(0, 2**32, 100_000, dtype=np.uint64).astype(np.uint32)
    u = (u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    ties = u.view(np.float32)
    ties = ties[np.isfinite(ties)]
    x = np.concatenate([x, ties])
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("name,n,always,keep", [
    ("tiny", 4, [], [2, 2]),
    ("views8", 86, [85], [43] * 16),
    ("views32", 344, [342, 343], [86] * 16),
    ("views100", 1074, [1069, 1070, 1071, 1072, 1073], [107] * 16),
])
def test_layout_and_budgets(name, n, always, keep):
    w = synth.get_workload(name)
    assert w.n_blocks == n
    assert list(np.nonzero(synth.always_keep_blocks(w))[0]) == always
    assert list(synth.keep_budgets(w)) == keep


def test_key_blocks_of_64_under_query_blocks_of_128():
    w = synth.get_workload("views100-k64")
    assert (w.block, w.kblock) == (128, 64)
    assert w.n_blocks == 1074 and w.n_kblocks == 2147      # ceil(137400 / 64)
    assert w.n_kblocks * 64 <= w.N_pad
    assert list(np.nonzero(synth.always_keep_blocks(w))[0]) == list(range(2139, 2147))
    assert list(synth.keep_budgets(w)) == [215] * 16       # floor(0.1 * 2147 + 0.5)
    assert w.shape_args() == (16, 137400, 137472, 64, 128, 64)


def test_views200_per_head_budgets():
    w = synth.get_workload("views200")
    k = synth.keep_budgets(w)
    assert w.n_blocks == 2147 and w.N == 274800 and w.N_pad == 274816
    assert k[0] == 644 and k[-1] == 107
    assert np.all(np.diff(k) < 0)
    assert list(np.nonzero(synth.always_keep_blocks(w))[0]) == list(range(2139, 2147))
    # the stated endpoints give a mean sparsity of 82.5%, not 85%
    assert 1 - k.mean() / w.n_blocks == pytest.approx(0.825, abs=2e-3)


def test_special_tokens_sit_in_the_always_kept_blocks():
    for name in ORDER[1:]:
        w = synth.get_workload(name)
        view, special = synth.token_views(w)
        flags = synth.always_keep_blocks(w)
        blocks_with_special = np.unique(np.nonzero(special)[0] // w.kblock)
        assert list(blocks_with_special) == list(np.nonzero(flags)[0])
        assert special.sum() == 5 * w.views


def test_inputs_shapes_padding_and_seed_stability():
    w = custom("t", views=3, patches_per_view=40, specials_per_view=5, heads=2,
               block=32, sparsity=(0.5, 0.5))
    a = synth.make_inputs(w)
    b = synth.make_inputs(w, threads=1)
    for t in ("q", "k", "v"):
        assert a[t].shape == (2, w.N_pad, 64) and a[t].dtype == np.uint16
        assert np.array_equal(a[t], b[t])
        assert np.all(a[t][:, w.N:] == 0)
        assert np.any(a[t][:, : w.N] != 0)


def test_tiny_inputs_digest():
    # pins the generator version: a change of draws must bump GEN_VERSION
    w = synth.get_workload("tiny")
    x = synth.make_inputs(w)
    h = hashlib.sha256()
    for t in ("q", "k", "v"):
        h.update(x[t].tobytes())
    assert x["q"].dtype == np.float32
    assert synth.GEN_VERSION == 1
    assert h.hexdigest()[:16] == DIGEST_TINY


DIGEST_TINY = "212f3e1bad2de40c"


def test_head_scores_and_hess_budget_line():
    # stand-in head scores: positive, seeded, reproducible
    s = synth.make_head_scores(16)
    assert s.shape == (16,) and np.all(s > 0)
    assert np.array_equal(s, synth.make_head_scores(16))
    # the bench line's budgets keep the workload's total and lie within the
    # cap, ordered like the scores (proportional allocation)
    import bench
    w = synth.get_workload("views100")
    x = bench.hess_inputs("views100")
    base = synth.make_inputs(w)["keep"]
    assert int(x["keep"].sum()) == int(base.sum())
    n_alw = int(x["always"].sum())
    assert np.all(x["keep"] >= n_alw + 1) and np.all(x["keep"] <= w.n_kblocks)
    order = np.argsort(-s, kind="stable")
    assert np.all(np.diff(x["keep"][order]) <= 0)
