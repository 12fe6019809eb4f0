"""Shared helpers of the parity tests: inputs on both sides, comparisons."""

from __future__ import annotations

import functools
import math

import numpy as np

import synth


def to_torch_tokens(x: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(x)
    return t.to(device).contiguous()


@functools.lru_cache(maxsize=2)
def case_inputs(name: str):
    w = synth.get_workload(name)
    x = synth.make_inputs(w)
    return w, x


def f64(x, w):
    return synth.as_f64(x, w.dtype)


def kept_mask_from_lists(idx: np.ndarray, cnt: np.ndarray, n: int) -> np.ndarray:
    H, nq, _ = idx.shape
    m = np.zeros((H, nq, n), dtype=bool)
    for h in range(H):
        for i in range(nq):
            js = idx[h, i, : cnt[h, i]]
            m[h, i, js] = True
    return m


def check_lists_wellformed(idx: np.ndarray, cnt: np.ndarray, keep, always, n: int):
    """Counts equal the budgets, lists ascending and in range, -1 padded,
    always-kept blocks present."""
    H, nq, kmax = idx.shape
    alw = np.nonzero(np.asarray(always))[0] if always is not None else np.array([], int)
    for h in range(H):
        assert np.all(cnt[h] == keep[h]), f"head {h}: counts {np.unique(cnt[h])} != {keep[h]}"
        rows = idx[h, :, : keep[h]]
        assert np.all(rows >= 0) and np.all(rows < n)
        assert np.all(np.diff(rows, axis=1) > 0), "lists must be strictly ascending"
        assert np.all(idx[h, :, keep[h]:] == -1)
        for j in alw:
            assert np.all(np.any(rows == j, axis=1)), f"always-kept block {j} missing"


def compare_masks(gpu: np.ndarray, ref: np.ndarray, key: np.ndarray, always,
                  keep, rel: float = 1e-6):
    """Keep sets must be equal; where a row differs, every block in the
    symmetric difference must carry an oracle key within `rel` (relative) of
    the oracle's cut value (the c-th largest candidate key) — a near-tie.
    Returns the number of rows that differ (all of them near-ties)."""
    H, nq, n = gpu.shape
    cand = (np.asarray(always) == 0) if always is not None else np.ones(n, bool)
    n_alw = n - int(cand.sum())
    differ = np.nonzero(np.any(gpu != ref, axis=-1))
    for h, i in zip(*differ):
        c = int(keep[h]) - n_alw
        kv = key[h, i, cand]
        cut = np.sort(kv)[::-1][c - 1]
        sym = np.nonzero(gpu[h, i] != ref[h, i])[0]
        for j in sym:
            assert cand[j], f"row ({h},{i}): always-kept block {j} differs"
            gap = abs(key[h, i, j] - cut) / max(abs(cut), 1e-300)
            assert gap <= rel, (f"row ({h},{i}) block {j}: key {key[h, i, j]!r} vs cut "
                                f"{cut!r} (rel gap {gap:.3e}) is not a near-tie")
    return len(differ[0])


def attn_errors(gpu: np.ndarray, ref: np.ndarray):
    d = np.abs(gpu.astype(np.float64) - ref)
    return float(d.max()), float(d.mean()), float(np.abs(ref).max())


def sample_blocks(H: int, n: int, count: int, seed: int = 0, must=()):
    """Distinct (h, i) query blocks: the listed ones, the last block of each
    head (holds the padding), then random ones."""
    rng = np.random.default_rng(seed)
    picks = set(tuple(m) for m in must)
    for h in range(H):
        picks.add((h, n - 1))
    while len(picks) < min(count, H * n):
        picks.add((int(rng.integers(H)), int(rng.integers(n))))
    return sorted(picks)


def row_rms(x: np.ndarray) -> float:
    return float(math.sqrt(np.mean(np.square(x))))


def worker_count() -> int:
    """Threads for the oracle comparisons: the CPUs this process may use,
    at most 16."""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def parallel_map(fn, items, threads=None):
    """fn over items on a thread pool, each BLAS call single-threaded (numpy
    releases the GIL inside BLAS and large ufunc loops)."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    items = list(items)
    with threadpool_limits(1), ThreadPoolExecutor(threads or worker_count()) as ex:
        return list(ex.map(fn, items))


def attention_parity(qf, kf, vf, kept, out, lse, N, B, Bk, scale, heads, chunk=64):
    """Every valid query row of every query block of `heads`: the oracle's
    masked attention (float64, one head at a time) against the GPU output and
    log-sum-exp. Returns max-abs, mean-abs, rel-rms of O, the max-abs LSE
    error and the number of query blocks compared; padded rows of `out` must
    be zero."""
    import oracle
    n = qf.shape[1] // B
    tasks = [(h, list(range(i0, min(n, i0 + chunk)))) for h in heads
             for i0 in range(0, n, chunk)]

    def one(task):
        h, rows = task
        sl = slice(h, h + 1)
        O, L = oracle.masked_attention(qf[sl], kf[sl], vf[sl], kept[sl], N, B, scale,
                                       blocks=[(0, i) for i in rows], Bk=Bk)
        t0, t1 = rows[0] * B, min((rows[-1] + 1) * B, N)
        if t1 <= t0:
            return 0.0, 0.0, 0.0, 0.0, 0, 0.0, True
        d = np.abs(out[h, t0:t1].astype(np.float64) - O[0, t0:t1])
        dl = np.abs(lse[h, t0:t1].astype(np.float64) - L[0, t0:t1]) if lse is not None else \
            np.zeros(1)
        pad_ok = bool(np.all(out[h, t1:(rows[-1] + 1) * B] == 0))
        return (float(d.max()), float(d.sum()), float(np.sum(d * d)),
                float(np.sum(O[0, t0:t1] ** 2)), d.size, float(dl.max()), pad_ok)

    res = parallel_map(one, tasks)
    mx = max(r[0] for r in res)
    cnt = sum(r[4] for r in res)
    mean = sum(r[1] for r in res) / cnt
    rel = math.sqrt(sum(r[2] for r in res) / sum(r[3] for r in res))
    lmax = max(r[5] for r in res)
    assert all(r[6] for r in res), "padded rows must be zero"
    return mx, mean, rel, lmax, len(heads) * n
