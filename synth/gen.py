"""Seeded random Q, K, V for the synthetic workloads.

Generators (readings; the pages print no input distribution):

* ``low_rank`` (the multi-view workloads): for every (head, view) a basis
  W in R^{8 x 64} with entries N(0, 1/8) is shared by the Q and K tokens of
  that view; each token draws its own coefficients a ~ N(0, I_8) (separately
  for Q and K) and Q, K = a W + N(0, 1) noise. V ~ N(0, 1). Special tokens
  are drawn as tokens of their own view.
* ``shared_vector`` (the tiny workload): Q, K ~ N(0, 1) plus one vector
  u ~ 0.5 * N(0, I_64) per (head, view), added to every Q and K token of that
  view. V ~ N(0, 1).

Values are drawn in float32 and, for bf16 workloads, rounded once to bf16
with round-to-nearest-even; both sides then read the same bit patterns.
Padded token rows are zero.

Streams: ``SeedSequence(seed)`` spawns one child per tensor role, and each
child spawns one stream per head, so a head can be drawn on its own.
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

from .layout import always_keep_blocks, keep_budgets, token_views
from .workloads import Workload

GEN_VERSION = 1

_ROLES = ("basis", "q", "k", "v")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); uint16 bits.

    NaN inputs map to a quiet NaN; infinities and overflow to infinity follow
    from the same integer rounding.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _streams(seed: int, heads: int):
    root = np.random.SeedSequence(seed)
    kids = root.spawn(len(_ROLES))
    return {role: kid.spawn(heads) for role, kid in zip(_ROLES, kids)}


def _head_tensors(w: Workload, h: int, streams, view, special):
    """float32 Q, K, V [N_pad][D] of head h."""
    D = w.head_dim
    N = w.N
    V = w.views
    out = []
    rb = np.random.default_rng(streams["basis"][h])
    if w.generator == "low_rank":
        basis = rb.standard_normal((V, 8, D), dtype=np.float32) * np.float32(
            np.sqrt(1.0 / 8.0)
        )
    elif w.generator == "shared_vector":
        shared = rb.standard_normal((V, D), dtype=np.float32) * np.float32(0.5)
    else:
        raise ValueError(w.generator)
    for role in ("q", "k"):
        rg = np.random.default_rng(streams[role][h])
        x = np.zeros((w.N_pad, D), dtype=np.float32)
        noise = rg.standard_normal((N, D), dtype=np.float32)
        if w.generator == "low_rank":
            coef = rg.standard_normal((N, 8), dtype=np.float32)
            for v in range(V):
                sel = view == v
                x[:N][sel] = coef[sel] @ basis[v]
            x[:N] += noise
        else:
            x[:N] = noise + shared[view]
        out.append(x)
    rv = np.random.default_rng(streams["v"][h])
    xv = np.zeros((w.N_pad, D), dtype=np.float32)
    xv[:N] = rv.standard_normal((N, D), dtype=np.float32)
    out.append(xv)
    return out


def make_inputs(w: Workload, threads: int | None = None):
    """All inputs of one workload.

    Returns a dict with
      q, k, v : [H][N_pad][D] uint16 bf16 bit patterns (bf16 workloads) or
                float32 (f32 workloads), C-contiguous;
      always  : uint8 [n] always-kept key-block flags;
      keep    : int32 [H] kept key blocks per row (always-kept included).
    """
    H, D = w.heads, w.head_dim
    view, special = token_views(w)
    streams = _streams(w.seed, H)
    dt = np.uint16 if w.dtype == "bf16" else np.float32
    res = {r: np.empty((H, w.N_pad, D), dtype=dt) for r in ("q", "k", "v")}

    def one(h):
        tq, tk, tv = _head_tensors(w, h, streams, view, special)
        for name, t in zip(("q", "k", "v"), (tq, tk, tv)):
            res[name][h] = f32_to_bf16_bits(t) if w.dtype == "bf16" else t

    nt = threads or min(H, max(1, len(os.sched_getaffinity(0))))
    if nt <= 1 or H == 1:
        for h in range(H):
            one(h)
    else:
        with ThreadPoolExecutor(nt) as ex:
            list(ex.map(one, range(H)))
    res["always"] = always_keep_blocks(w)
    res["keep"] = keep_budgets(w)
    return res


def as_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """The exact values of an input tensor, as float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def make_wo(heads: int, head_dim: int = 64, d_model: int = 1024, seed: int = 2,
            scale: float = 0.03):
    """A random output projection W_O [d_model][heads*head_dim] (the layout of
    a linear layer's weight), entries N(0, scale^2) rounded once to bf16 and
    returned as bf16 bit patterns (uint16). Stands in for a trained
    projection, which does not exist here."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((d_model, heads * head_dim)) * scale).astype(np.float32)
    return f32_to_bf16_bits(w)


def make_sublayer(n_tokens: int, heads: int, head_dim: int = 64, d_model: int = 1024,
                  seed: int = 4):
    """Random token features and linear-layer weights of one attention
    sublayer, all rounded once to bf16 and returned as bf16 bit patterns
    (uint16): x [n_tokens][d_model] ~ N(0, 1); w_qkv [3 H D][d_model] and
    w_o [d_model][H D] with entries N(0, 1/d_model) and N(0, 1/(H D)), so
    that projected values stay of order one; b_qkv [3 H D] and b_o [d_model]
    ~ N(0, 0.1^2). They stand in for a trained layer and its inputs, which do
    not exist here."""
    rng = np.random.default_rng(seed)
    hd = heads * head_dim
    g = lambda shape, sd: f32_to_bf16_bits((rng.standard_normal(shape) * sd).astype(np.float32))
    return {
        "x": g((n_tokens, d_model), 1.0),
        "w_qkv": g((3 * hd, d_model), d_model ** -0.5),
        "b_qkv": g((3 * hd,), 0.1),
        "w_o": g((d_model, hd), hd ** -0.5),
        "b_o": g((d_model,), 0.1),
    }


def make_head_scores(heads: int, seed: int = 3, sigma: float = 0.5):
    """Random per-head importance scores, float64 [heads], log-normal
    exp(N(0, sigma^2)). Stand in for calibrated head scores (a Fisher trace
    per head over a calibration set), which need trained weights and data that
    do not exist here."""
    rng = np.random.default_rng(seed)
    return np.exp(rng.standard_normal(heads) * sigma)


def make_gram(heads: int, head_dim: int = 64, width: int = 1024, seed: int = 1):
    """Random symmetric positive semi-definite matrices [H][D][D], float64.

    Stands in for per-head Gram matrices of an output projection: each is
    A^T A / width with A in R^{width x D} drawn N(0, 1). Used only to exercise
    the non-identity path; no trained weights exist here.
    """
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((heads, width, head_dim))
    return np.ascontiguousarray(np.einsum("hwd,hwe->hde", A, A) / width)
