"""float64 CPU oracle of block-sparse global attention — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module. It is deliberately plain: numpy in
float64, no blocking, fusion or reordering beyond what the definitions state,
so that each function can be checked against the pages by eye.

Sources ("the ReSS page" below is "ReSS: Residual-Restoring Sparse Attention
for 3D Vision Transformers"; "the subject page" is "Block-Sparse Global
Attention for Efficient Multi-View Geometry Transformers"):

* §3 "Block-Sparse Attention for 3D ViTs" of the ReSS page: blocks are mean
  pooled into a block-level attention map; per (query block, head) key blocks
  are selected up to a per-head budget; exact attention runs over the
  selected blocks only, with softmax renormalised among them; blocks holding
  special tokens are never dropped.
* §4.1 (Eq. 1-2), §4.2 (Eq. 3-9), §4.3 (Eq. 10-17) of the ReSS page: the
  pooled dense output, the drift score and the drop-set refinement.
* The subject page's abstract: training-free block-sparse replacement of
  dense global attention.

Readings where the pages leave a step open (each one is listed with its
reason in the design notes of the repository):

* softmax scale 1/sqrt(D) for both the pooled map and token attention;
* the pooled map is the softmax over all key blocks of the scaled dot
  products of mean-pooled Q and K (not token probabilities pooled after the
  fact); a partial (padded) block is pooled over its valid tokens only;
* ties in any top-k / top-m go to the lower block index;
* the cumulative-probability (CDF) selection takes the always-kept blocks'
  mass first, then candidates by probability descending until the mass
  reaches the threshold, capped by the per-head budget and raised to the
  two-block floor;
* refinement rounds are batched: restore and drop gains both come from the
  round-start state, m_r = floor(rho * c / 2^(r+1)), both sets applied, then
  g, K, G recomputed from their definitions; a drop whose K + u <= 0 gets a
  gain of -inf; track-best keeps a new set only when its J is strictly lower.

Parity pins: every function here is checked against closed forms, library
routines, explicit masking and brute force in ``tests/test_oracle_pins.py``.
"""

from __future__ import annotations

import math
from typing import Optional

import numpy as np


# ---------------------------------------------------------------------------
# Step 1: mean pooling and the pooled block-level map (ReSS page, §3 step (1))
# ---------------------------------------------------------------------------

def block_pool(x: np.ndarray, N: int, B: int) -> np.ndarray:
    """Mean of the valid tokens of every block.

    x: float64 [H][N_pad][D]; tokens t >= N are padding and are ignored.
    Returns float64 [H][n][D] with n = ceil(N / B) blocks of B tokens, the
    last one possibly partial.  (ReSS page, §3: "mean pooling within each
    block".)
    """
    H, N_pad, D = x.shape
    n = -(-N // B)
    out = np.empty((H, n, D), dtype=np.float64)
    for b in range(n):
        lo, hi = b * B, min((b + 1) * B, N)
        out[:, b, :] = x[:, lo:hi, :].mean(axis=1)
    return out


def block_map(qpool: np.ndarray, kpool: np.ndarray, scale: float) -> np.ndarray:
    """Pooled attention probabilities P[h][i][j], normalised over all key blocks.

    P_ij = softmax_j(scale * qpool_i . kpool_j) over every key block j
    (ReSS page, §4.1: the map is normalised over the set of all key blocks).
    """
    logits = scale * np.matmul(qpool, np.swapaxes(kpool, 1, 2))
    m = logits.max(axis=-1, keepdims=True)
    e = np.exp(logits - m)
    return e / e.sum(axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
# Step 2: block scores
# ---------------------------------------------------------------------------

def pooled_output(P: np.ndarray, vpool: np.ndarray) -> np.ndarray:
    """Dense pooled attention output, ReSS page Eq. 1: vout_i = sum_j P_ij V_j."""
    return np.matmul(P, vpool)


def _gram(M: Optional[np.ndarray], h: int, D: int) -> np.ndarray:
    return np.eye(D) if M is None else M[h]


def gram_from_wo(W: np.ndarray, H: int, D: int) -> np.ndarray:
    """Per-head Gram matrices of the output projection, ReSS page Eq. 8:
    M_h = (W_O^h)^T W_O^h with W_O^h the columns h*D .. h*D+D-1 of
    W [d_model][H*D] (the head's slice of the projection into the residual
    stream). Returns float64 [H][D][D]."""
    M = np.empty((H, D, D), dtype=np.float64)
    for h in range(H):
        Wh = np.asarray(W[:, h * D:(h + 1) * D], dtype=np.float64)
        M[h] = Wh.T @ Wh
    return M


def drift_key(P: np.ndarray, vpool: np.ndarray, M: Optional[np.ndarray],
              eps: float = 1e-4, row_chunk: int = 64):
    """ReSS drift ranking key, Eq. 5-7, in the direct (unexpanded) form.

    e_ij = vout_i - V_j (Eq. 4's deviation), q_ij = e_ij^T M_h e_ij (the
    squared residual-space norm of Eq. 6 written with the Gram matrix of
    Eq. 8; M_h = I when M is None), s_ij = P_ij sqrt(q_ij) (Eq. 6), and the
    key is s_ij / max(1 - P_ij, eps) (Eq. 7). q is clamped at 0 against
    rounding. Returns (key, vout, q), all float64.
    """
    H, nq, nk = P.shape
    D = vpool.shape[-1]
    vout = pooled_output(P, vpool)
    q = np.empty((H, nq, nk), dtype=np.float64)
    for h in range(H):
        Mh = _gram(M, h, D)
        for i0 in range(0, nq, row_chunk):
            i1 = min(nq, i0 + row_chunk)
            e = vout[h, i0:i1, None, :] - vpool[h, None, :, :]  # [ci][n][D]
            Me = e if M is None else np.matmul(e, Mh)          # M_h = I: e itself
            q[h, i0:i1] = np.sum(Me * e, axis=-1)
    q = np.maximum(q, 0.0)
    s = P * np.sqrt(q)
    key = s / np.maximum(1.0 - P, eps)
    return key, vout, q


# ---------------------------------------------------------------------------
# Step 3: per-row top-k selection (ReSS page, §3 step (2) and §4.1 Eq. 2)
# ---------------------------------------------------------------------------

def _order_desc(values: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Positions of idx sorted by value descending, then index ascending."""
    return np.lexsort((idx, -values))


def _rel_gap(a: float, b: float) -> float:
    den = max(abs(a), abs(b))
    if den == 0.0:
        return 0.0
    if not (math.isfinite(a) and math.isfinite(b)):
        return math.inf if a != b else 0.0
    return abs(a - b) / den


def select_topk(key: np.ndarray, keep: np.ndarray, always: np.ndarray):
    """Kept key blocks of every (head, query-block row).

    Candidates are the blocks not flagged in ``always``; per row the c_h =
    keep[h] - |always| candidates with the largest key are selected (ties to
    the lower block index), and the always-kept blocks are added (ReSS page
    §4.1: blocks holding special tokens are always kept, the candidate set P
    is the rest, |S| = c_h).

    Returns (kept bool [H][n][n], margin float64 [H][n]) where margin is the
    relative gap between the c-th and (c+1)-th candidate keys of the row
    (inf when every candidate is kept).
    """
    H, n, _ = key.shape
    cand = np.nonzero(always == 0)[0]
    alw = np.nonzero(always != 0)[0]
    kept = np.zeros(key.shape, dtype=bool)
    margin = np.full((H, n), np.inf)
    for h in range(H):
        c = int(keep[h]) - len(alw)
        for i in range(n):
            kv = key[h, i, cand]
            order = _order_desc(kv, cand)
            chosen = cand[order[:c]]
            kept[h, i, chosen] = True
            kept[h, i, alw] = True
            if c < len(cand):
                margin[h, i] = _rel_gap(kv[order[c - 1]], kv[order[c]])
    return kept, margin


def select_cdf(P: np.ndarray, keep: np.ndarray, always: np.ndarray, tau: float,
               floor: int = 2, rows=None):
    """Kept key blocks under a cumulative-probability (top-p, "CDF") threshold
    with the per-head budget as a cap.

    This is the probability selection the ReSS page compares against: its
    related-work section describes SparseVGGT as keeping the blocks with large
    mass on the pooled map through top-k and top-p criteria; §4.4 and the
    "+ CDF threshold" row of Table 2 contrast such a threshold, whose keep
    count depends on the data, with a fixed budget; Appendix F applies the
    sink rule (special blocks always kept) and a floor of two key blocks per
    query row to every method. The pages do not print the rule itself; the
    reading taken here, per (head, query-block row):

    * s = sum of P over the always-kept blocks, accumulated in ascending
      block order (those blocks are kept whatever the threshold);
    * candidates (the other blocks) are visited by P descending, ties to the
      lower block index; while s < tau and fewer than c_h = keep[h] - |always|
      candidates are taken, take the next one and add its P to s (float64,
      one addition at a time in that order);
    * the row is then raised to at least ``floor`` kept blocks by taking the
      next candidates in the same order.

    Returns (kept bool [H][n][n], taken int [H][n] = number of candidates
    kept, margin float64 [H][n]) where margin is the relative distance
    between tau and the cumulative mass just before and just after the
    decisive candidate (the smaller of the two; inf when the cap or the
    floor decided the count), for near-tie checks.
    """
    H, n, _ = P.shape
    cand = np.nonzero(always == 0)[0]
    alw = np.nonzero(always != 0)[0]
    kept = np.zeros(P.shape, dtype=bool)
    taken = np.zeros((H, n), dtype=np.int64)
    margin = np.full((H, n), np.inf)
    todo = rows if rows is not None else [(h, i) for h in range(H) for i in range(n)]
    for h, i in todo:
        c = int(keep[h]) - len(alw)
        s = 0.0
        for j in alw:
            s += float(P[h, i, j])
        pv = P[h, i, cand]
        order = _order_desc(pv, cand)
        m = 0
        before = s
        while s < tau and m < c:
            before = s
            s += float(pv[order[m]])
            m += 1
        if s >= tau and m > 0:
            margin[h, i] = min(_rel_gap(before, tau), _rel_gap(s, tau))
        elif s >= tau:
            margin[h, i] = _rel_gap(s, tau)
        m = max(m, floor - len(alw))
        m = min(m, c)
        kept[h, i, cand[order[:m]]] = True
        kept[h, i, alw] = True
        taken[h, i] = m
    return kept, taken, margin


def kept_lists(kept: np.ndarray):
    """Ascending block-index lists and counts from a kept mask."""
    H, n, nk = kept.shape
    cnt = kept.sum(axis=-1).astype(np.int32)
    kmax = int(cnt.max()) if cnt.size else 0
    idx = np.full((H, n, kmax), -1, dtype=np.int32)
    for h in range(H):
        for i in range(n):
            js = np.nonzero(kept[h, i])[0]
            idx[h, i, : len(js)] = js
    return idx, cnt


def head_budgets(score, n_k: int, always, total_keep: int):
    """Per-head keep budgets from head importance scores: the HeSS allocation
    the ReSS page adopts (§4.4; Appendix D: proportional allocation with
    iterative clipping at the cap).

    Reading: every head first gets the floor f = max(1, 2 - |always|)
    candidates (two kept blocks per row, Appendix F, and at least one
    candidate); the surplus U = total_keep - H (|always| + f) is split in
    proportion to the scores (equally if all are 0); heads whose share
    exceeds the cap (n_k - |always| - f) are fixed at the cap and the rest
    of U is split again among the others, until no share exceeds the cap.
    Integers: shares rounded down, then one unit each to the largest
    fractional parts (ties: lower head), never beyond the cap.

    Returns (keep int [H], share float64 [H]) with share the real-valued
    surplus allocation before rounding.
    """
    score = [float(x) for x in score]
    H = len(score)
    n_alw = int(np.sum(np.asarray(always) != 0)) if always is not None else 0
    f = max(1, 2 - n_alw)
    capU = float(n_k - n_alw - f)
    U = float(total_keep - H * (n_alw + f))
    clipped = [False] * H
    a = [0.0] * H
    while True:
        active = [h for h in range(H) if not clipped[h]]
        S = 0.0
        for h in active:
            S += score[h]
        R = U - capU * (H - len(active))
        for h in active:
            a[h] = R * score[h] / S if S > 0.0 else R / len(active)
        over = [h for h in active if a[h] > capU]
        if not over:
            break
        for h in over:
            clipped[h] = True
            a[h] = capU
    share = list(a)
    b = [min(math.floor(x), int(capU)) for x in a]
    rem = int(U) - sum(b)
    frac = [x - math.floor(x) for x in a]
    while rem > 0:
        cands = [h for h in range(H) if b[h] < int(capU)]
        best = max(cands, key=lambda h: (frac[h], -h))
        b[best] += 1
        frac[best] = 0.0
        rem -= 1
    keep = np.array([n_alw + f + x for x in b], dtype=np.int32)
    return keep, np.array(share)


# ---------------------------------------------------------------------------
# Step 4: drop-set refinement (ReSS page, §4.3, Eq. 10-17)
# ---------------------------------------------------------------------------

def swap_schedule(c: int, rounds: int, rho: float):
    """Swaps per round, Eq. 17 m_r = rho 2^-(r+1) c, rounded down."""
    return [int(math.floor(rho * c / (2.0 ** (r + 1)))) for r in range(rounds)]


def drop_objective(p_row, d_row, Mh, D_mask):
    """Eq. 10 and Eq. 12 for one row and drop set D.

    g = sum_{j in D} d_j, K = 1 - sum_{j in D} P_j, G = g^T M g, J = G / K^2.
    J is +inf when K <= 0.
    """
    g = d_row[D_mask].sum(axis=0)
    K = 1.0 - p_row[D_mask].sum()
    G = float(g @ Mh @ g)
    J = G / (K * K) if K > 0 else math.inf
    return g, K, G, J


def swap_gains(p_row, d, s2, Mh, g, K, G):
    """Objective decrease of every single swap from the state (g, K, G).

    Restore of k (k in D): Delta G = -2 d_k^T M g + s_k^2 (Eq. 14), u = +P_k.
    Drop of k (k kept):    Delta G = +2 d_k^T M g + s_k^2 (Eq. 15), u = -P_k.
    Delta J = G / K^2 - (G + Delta G) / (K + u)^2 (Eq. 16); a drop with
    K + u <= 0 gets -inf. Both arrays cover every k; the caller masks them.
    """
    dMg = d @ (Mh @ g)                      # d_k^T M g for every k
    dG_restore = -2.0 * dMg + s2
    dG_drop = 2.0 * dMg + s2
    dJ_restore = G / K**2 - (G + dG_restore) / (K + p_row) ** 2
    Kd = K - p_row
    with np.errstate(divide="ignore", invalid="ignore"):
        dJ_drop = np.where(Kd > 0, G / K**2 - (G + dG_drop) / Kd**2, -np.inf)
    return dJ_restore, dJ_drop


def _top_m(gain, members, m):
    """Indices of the m members with the largest gain (ties: lower index),
    and the relative gap at the cut (inf if all members are taken)."""
    idx = np.nonzero(members)[0]
    order = _order_desc(gain[idx], idx)
    chosen = idx[order[:m]]
    gap = math.inf
    if m < len(idx):
        gap = _rel_gap(gain[idx[order[m - 1]]], gain[idx[order[m]]])
    return chosen, gap


def refine_row(p_row, vpool_h, vout_row, Mh, cand, kept_row, c, rounds, rho):
    """Iterative residual restoration of one (head, query-block) row.

    Follows §4.3 of the ReSS page: start from D = P minus the initial
    selection; each round r computes, from the round-start g, K and G, the
    restore gain of every k in D (Eq. 13-14, u = +P_k) and the drop gain of
    every kept candidate (Eq. 15, u = -P_k) as the exact objective decrease
    of Eq. 16; restores the m_r blocks of D with the largest gains and drops
    the m_r kept candidates with the largest gains (Eq. 17); then recomputes
    g, K, G (Eq. 10, 12). The drop set with the smallest J seen is returned
    (track-best).

    Returns (best_kept_row bool [n], J_init, J_best, min_margin) where
    min_margin is the smallest relative gap met at any selection cut or
    track-best comparison along the way.
    """
    e = vout_row[None, :] - vpool_h            # e_j = vout_i - V_j
    d = p_row[:, None] * e                      # Eq. 5
    s2 = np.einsum("jd,de,je->j", d, Mh, d)     # (s_j)^2 = d_j^T M d_j (Eq. 6)
    D_mask = cand & ~kept_row
    g, K, G, J = drop_objective(p_row, d, Mh, D_mask)
    J_init = J
    best, J_best = D_mask.copy(), J
    margin = math.inf
    for m in swap_schedule(c, rounds, rho):
        S_mask = cand & ~D_mask
        m = min(m, int(D_mask.sum()), int(S_mask.sum()))
        if m <= 0:
            continue
        dJ_restore, dJ_drop = swap_gains(p_row, d, s2, Mh, g, K, G)
        restore, gap_r = _top_m(dJ_restore, D_mask, m)
        drop, gap_d = _top_m(dJ_drop, S_mask, m)
        margin = min(margin, gap_r, gap_d)
        D_mask = D_mask.copy()
        D_mask[restore] = False
        D_mask[drop] = True
        g, K, G, J = drop_objective(p_row, d, Mh, D_mask)
        margin = min(margin, _rel_gap(J, J_best))
        if J < J_best:
            best, J_best = D_mask.copy(), J
    return cand & ~best, J_init, J_best, margin


def refine_dropset(P, vpool, vout, M, keep, always, kept, rounds, rho,
                   rows=None):
    """Refine every (or the listed) rows. Returns (kept', J_init, J_final,
    margin); kept' is a copy of ``kept`` with the refined rows replaced, and
    the per-row arrays are NaN for rows not refined."""
    H, nq, nk = P.shape
    D = vpool.shape[-1]
    cand = always == 0
    n_alw = int((always != 0).sum())
    out = kept.copy()
    J0 = np.full((H, nq), np.nan)
    J1 = np.full((H, nq), np.nan)
    mg = np.full((H, nq), np.nan)
    todo = rows if rows is not None else [(h, i) for h in range(H) for i in range(nq)]
    for h, i in todo:
        Mh = _gram(M, h, D)
        c = int(keep[h]) - n_alw
        kr, a, b, m = refine_row(P[h, i], vpool[h], vout[h, i], Mh, cand,
                                 kept[h, i] & cand, c, rounds, rho)
        out[h, i] = kr | (always != 0)
        J0[h, i], J1[h, i], mg[h, i] = a, b, m
    return out, J0, J1, mg


# ---------------------------------------------------------------------------
# Step 5: exact attention over the kept blocks (ReSS page §3 step (3))
# ---------------------------------------------------------------------------

def masked_attention(q, k, v, kept, N: int, B: int, scale: float,
                     blocks=None, Bk: Optional[int] = None):
    """O[h, t] = sum_u softmax_u(scale q_t . k_u) v_u over the valid keys u < N
    of the blocks kept for t's query block; softmax renormalised among them
    (ReSS page §3: the unselected blocks take no part in the softmax).

    q, k, v: float64 [H][N_pad][D]; query block i holds tokens i*B ..
    i*B + B - 1 and key block j tokens j*Bk .. j*Bk + Bk - 1 (Bk = B when not
    given); kept: bool [H][n_q][n_k]. Padded query rows are 0. ``blocks``:
    optional list of (h, i) query blocks to compute (the rest stay 0).
    Returns (O float64 [H][N_pad][D], lse float64 [H][N_pad]).
    """
    H, N_pad, D = q.shape
    Bk = B if Bk is None else Bk
    n = N_pad // B
    O = np.zeros((H, N_pad, D), dtype=np.float64)
    lse = np.full((H, N_pad), np.nan)
    todo = blocks if blocks is not None else [(h, i) for h in range(H) for i in range(n)]
    for h, i in todo:
        r0, r1 = i * B, min((i + 1) * B, N)
        if r1 <= r0:
            continue
        keys = np.concatenate([np.arange(j * Bk, min((j + 1) * Bk, N))
                               for j in np.nonzero(kept[h, i])[0]])
        s = scale * (q[h, r0:r1] @ k[h, keys].T)
        m = s.max(axis=1, keepdims=True)
        p = np.exp(s - m)
        l = p.sum(axis=1, keepdims=True)
        O[h, r0:r1] = (p @ v[h, keys]) / l
        lse[h, r0:r1] = (m + np.log(l))[:, 0]
    return O, lse


def dense_attention(q, k, v, N: int, B: int, scale: float, blocks=None,
                    Bk: Optional[int] = None):
    """Dense softmax attention over all valid keys: every block kept."""
    H, N_pad, _ = q.shape
    Bk = B if Bk is None else Bk
    kept = np.ones((H, N_pad // B, -(-N // Bk)), dtype=bool)
    return masked_attention(q, k, v, kept, N, B, scale, blocks, Bk)


def residual_drift(O_sparse, O_dense, M, N: int, B: int):
    """Mean over the valid tokens t of every query block of e_t^T M_h e_t,
    e_t = O_sparse[h, t] - O_dense[h, t] (ReSS page Eq. 6 and 9 at token
    level: ||W_O^h e_t||^2 when M_h = (W_O^h)^T W_O^h; ||e_t||^2 for M None).

    O_sparse, O_dense: float64 [H][N_pad][D]. Returns float64 [H][n_q].
    """
    H, N_pad, D = O_sparse.shape
    n = N_pad // B
    out = np.zeros((H, n), dtype=np.float64)
    for h in range(H):
        Mh = _gram(M, h, D)
        for i in range(n):
            t0, t1 = i * B, min((i + 1) * B, N)
            if t1 <= t0:
                continue
            e = O_sparse[h, t0:t1] - O_dense[h, t0:t1]
            out[h, i] = np.mean(np.sum((e @ Mh) * e, axis=1))
    return out


# ---------------------------------------------------------------------------
# The linear maps around the attention call (ReSS page §3: pre-LN residual
# sublayer; §4.2 "Mapping to the residual space", Eq. 6 and 8)
# ---------------------------------------------------------------------------

def qkv_project(x, W, b, H: int, D: int, N: int):
    """Per-head Q, K, V from the token features: the linear layer
    y = x W^T + b with output channel c = which * H*D + h*D + d (which = 0, 1,
    2 for Q, K, V). x: float64 [N_pad][d_model]; W: [3 H D][d_model]; b:
    [3 H D] or None. Returns q, k, v float64 [H][N_pad][D], rows t >= N zero."""
    y = x @ W.T
    if b is not None:
        y = y + b[None, :]
    N_pad = x.shape[0]
    out = []
    for which in range(3):
        t = np.zeros((H, N_pad, D), dtype=np.float64)
        for h in range(H):
            c0 = which * H * D + h * D
            t[h, :N] = y[:N, c0:c0 + D]
        out.append(t)
    return tuple(out)


def out_project(o, W, b, residual):
    """The output projection with the residual add: head h's output o[h]
    enters the residual stream as W_O^h o^h (Eq. 6, 8), W_O^h the columns
    h*D .. h*D+D-1 of W [d_model][H D]:
    y[t] = residual[t] + b + sum_h W_O^h o[h][t]. o: float64 [H][N_pad][D];
    b: [d_model] or None; residual: [N_pad][d_model] or None."""
    H, N_pad, D = o.shape
    y = np.zeros((N_pad, W.shape[0]), dtype=np.float64)
    for h in range(H):
        y += o[h] @ W[:, h * D:(h + 1) * D].T
    if b is not None:
        y = y + b[None, :]
    if residual is not None:
        y = y + residual
    return y


# ---------------------------------------------------------------------------
# The whole selection path for one workload
# ---------------------------------------------------------------------------

def run_selection(q, k, v, N, B, keep, always, mode, rounds=0, rho=0.5,
                  M=None, eps=1e-4, scale=None, Bk=None):
    """pool -> map -> key -> top-k (-> refine) on float64 inputs; queries in
    blocks of B tokens, keys and values in blocks of Bk (default B).

    Returns a dict with qpool, kpool, vpool, P, key, vout (drift only),
    kept (after top-k), topk_margin, and when rounds > 0: kept_refined,
    J_init, J_final, refine_margin.
    """
    D = q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = {}
    Bk = B if Bk is None else Bk
    out["qpool"] = block_pool(q, N, B)
    out["kpool"] = block_pool(k, N, Bk)
    out["P"] = block_map(out["qpool"], out["kpool"], scale)
    if mode == "drift" or rounds > 0:
        out["vpool"] = block_pool(v, N, Bk)
    if mode == "drift":
        key, vout, qd = drift_key(out["P"], out["vpool"], M, eps)
        out["key"], out["vout"], out["q"] = key, vout, qd
    else:
        out["key"] = out["P"].copy()
    out["kept"], out["topk_margin"] = select_topk(out["key"], keep, always)
    if rounds > 0:
        if "vout" not in out:
            out["vout"] = pooled_output(out["P"], out["vpool"])
        kr, J0, J1, mg = refine_dropset(out["P"], out["vpool"], out["vout"], M,
                                        keep, always, out["kept"], rounds, rho)
        out["kept_refined"], out["J_init"], out["J_final"], out["refine_margin"] = (
            kr, J0, J1, mg)
    return out
