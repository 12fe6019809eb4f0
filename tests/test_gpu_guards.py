"""Guard bytes around every output buffer of every entry point (including the
no-allocation refinement, the fused selection and both projections).

Each output (and the refinement workspace) is a view into a larger device
allocation whose 256 bytes before and after it are filled with a sentinel;
after the call (and a synchronisation) the sentinels must be intact, so no
kernel writes outside the extent its arguments give. Run at 8 views and on
seeded ragged shapes (both block grids, partial last blocks).
"""

from __future__ import annotations

import numpy as np
import pytest

import synth
from synth.workloads import custom
from tests.helpers import to_torch_tokens

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GUARD = 256           # bytes on either side
SENTINEL = 0xA5


class Guarded:
    """A contiguous device tensor of `shape` inside a sentinel-filled buffer."""

    def __init__(self, shape, dtype, fill=None):
        esize = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape))
        self.raw = torch.full((n * esize + 2 * GUARD,), SENTINEL, dtype=torch.uint8,
                              device="cuda")
        body = self.raw[GUARD:GUARD + n * esize]
        self.t = body.view(dtype).view(shape)
        if fill is not None:
            self.t.copy_(fill)

    def check(self, what):
        torch.cuda.synchronize()
        head = self.raw[:GUARD].cpu().numpy()
        tail = self.raw[-GUARD:].cpu().numpy()
        assert np.all(head == SENTINEL), f"{what}: bytes before the buffer overwritten"
        assert np.all(tail == SENTINEL), f"{what}: bytes after the buffer overwritten"


def _workloads():
    yield "views8", synth.get_workload("views8")
    rng = np.random.default_rng(2024)
    made = 0
    while made < 4:
        block = int(rng.choice([64, 128]))
        w = custom(name=f"g{made}", views=int(rng.integers(1, 4)),
                   patches_per_view=int(rng.integers(50, 700)),
                   specials_per_view=int(rng.choice([0, 5])), heads=int(rng.integers(1, 4)),
                   block=block, key_block=int(rng.choice([0, 64])) if block == 128 else 0,
                   sparsity=(0.5, 0.8), score="drift", rounds=2,
                   seed=int(rng.integers(1 << 30)))
        if w.n_kblocks < 3:
            continue
        made += 1
        yield w.name, w


@pytest.mark.parametrize("name,w", list(_workloads()), ids=lambda v: v if isinstance(v, str) else "")
def test_guard_bytes_around_every_output(name, w):
    import block_sparse_global_amd as b
    x = synth.make_inputs(w)
    shape = b.Shape(*w.shape_args())
    H, nq, nk, D, Np = shape.H, shape.nq, shape.nk, shape.D, shape.N_pad
    q, k, v = (to_torch_tokens(x[t], w.dtype) for t in ("q", "k", "v"))
    f64 = torch.float64
    keep, alw = x["keep"], x["always"]
    k_max = int(np.max(keep))

    qp, kp, vp = Guarded((H, nq, D), f64), Guarded((H, nk, D), f64), Guarded((H, nk, D), f64)
    b.ress_block_pool(q, k, v, shape, qp.t, kp.t, vp.t)
    for g, s in ((qp, "qpool"), (kp, "kpool"), (vp, "vpool")):
        g.check(f"ress_block_pool {s}")

    M = torch.from_numpy(synth.make_gram(H, D, seed=5)).cuda()
    P, key = Guarded((H, nq, nk), f64), Guarded((H, nq, nk), f64)
    vout, vmv = Guarded((H, nq, D), f64), Guarded((H, nk), f64)
    b.ress_block_score(qp.t, kp.t, vp.t, M, shape, b.RESS_SCORE_DRIFT, 0.125, 1e-4, P.t, key.t,
                       vout.t, vmv.t)
    for g, s in ((P, "P"), (key, "key"), (vout, "vout"), (vmv, "vmv")):
        g.check(f"ress_block_score {s}")

    idx, cnt = Guarded((H, nq, k_max), torch.int32), Guarded((H, nq), torch.int32)
    b.ress_select_topk(key.t, shape, keep, alw, k_max, idx.t, cnt.t)
    idx.check("ress_select_topk kept_idx")
    cnt.check("ress_select_topk kept_cnt")
    idx0, cnt0 = idx.t.clone(), cnt.t.clone()

    ci, cc = Guarded((H, nq, k_max), torch.int32), Guarded((H, nq), torch.int32)
    b.ress_select_cdf(P.t, shape, keep, alw, 0.2, k_max, ci.t, cc.t)
    ci.check("ress_select_cdf kept_idx")
    cc.check("ress_select_cdf kept_cnt")

    ws_bytes = b.ress_refine_workspace_size(shape)
    for impl in ("rounds", "fused"):
        if impl == "fused" and nk > b.REFINE_FUSED_MAX_BLOCKS:
            continue
        ri, rc = Guarded((H, nq, k_max), torch.int32, idx0), Guarded((H, nq), torch.int32, cnt0)
        J0, J1 = Guarded((H, nq), f64), Guarded((H, nq), f64)
        if impl == "rounds":
            ws = Guarded((ws_bytes,), torch.uint8)
            b.ress_refine_dropset(P.t, key.t, vp.t, vout.t, M, shape, keep, alw, 2, 0.5, 1e-4,
                                  k_max, ri.t, rc.t, J0.t, J1.t, ws.t)
            ws.check("ress_refine_dropset workspace")
        else:
            b.ress_refine_dropset_fused(P.t, key.t, vp.t, vout.t, M, shape, keep, alw, 2, 0.5,
                                        1e-4, k_max, ri.t, rc.t, J0.t, J1.t)
        for g, s in ((ri, "kept_idx"), (rc, "kept_cnt"), (J0, "J_init"), (J1, "J_final")):
            g.check(f"refine ({impl}) {s}")

    Mg = Guarded((H, D, D), f64)
    wo = torch.from_numpy(synth.make_wo(H, D, 256).view(np.int16)).view(torch.bfloat16).cuda()
    b.ress_gram_from_wo(wo, shape, Mg.t)
    Mg.check("ress_gram_from_wo M")

    dt = q.dtype
    out, lse = Guarded((H, Np, D), dt), Guarded((H, Np), torch.float32)
    b.ress_sparse_attn_fwd(q, k, v, shape, idx0, cnt0, k_max, 0.125, out.t, lse.t)
    out.check("ress_sparse_attn_fwd out")
    lse.check("ress_sparse_attn_fwd lse")
    dout, dlse = Guarded((H, Np, D), dt), Guarded((H, Np), torch.float32)
    b.dense_attention(q, k, v, shape, dout.t, lse=dlse.t)
    dout.check("ress_sparse_attn_fwd (dense) out")
    dlse.check("ress_sparse_attn_fwd (dense) lse")

    drift = Guarded((H, nq), f64)
    b.ress_residual_drift(out.t, dout.t, shape, drift.t, M)
    drift.check("ress_residual_drift drift")

    ri, rc = Guarded((H, nq, k_max), torch.int32, idx0), Guarded((H, nq), torch.int32, cnt0)
    J0, J1 = Guarded((H, nq), f64), Guarded((H, nq), f64)
    b.ress_refine_dropset_noalloc(P.t, key.t, vp.t, vout.t, M, shape, keep, alw, 2, 0.5, 1e-4,
                                  k_max, ri.t, rc.t, J0.t, J1.t)
    for g, s in ((ri, "kept_idx"), (rc, "kept_cnt"), (J0, "J_init"), (J1, "J_final")):
        g.check(f"ress_refine_dropset_noalloc {s}")

    if nk <= b.SELECT_FUSED_MAX_BLOCKS:
        fi, fc = Guarded((H, nq, k_max), torch.int32), Guarded((H, nq), torch.int32)
        fv = Guarded((H, nk), f64)
        b.ress_select_fused(qp.t, kp.t, vp.t, M, shape, b.RESS_SCORE_DRIFT, 0.125, 1e-4, keep,
                            alw, k_max, fv.t, fi.t, fc.t)
        for g, s in ((fi, "kept_idx"), (fc, "kept_cnt"), (fv, "vmv")):
            g.check(f"ress_select_fused {s}")

    if nk <= b.SELECT_REFINE_FUSED_MAX_BLOCKS:
        fi, fc = Guarded((H, nq, k_max), torch.int32), Guarded((H, nq), torch.int32)
        fv, J0, J1 = Guarded((H, nk), f64), Guarded((H, nq), f64), Guarded((H, nq), f64)
        b.ress_select_refine_fused(qp.t, kp.t, vp.t, M, shape, 0.125, 1e-4, keep, alw, 2, 0.5,
                                   k_max, fv.t, fi.t, fc.t, J0.t, J1.t)
        for g, s in ((fi, "kept_idx"), (fc, "kept_cnt"), (fv, "vmv"), (J0, "J_init"),
                     (J1, "J_final")):
            g.check(f"ress_select_refine_fused {s}")

    if w.dtype == "bf16":
        dm = 128
        L = synth.make_sublayer(Np, H, D, dm, seed=7)
        bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(  # noqa: E731
            torch.bfloat16).cuda()
        xs, wq, bq, wo2, bo = (bf(L[n]) for n in ("x", "w_qkv", "b_qkv", "w_o", "b_o"))
        pq, pk, pv = (Guarded((H, Np, D), torch.bfloat16) for _ in range(3))
        b.ress_qkv_project(xs, wq, bq, shape, pq.t, pk.t, pv.t)
        for g, s in ((pq, "q"), (pk, "k"), (pv, "v")):
            g.check(f"ress_qkv_project {s}")
        y = Guarded((Np, dm), torch.bfloat16)
        b.ress_out_project(pq.t, wo2, bo, xs, shape, y.t)
        y.check("ress_out_project y")
        yr = Guarded((Np, dm), torch.bfloat16, xs)
        b.ress_out_project(pq.t, wo2, bo, yr.t, shape, yr.t)
        yr.check("ress_out_project y (in place)")
