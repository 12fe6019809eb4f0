"""ress_refine_dropset_noalloc (state in the library's fixed per-GPU scratch)
against ress_refine_dropset (caller workspace): identical keep lists and
J values, bit for bit, on two calls in a row, the second with a smaller
input, so the second call runs on the scratch the first one left behind."""

from __future__ import annotations

import numpy as np
import pytest

import synth
from tests.helpers import to_torch_tokens

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _scored(name):
    import block_sparse_global_amd as b
    w = synth.get_workload(name)
    x = synth.make_inputs(w)
    shape = b.Shape(*w.shape_args())
    layer = b.BlockSparseGlobalAttention(shape, x["keep"], x["always"], mode="drift",
                                         rounds=w.rounds, rho=w.rho)
    q, k, v = (to_torch_tokens(x[t], w.dtype) for t in ("q", "k", "v"))
    layer.pool(q, k, v)
    layer.score()
    layer.select()
    torch.cuda.synchronize()
    return w, x, shape, layer


def _both(w, x, shape, layer):
    import block_sparse_global_amd as b
    idx0, cnt0 = layer.kept_idx.clone(), layer.kept_cnt.clone()
    res = {}
    for impl in ("workspace", "noalloc"):
        idx, cnt = idx0.clone(), cnt0.clone()
        J0 = torch.full((shape.H, shape.nq), np.nan, dtype=torch.float64, device="cuda")
        J1 = torch.full_like(J0, np.nan)
        args = (layer.P, layer.key, layer.vpool, layer.vout, None, shape, x["keep"],
                x["always"], w.rounds, w.rho, 1e-4, layer.k_max, idx, cnt, J0, J1)
        if impl == "workspace":
            b.ress_refine_dropset(*args, workspace=layer.workspace)
        else:
            b.ress_refine_dropset_noalloc(*args)
        torch.cuda.synchronize()
        res[impl] = [t.cpu().numpy() for t in (idx, cnt, J0, J1)]
    for a, c, what in zip(res["workspace"], res["noalloc"], ("kept_idx", "kept_cnt", "J_init",
                                                              "J_final")):
        assert np.array_equal(a, c, equal_nan=False), f"{w.name}: {what} differs"
    assert not np.any(np.isnan(res["noalloc"][3]))
    return res


def test_noalloc_refine_matches_workspace_refine_twice():
    import block_sparse_global_amd as b
    # 100 views: 202 MB of state, refined in groups of heads through the scratch
    w, x, shape, layer = _scored("views100")
    one = b.Shape(1, shape.N, shape.N_pad, shape.D, shape.B)
    assert b.ress_refine_workspace_size(shape) > b.RESS_NOALLOC_SCRATCH_BYTES
    assert b.ress_refine_workspace_size(one) <= b.RESS_NOALLOC_SCRATCH_BYTES
    print(f"\n[noalloc] views100: workspace {b.ress_refine_workspace_size(shape) / 2**20:.1f} MiB",
          flush=True)
    _both(w, x, shape, layer)
    del layer
    # then a smaller shape, all heads in one group, on the scratch as left
    w, x, shape, layer = _scored("views8-k64")
    assert b.ress_refine_workspace_size(shape) <= b.RESS_NOALLOC_SCRATCH_BYTES
    print(f"[noalloc] views8-k64: workspace {b.ress_refine_workspace_size(shape) / 2**20:.2f} MiB",
          flush=True)
    _both(w, x, shape, layer)


def test_noalloc_refine_rejects_a_head_beyond_the_scratch():
    import block_sparse_global_amd as b
    shape = b.Shape(1, 4096 * 64, 4096 * 64, 64, 64)
    assert b.ress_refine_workspace_size(shape) > b.RESS_NOALLOC_SCRATCH_BYTES
    f64 = dict(dtype=torch.float64, device="cuda")
    n = 4096
    P = torch.zeros((1, n, n), **f64)
    V = torch.zeros((1, n, 64), **f64)
    idx = torch.zeros((1, n, 2), dtype=torch.int32, device="cuda")
    cnt = torch.zeros((1, n), dtype=torch.int32, device="cuda")
    with pytest.raises(b.RessError) as ei:
        b.ress_refine_dropset_noalloc(P, P, V, V, None, shape, [2], None, 1, 0.5, 1e-4, 2, idx,
                                      cnt)
    assert ei.value.code == b.RESS_ERR_UNSUPPORTED
