"""GPU parity of the linear maps around the attention call: the QKV
projection and the output projection with the residual add (bf16 matrix
cores, float32 accumulation), against the float64 oracle; then the whole
sublayer x -> QKV -> selection -> attention -> W_O + residual, and the
ReSS page's Eq. 6/8 at token level on the GPU's own outputs."""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import synth
from tests.helpers import attention_parity, kept_mask_from_lists

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _t(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _f(t):
    return t.float().cpu().numpy().astype(np.float64)


def _close_bf16(got, want, absmag, what):
    """Each output within one bf16 rounding (2^-8 relative, the rounding of
    the float32 result plus its own) of the exact value, plus the float32
    accumulation error, bounded by 2^-14 times the sum of the magnitudes of
    the terms (K <= 1024 terms)."""
    err = np.abs(got - want)
    tol = 2.0 ** -8 * np.abs(want) + 2.0 ** -14 * absmag + 1e-30
    bad = err > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} outputs off; worst excess "
                           f"{np.max(err - tol):.3e}")


SHAPES = [  # H, N, N_pad, B, d_model
    (2, 1000, 1024, 128, 192),
    (1, 300, 320, 64, 64),        # partial 128-row tiles, 192 output channels
    (16, 10992, 11008, 128, 1024),  # the 8-view VGGT-L global layer
]
# Products with at least four 256 x 256 tiles per CU take the big-tile kernel:
# 86 x 12 tiles for this QKV projection (the last row tile partial), 256 x 4
# for this output projection.
BIG_QKV = (16, 22000, 22016, 128, 1024)
BIG_OUT = (16, 65500, 65536, 128, 1024)


@pytest.mark.parametrize("H,N,N_pad,B,dm", SHAPES + [BIG_QKV])
def test_qkv_project(H, N, N_pad, B, dm):
    import block_sparse_global_amd as b
    L = synth.make_sublayer(N_pad, H, 64, dm, seed=H + dm)
    shape = b.Shape(H, N, N_pad, 64, B)
    x, w, bias = _t(L["x"]), _t(L["w_qkv"]), _t(L["b_qkv"])
    q, k, v = (torch.full((H, N_pad, 64), float("nan"), dtype=torch.bfloat16, device="cuda")
               for _ in range(3))
    b.ress_qkv_project(x, w, bias, shape, q, k, v)
    torch.cuda.synchronize()
    xf, wf, bf = (synth.as_f64(L[n], "bf16") for n in ("x", "w_qkv", "b_qkv"))
    want = oracle.qkv_project(xf, wf, bf, H, 64, N)
    mags = oracle.qkv_project(np.abs(xf), np.abs(wf), np.abs(bf), H, 64, N)
    for name, g_t, r, m in zip("qkv", (q, k, v), want, mags):
        g = _f(g_t)
        _close_bf16(g[:, :N], r[:, :N], m[:, :N], name)
        assert np.all(g[:, N:] == 0), f"{name}: padded rows must be zero"


@pytest.mark.parametrize("H,N,N_pad,B,dm,mode",
                         [s + (m,) for s in SHAPES for m in ("residual", "in_place", "plain")]
                         + [BIG_OUT + ("residual",), BIG_OUT + ("in_place",)])
def test_out_project(H, N, N_pad, B, dm, mode):
    import block_sparse_global_amd as b
    L = synth.make_sublayer(N_pad, H, 64, dm, seed=7 * H + dm)
    shape = b.Shape(H, N, N_pad, 64, B)
    r = np.random.default_rng(H)
    o_bits = synth.f32_to_bf16_bits(r.standard_normal((H, N_pad, 64)).astype(np.float32))
    o, w, bias = _t(o_bits), _t(L["w_o"]), _t(L["b_o"])
    res = _t(L["x"]) if mode != "plain" else None
    if mode == "in_place":
        y = res
    else:
        y = torch.full((N_pad, dm), float("nan"), dtype=torch.bfloat16, device="cuda")
    b.ress_out_project(o, w, bias if mode != "plain" else None, res, shape, y)
    torch.cuda.synchronize()
    of, wf, bf, xf = (synth.as_f64(a, "bf16") for a in (o_bits, L["w_o"], L["b_o"], L["x"]))
    use_b, use_r = (bf, xf) if mode != "plain" else (None, None)
    want = oracle.out_project(of, wf, use_b, use_r)
    mag = oracle.out_project(np.abs(of), np.abs(wf), None if use_b is None else np.abs(use_b),
                             None if use_r is None else np.abs(use_r))
    _close_bf16(_f(y), want, mag, f"y ({mode})")


def test_sublayer_end_to_end_and_residual_drift_at_token_level():
    """x -> ress_qkv_project -> pool/score/top-k/refine -> attention ->
    ress_out_project (in place on the residual x) at 8 views with a 1024-wide
    model. Each stage is checked against the oracle on the GPU's own inputs to
    that stage; then Eq. 6 and 8 at token level: with the residual and bias
    left out, the mean over a block of ||y_sparse - y_dense||^2 (two real W_O
    products on the GPU) equals ress_residual_drift with M = W_O^T W_O from
    ress_gram_from_wo, up to the bf16 rounding of y."""
    import block_sparse_global_amd as b
    w = synth.get_workload("views8")
    H, N, N_pad, B = w.heads, w.N, w.N_pad, w.block
    dm = 1024
    L = synth.make_sublayer(N_pad, H, 64, dm, seed=11)
    shape = b.Shape(H, N, N_pad, 64, B)
    x = _t(L["x"])
    q, k, v = (torch.empty((H, N_pad, 64), dtype=torch.bfloat16, device="cuda") for _ in range(3))
    b.ress_qkv_project(x, _t(L["w_qkv"]), _t(L["b_qkv"]), shape, q, k, v)
    x0 = synth.make_inputs(w)  # the workload's budgets and always-kept blocks
    Mg = torch.empty((H, 64, 64), dtype=torch.float64, device="cuda")
    b.ress_gram_from_wo(_t(L["w_o"]), shape, Mg)
    layer = b.BlockSparseGlobalAttention(shape, x0["keep"], x0["always"], mode="drift",
                                         rounds=2, rho=0.5, M=Mg, with_lse=True)
    o = torch.empty_like(q)
    layer(q, k, v, o)
    y = x.clone()
    b.ress_out_project(o, _t(L["w_o"]), _t(L["b_o"]), y, shape, y)
    torch.cuda.synchronize()
    # projection in front, against the oracle
    xf, wq, bq = (synth.as_f64(L[n], "bf16") for n in ("x", "w_qkv", "b_qkv"))
    want = oracle.qkv_project(xf, wq, bq, H, 64, N)
    mags = oracle.qkv_project(np.abs(xf), np.abs(wq), np.abs(bq), H, 64, N)
    qkv = [_f(t) for t in (q, k, v)]
    for name, g, r, m in zip("qkv", qkv, want, mags):
        _close_bf16(g[:, :N], r[:, :N], m[:, :N], name)
    # attention on the GPU's q, k, v and kept lists, every query block
    kept = kept_mask_from_lists(layer.kept_idx.cpu().numpy(), layer.kept_cnt.cpu().numpy(),
                                w.n_kblocks)
    mx, mean, rel, lmax, _ = attention_parity(*qkv, kept, _f(o), layer.lse.cpu().numpy(), N, B,
                                              B, 0.125, list(range(H)))
    assert mx <= 2e-2 and mean <= 2e-3, (mx, mean)
    # output projection with the residual, on the GPU's attention output
    wo, bo = synth.as_f64(L["w_o"], "bf16"), synth.as_f64(L["b_o"], "bf16")
    of = _f(o)
    _close_bf16(_f(y), oracle.out_project(of, wo, bo, xf),
                oracle.out_project(np.abs(of), np.abs(wo), np.abs(bo), np.abs(xf)), "y")
    # Eq. 6/8 at token level: y_sparse - y_dense through the real W_O product
    dense = torch.empty_like(q)
    b.dense_attention(q, k, v, shape, dense)
    ys = torch.empty_like(x)
    yd = torch.empty_like(x)
    b.ress_out_project(o, _t(L["w_o"]), None, None, shape, ys)
    b.ress_out_project(dense, _t(L["w_o"]), None, None, shape, yd)
    drift = torch.empty((H, shape.nq), dtype=torch.float64, device="cuda")
    b.ress_residual_drift(o, dense, shape, drift, Mg)
    torch.cuda.synchronize()
    dy = _f(ys)[:N] - _f(yd)[:N]
    per_tok = np.sum(dy * dy, axis=1)
    nb = shape.nq
    blockmean = np.array([per_tok[i * B:min((i + 1) * B, N)].mean() for i in range(nb)])
    # all heads change at once here, so the token-level change is the sum over
    # heads of W_O^h e_h, and ||.||^2 includes the cross terms between heads:
    # compare against the oracle's residual stream change instead, and check
    # the per-head Gram form separately on one head
    e = _f(o) - _f(dense)
    oy = oracle.out_project(e, wo, None, None)[:N]
    want_bm = np.array([np.sum(oy[i * B:min((i + 1) * B, N)] ** 2, axis=1).mean()
                        for i in range(nb)])
    rel_err = np.abs(blockmean - want_bm) / want_bm
    assert np.median(rel_err) < 2e-2 and rel_err.max() < 0.2, (np.median(rel_err), rel_err.max())
    # one head alone: the GPU's Gram-form drift equals the explicit W_O^h product
    h = 3
    e1 = np.zeros_like(e)
    e1[h] = e[h]
    y1 = oracle.out_project(e1, wo, None, None)[:N]
    want1 = np.array([np.sum(y1[i * B:min((i + 1) * B, N)] ** 2, axis=1).mean()
                      for i in range(nb)])
    np.testing.assert_allclose(drift.cpu().numpy()[h], want1, rtol=1e-9)
    print(f"\n[sublayer] attention max-abs {mx:.3e}; token-level drift: median rel "
          f"{np.median(rel_err):.2e} vs the oracle's W_O product")
