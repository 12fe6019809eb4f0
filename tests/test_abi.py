"""The C-ABI library on the CPU host: it loads, exports every entry point the
header declares, and rejects invalid arguments before any HIP call."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ress.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ress_[a-z_]+)\s*\(", text)))


def test_header_declares_every_call():
    names = declared_functions()
    for f in ("ress_block_pool", "ress_block_score", "ress_select_topk", "ress_select_cdf",
              "ress_select_fused", "ress_select_refine_fused", "ress_refine_dropset", "ress_refine_dropset_fused", "ress_refine_dropset_noalloc",
              "ress_refine_workspace_size",
              "ress_sparse_attn_fwd",
              "ress_gram_from_wo", "ress_head_budgets", "ress_residual_drift",
              "ress_last_error", "ress_version"):
        assert f in names


def test_library_exports_every_declared_symbol():
    import block_sparse_global_amd as b
    lib = ctypes.CDLL(b.LIB_PATH)
    for f in declared_functions():
        assert hasattr(lib, f), f"{f} declared in ress.h but not exported"
    assert b.ress_version() == 5
    assert set(b.ENTRY_POINTS) == set(declared_functions())


def _shape(H=2, N=256, N_pad=256, D=64, B=64, Bk=0):
    import block_sparse_global_amd as b
    return b.Shape(H, N, N_pad, D, B, Bk).c()


FAKE = ctypes.c_void_p(0x1000)        # 16-byte aligned, never dereferenced
MISALIGNED = ctypes.c_void_p(0x1008)


@pytest.mark.parametrize("shape,code,msg", [
    (dict(D=32), -2, "head dimension"),
    (dict(B=32), -2, "block size"),
    (dict(H=0), -1, "H="),
    (dict(N_pad=250), -1, "multiple"),
    (dict(N=100), -1, "N="),
    (dict(N=300), -1, "N="),
    (dict(N=4097 * 64, N_pad=4097 * 64), -2, "cap"),
    (dict(Bk=32), -2, "key block"),
    (dict(Bk=128), -2, "key block"),             # larger than B = 64
    (dict(B=128, Bk=64, N=4096 * 64 + 1, N_pad=4096 * 64 + 128), -2, "cap"),  # n_k = 4097
])
def test_attention_rejects_bad_shapes(shape, code, msg):
    import block_sparse_global_amd as b
    rc = b.LIB.ress_sparse_attn_fwd(FAKE, FAKE, FAKE, 0, _shape(**shape), None, None, 1,
                                    ctypes.c_float(0.125), FAKE, None, None)
    assert rc == code
    assert msg in b.ress_last_error()


def test_attention_argument_checks():
    import block_sparse_global_amd as b
    L = b.LIB
    s = _shape()
    f = ctypes.c_float(0.125)
    assert L.ress_sparse_attn_fwd(None, FAKE, FAKE, 0, s, None, None, 1, f, FAKE, None, None) == -1
    assert L.ress_sparse_attn_fwd(MISALIGNED, FAKE, FAKE, 0, s, None, None, 1, f, FAKE, None, None) == -1
    assert "aligned" in b.ress_last_error()
    assert L.ress_sparse_attn_fwd(FAKE, FAKE, FAKE, 7, s, None, None, 1, f, FAKE, None, None) == -1
    assert L.ress_sparse_attn_fwd(FAKE, FAKE, FAKE, 0, s, None, None, 1, ctypes.c_float(0.0),
                                  FAKE, None, None) == -1
    # kept lists need counts and a sane k_max
    assert L.ress_sparse_attn_fwd(FAKE, FAKE, FAKE, 0, s, FAKE, None, 1, f, FAKE, None, None) == -1
    assert L.ress_sparse_attn_fwd(FAKE, FAKE, FAKE, 0, s, FAKE, FAKE, 0, f, FAKE, None, None) == -1
    assert L.ress_sparse_attn_fwd(FAKE, FAKE, FAKE, 0, s, FAKE, FAKE, 5, f, FAKE, None, None) == -1


def test_pool_argument_checks():
    import block_sparse_global_amd as b
    L = b.LIB
    s = _shape()
    assert L.ress_block_pool(None, None, None, 0, s, None, None, None, None) == -1
    assert L.ress_block_pool(FAKE, None, None, 0, s, None, None, None, None) == -1
    assert "both" in b.ress_last_error()
    assert L.ress_block_pool(FAKE, None, None, 3, s, FAKE, None, None, None) == -1


def test_score_argument_checks():
    import block_sparse_global_amd as b
    L = b.LIB
    s = _shape()
    d = ctypes.c_double
    assert L.ress_block_score(FAKE, FAKE, None, None, s, 2, d(0.1), d(1e-4), FAKE, None, None,
                              None, None) == -1
    assert L.ress_block_score(FAKE, FAKE, None, None, s, 0, d(-1), d(1e-4), FAKE, None, None,
                              None, None) == -1
    # drift needs vpool, key, vout, vmv and eps > 0
    assert L.ress_block_score(FAKE, FAKE, None, None, s, 1, d(0.1), d(1e-4), FAKE, FAKE, FAKE,
                              FAKE, None) == -1
    assert L.ress_block_score(FAKE, FAKE, FAKE, None, s, 1, d(0.1), d(0.0), FAKE, FAKE, FAKE,
                              FAKE, None) == -1
    assert L.ress_block_score(FAKE, FAKE, FAKE, MISALIGNED, s, 1, d(0.1), d(1e-4), FAKE, FAKE,
                              FAKE, FAKE, None) == -1


def _arr(a, t):
    a = np.ascontiguousarray(np.asarray(a, dtype=t))
    return a, a.ctypes.data_as(ctypes.c_void_p)


def test_gram_argument_checks():
    import block_sparse_global_amd as b
    L = b.LIB
    s = _shape(H=2)
    assert L.ress_gram_from_wo(None, 0, 64, s, FAKE, None) == -1
    assert L.ress_gram_from_wo(FAKE, 0, 64, s, MISALIGNED, None) == -1
    assert L.ress_gram_from_wo(FAKE, 5, 64, s, FAKE, None) == -1
    assert L.ress_gram_from_wo(FAKE, 0, 0, s, FAKE, None) == -1
    assert "d_model" in b.ress_last_error()
    assert L.ress_gram_from_wo(FAKE, 0, 64, _shape(D=32), FAKE, None) == -2


def test_selection_budget_checks():
    import block_sparse_global_amd as b
    L = b.LIB
    s = _shape(H=2)           # n = 4
    _, ok_keep = _arr([2, 3], np.int32)
    _, alw = _arr([0, 0, 0, 1], np.uint8)
    assert L.ress_select_topk(FAKE, s, None, None, 3, FAKE, FAKE, None) == -1      # keep NULL
    _, low = _arr([1, 3], np.int32)
    assert L.ress_select_topk(FAKE, s, low, None, 3, FAKE, FAKE, None) == -1       # keep < 2
    _, high = _arr([2, 5], np.int32)
    assert L.ress_select_topk(FAKE, s, high, None, 5, FAKE, FAKE, None) == -1      # keep > n
    assert L.ress_select_topk(FAKE, s, ok_keep, None, 2, FAKE, FAKE, None) == -1   # k_max < keep
    _, alw3 = _arr([1, 1, 1, 0], np.uint8)
    assert L.ress_select_topk(FAKE, s, ok_keep, alw3, 3, FAKE, FAKE, None) == -1   # keep <= always
    _, bad = _arr([0, 2, 0, 0], np.uint8)
    assert L.ress_select_topk(FAKE, s, ok_keep, bad, 3, FAKE, FAKE, None) == -1    # flag not 0/1
    big = _shape(H=65)
    _, k65 = _arr([2] * 65, np.int32)
    assert L.ress_select_topk(FAKE, big, k65, None, 2, FAKE, FAKE, None) == -2     # too many heads
    d = ctypes.c_double
    # the cumulative threshold: the same budget checks, and tau finite and > 0
    assert L.ress_select_cdf(FAKE, s, low, None, d(0.9), 3, FAKE, FAKE, None) == -1
    assert L.ress_select_cdf(FAKE, s, ok_keep, alw3, d(0.9), 3, FAKE, FAKE, None) == -1
    assert L.ress_select_cdf(None, s, ok_keep, None, d(0.9), 3, FAKE, FAKE, None) == -1
    assert L.ress_select_cdf(MISALIGNED, s, ok_keep, None, d(0.9), 3, FAKE, FAKE, None) == -1
    for bad_tau in (0.0, -0.5, float("nan"), float("inf")):
        assert L.ress_select_cdf(FAKE, s, ok_keep, None, d(bad_tau), 3, FAKE, FAKE, None) == -1
        assert "tau" in b.ress_last_error()
    assert L.ress_select_cdf(FAKE, big, k65, None, d(0.9), 2, FAKE, FAKE, None) == -2
    d = ctypes.c_double
    e = d(1e-4)
    assert L.ress_refine_dropset(FAKE, FAKE, FAKE, FAKE, None, s, ok_keep, alw, -1, d(0.5), e,
                                 3, FAKE, FAKE, None, None, FAKE, 1 << 40, None) == -1            # rounds < 0
    assert L.ress_refine_dropset(FAKE, FAKE, FAKE, FAKE, None, s, ok_keep, alw, 2, d(1.5), e,
                                 3, FAKE, FAKE, None, None, FAKE, 1 << 40, None) == -1            # rho > 1
    assert L.ress_refine_dropset(FAKE, FAKE, FAKE, None, None, s, ok_keep, alw, 2, d(0.5), e,
                                 3, FAKE, FAKE, None, None, FAKE, 1 << 40, None) == -1            # vout NULL
    assert L.ress_refine_dropset(FAKE, None, FAKE, FAKE, None, s, ok_keep, alw, 2, d(0.5), e,
                                 3, FAKE, FAKE, None, None, FAKE, 1 << 40, None) == -1            # key NULL
    assert L.ress_refine_dropset(FAKE, FAKE, FAKE, FAKE, None, s, ok_keep, alw, 2, d(0.5),
                                 d(0.0), 3, FAKE, FAKE, None, None, FAKE, 1 << 40, None) == -1    # eps <= 0


def test_refine_workspace_checks():
    import block_sparse_global_amd as b
    L = b.LIB
    s = _shape(H=2)           # n = 4
    _, keep = _arr([2, 3], np.int32)
    _, alw = _arr([0, 0, 0, 1], np.uint8)
    d = ctypes.c_double
    need = L.ress_refine_workspace_size(s)
    # gains (8 n^2 H), two flag maps (n^2 H each), g and M g (512 n H each),
    # row state (64 n H), every region rounded up to 256 bytes
    r256 = lambda x: -(-x // 256) * 256  # noqa: E731
    n, H = 4, 2
    assert need == r256(8 * n * n * H) + 2 * r256(n * n * H) + 2 * r256(512 * n * H) + \
        r256(64 * n * H)
    assert L.ress_refine_workspace_size(_shape(D=32)) == 0 and b.ress_last_error()
    args = (FAKE, FAKE, FAKE, FAKE, None, s, keep, alw, 2, d(0.5), d(1e-4), 3, FAKE, FAKE,
            None, None)
    assert L.ress_refine_dropset(*args, None, need, None) == -1          # no workspace
    assert "workspace is NULL" in b.ress_last_error()
    assert L.ress_refine_dropset(*args, ctypes.c_void_p(0x1010), need, None) == -1
    assert "256-byte" in b.ress_last_error()
    assert L.ress_refine_dropset(*args, FAKE, need - 1, None) == -1      # too small
    assert "smaller" in b.ress_last_error()


def test_fused_refine_argument_checks():
    import block_sparse_global_amd as b
    L = b.LIB
    d = ctypes.c_double
    _, keep = _arr([2, 3], np.int32)
    _, alw = _arr([0, 0, 0, 1], np.uint8)

    def call(s, P=FAKE, keep=keep, alw=alw, rounds=2, rho=0.5, eps=1e-4, k_max=3):
        return L.ress_refine_dropset_fused(P, FAKE, FAKE, FAKE, None, s, keep, alw, rounds,
                                           d(rho), d(eps), k_max, FAKE, FAKE, None, None, None)
    # rows longer than the fused kernel's LDS holds: unsupported, nothing launched
    long = _shape(H=1, N=1089 * 64, N_pad=1089 * 64)
    _, keep1 = _arr([2], np.int32)
    assert call(long, keep=keep1, alw=None) == -2
    assert "1088" in b.ress_last_error()
    s = _shape(H=2)  # n = 4
    assert call(s, P=None) == -1 and "P" in b.ress_last_error()
    assert call(s, rounds=-1) == -1 and "rounds" in b.ress_last_error()
    assert call(s, rho=0.0) == -1 and "rho" in b.ress_last_error()
    assert call(s, eps=0.0) == -1 and "eps" in b.ress_last_error()
    assert call(s, k_max=2) == -1                     # k_max below a budget
    assert b.REFINE_FUSED_MAX_BLOCKS == 1088


def test_select_refine_fused_argument_checks():
    import block_sparse_global_amd as b
    L = b.LIB
    d = ctypes.c_double
    _, keep = _arr([2, 3], np.int32)
    _, alw = _arr([0, 0, 0, 1], np.uint8)

    def call(s, qp=FAKE, vp=FAKE, vmv=FAKE, keep=keep, alw=alw, rounds=2, rho=0.5, eps=1e-4,
             scale=0.125, k_max=3):
        return L.ress_select_refine_fused(qp, FAKE, vp, None, s, d(scale), d(eps), keep, alw,
                                          rounds, d(rho), k_max, vmv, FAKE, FAKE, None, None,
                                          None)
    # rows longer than the tile's LDS holds: unsupported, nothing launched
    long = _shape(H=1, N=1089 * 64, N_pad=1089 * 64)
    _, keep1 = _arr([2], np.int32)
    assert call(long, keep=keep1, alw=None) == -2
    assert "1088" in b.ress_last_error()
    s = _shape(H=2)  # n = 4
    assert call(s, qp=None) == -1 and "qpool" in b.ress_last_error()
    assert call(s, vp=None) == -1 and "vpool" in b.ress_last_error()
    assert call(s, vmv=None) == -1 and "vmv" in b.ress_last_error()
    assert call(s, qp=MISALIGNED) == -1 and "aligned" in b.ress_last_error()
    assert call(s, rounds=-1) == -1 and "rounds" in b.ress_last_error()
    assert call(s, rho=0.0) == -1 and "rho" in b.ress_last_error()
    assert call(s, eps=0.0) == -1 and "eps" in b.ress_last_error()
    assert call(s, scale=float("inf")) == -1 and "scale" in b.ress_last_error()
    assert call(s, k_max=2) == -1                     # k_max below a budget
    assert b.SELECT_REFINE_FUSED_MAX_BLOCKS == 1088


def test_noalloc_refine_argument_checks():
    import block_sparse_global_amd as b
    L = b.LIB
    d = ctypes.c_double
    _, keep = _arr([2, 3], np.int32)
    _, alw = _arr([0, 0, 0, 1], np.uint8)

    def call(s, P=FAKE, keep=keep, alw=alw, rounds=2, rho=0.5, eps=1e-4, k_max=3):
        return L.ress_refine_dropset_noalloc(P, FAKE, FAKE, FAKE, None, s, keep, alw, rounds,
                                             d(rho), d(eps), k_max, FAKE, FAKE, None, None, None)
    s = _shape(H=2)  # n = 4
    assert call(s, P=None) == -1 and "P" in b.ress_last_error()
    assert call(s, P=MISALIGNED) == -1 and "aligned" in b.ress_last_error()
    assert call(s, rounds=-1) == -1 and "rounds" in b.ress_last_error()
    assert call(s, rho=1.5) == -1 and "rho" in b.ress_last_error()
    assert call(s, eps=0.0) == -1 and "eps" in b.ress_last_error()
    assert call(s, k_max=2) == -1                     # k_max below a budget
    # a single head whose refinement state exceeds the fixed scratch:
    # unsupported, reported before any HIP call
    big = _shape(H=1, N=2536 * 64, N_pad=2536 * 64)
    _, keep1 = _arr([2], np.int32)
    assert call(big, keep=keep1, alw=None, k_max=2) == -2
    assert "scratch" in b.ress_last_error()
    assert b.RESS_NOALLOC_SCRATCH_BYTES == 64 << 20
    hdr = open(HEADER).read()
    assert "#define RESS_NOALLOC_SCRATCH_BYTES (64u << 20)" in hdr


def test_layer_argument_checks_before_any_allocation():
    import block_sparse_global_amd as b
    from block_sparse_global_amd.layer import refine_path
    s = b.Shape(1, 1089 * 64, 1089 * 64, 64, 64)
    # rows beyond the fused kernel's limit fall back to the per-round kernels
    assert refine_path(s, "fused") == "rounds"
    assert refine_path(b.Shape(1, 1088 * 64, 1088 * 64, 64, 64), "fused") == "fused"
    assert refine_path(s, "rounds") == "rounds"
    with pytest.raises(ValueError):
        refine_path(s, "auto")
    from block_sparse_global_amd.layer import SELECT_FUSED_AUTO_MAX_BLOCKS, select_path
    short = b.Shape(1, SELECT_FUSED_AUTO_MAX_BLOCKS * 64, SELECT_FUSED_AUTO_MAX_BLOCKS * 64,
                    64, 64)
    longer = b.Shape(1, (SELECT_FUSED_AUTO_MAX_BLOCKS + 1) * 64,
                     (SELECT_FUSED_AUTO_MAX_BLOCKS + 1) * 64, 64, 64)
    # "auto": the fused pass on short rows without refinement or threshold
    assert select_path(short, "auto", 0, None) == "fused"
    assert select_path(longer, "auto", 0, None) == "unfused"
    assert select_path(short, "auto", 1, None) == "unfused"
    assert select_path(short, "auto", 0, 0.5) == "unfused"
    assert select_path(longer, "fused", 0, None) == "fused"
    assert select_path(s, "fused", 0, None) == "fused"
    assert select_path(b.Shape(1, 2177 * 64, 2177 * 64, 64, 64), "fused", 0, None) == "unfused"
    # with refinement rounds "fused" is the one-pass selection up to 1088 blocks
    assert select_path(short, "fused", 2, None) == "fused"
    assert select_path(s, "fused", 2, None) == "unfused"
    assert select_path(b.Shape(1, 1088 * 64, 1088 * 64, 64, 64), "fused", 2, None) == "fused"
    assert select_path(short, "fused", 2, 0.5) == "unfused"
    assert select_path(short, "unfused", 0, None) == "unfused"
    with pytest.raises(ValueError):
        select_path(short, "fast", 0, None)
    with pytest.raises(ValueError):
        b.BlockSparseGlobalAttention(s, [2], None, mode="drift", rounds=1, refine_impl="auto")
    with pytest.raises(ValueError, match="drift"):
        b.BlockSparseGlobalAttention(s, [2], None, mode="prob", rounds=1)


def test_error_string_is_cleared_per_thread():
    import threading
    import block_sparse_global_amd as b
    b.LIB.ress_block_pool(None, None, None, 0, _shape(D=32), None, None, None, None)
    assert b.ress_last_error()
    seen = []
    th = threading.Thread(target=lambda: seen.append(b.ress_last_error()))
    th.start(); th.join()
    assert seen == [""]


def test_python_binding_rejects_host_tensors():
    import torch
    import block_sparse_global_amd as b
    shape = b.Shape(1, 128, 128, 64, 64)
    x = torch.zeros((1, 128, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        b.ress_sparse_attn_fwd(x, x, x, shape, None, None, 1, 0.125, x)


def test_head_budgets_match_the_oracle_and_check_arguments():
    """The host allocation against the oracle on random scores (bit-exact
    integers), and its argument checks."""
    import block_sparse_global_amd as b
    import oracle
    r = np.random.default_rng(61)
    for trial in range(200):
        H = int(r.integers(1, 65))
        n_k = int(r.integers(4, 2200))
        n_alw = int(r.integers(0, 9))
        always = np.zeros(n_k, np.uint8); always[n_k - n_alw:] = 1
        f = max(1, 2 - n_alw)
        score = r.gamma(0.5, 1.0, H) * (r.uniform(size=H) < 0.9)
        if trial % 17 == 0:
            score[:] = 0.0
        total = int(r.integers(H * (n_alw + f), H * n_k + 1))
        got = b.ress_head_budgets(score, n_k, always if n_alw else None, total)
        want, _ = oracle.head_budgets(score, n_k, always if n_alw else None, total)
        assert np.array_equal(got, want), (trial, got, want)
    with pytest.raises(b.RessError):
        b.ress_head_budgets([1.0, -1.0], 10, None, 10)
    with pytest.raises(b.RessError):
        b.ress_head_budgets([1.0, float("nan")], 10, None, 10)
    with pytest.raises(b.RessError):
        b.ress_head_budgets([1.0, 1.0], 10, None, 3)      # below two blocks per head
    with pytest.raises(b.RessError):
        b.ress_head_budgets([1.0, 1.0], 10, None, 21)     # above n_k per head
    with pytest.raises(b.RessError):
        b.ress_head_budgets([1.0] * 65, 10, None, 200)    # too many heads

