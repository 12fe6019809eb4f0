"""Benchmark of one block-sparse global-attention step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload views100]

A step is the whole path over one synthetic multi-view input already
resident in HBM: pool -> score -> top-k -> [refine] -> sparse attention. The
default workload is 100 views x 1374 tokens (137,400 tokens, 16 heads,
head_dim 64, block 128, 90% sparsity, drift score + 3 refinement rounds),
the only configuration that exercises every step. Printed: one JSON line with
the kept-block attention throughput of the whole step (kept FLOPs / step
time), the layer latency against the dense kernel at 8/32/100 views (and 200
views with either score), the
roofline of the attention kernel (timed with HIP events on the launch
stream) and the CPU oracle timed on a bounded sample.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "kept-block attention TFLOP/s + layer latency (ms) vs dense at 8/32/100 views"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0

# Cumulative-probability threshold of the "views100-cdf" line. The synthetic
# pooled maps are flat (the 107 best of 1074 blocks hold ~10% of a row's
# mass), so a threshold that binds below the 10% cap is small: 0.05 keeps
# about 53 blocks per row, a data-dependent count (46..48 candidates + 5).
CDF_TAU = 0.05

# HBM bytes of one attention launch on the 100-view workload, from two
# rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE, KiB per
# dispatch, median over dispatches), scaled by what the same counters read for
# a 1 GiB device copy (FETCH_SIZE x2.0, WRITE_SIZE x1.0). The figures hold only
# for the kernel source they were taken on; any other source reports null.
ATTN_TRAFFIC = {
    "workload": "views100",
    "source_sha256": "eb6ff29c685cdab33915feda1976406b89f456d3c9d7cba45c2b0c290ec67883",
    "read_bytes": 8715566336,
    "write_bytes": 457521152,
}


# The pages' own speed figures, for context only: whole-model forward times
# of VGGT on NVIDIA GPUs (every layer, not the attention call alone), so not
# comparable with the attention-layer speedups measured here.
PAGES_CONTEXT = [
    {"what": "SparseVGGT vs dense VGGT forward, 100 views, sparsity 0.745",
     "speedup": round(10.47 / 7.58, 2), "seconds": [10.47, 7.58], "hardware": "RTX 4090",
     "source": "ReSS page, Table 1 (cost analysis) and Table S7 (dense latency)"},
    {"what": "ReSS selection (drift score + 5 fused restoration rounds) added to that forward",
     "seconds_added": 0.24, "seconds_added_unfused": 1.26, "hardware": "RTX 4090",
     "source": "ReSS page, Table 1 (cost analysis)"},
    {"what": "VASC vs dense VGGT forward, NRGBD stride-10 sequences, 85% sparsity",
     "speedup": 2.29, "seconds": [15.631, 6.822], "hardware": "RTX 4090",
     "source": "VASC page, Table 2 (full-model efficiency on NeuralRGB-D)"},
]


def _valid_tokens(N, blk, nb):
    valid = np.full(nb, blk, dtype=np.int64)
    valid[-1] = N - (nb - 1) * blk
    return valid


def kept_flops(w, idx, cnt):
    """4 * D * sum over kept (query block, key block) pairs of valid q * valid k."""
    n = w.n_blocks
    vq = _valid_tokens(w.N, w.block, n)
    vk = _valid_tokens(w.N, w.kblock, w.n_kblocks)
    tot = 0
    for h in range(idx.shape[0]):
        for i in range(n):
            js = idx[h, i, : cnt[h, i]]
            tot += int(vq[i]) * int(vk[js].sum())
    return 4.0 * w.head_dim * tot


def sparsity_of(w, cnt):
    """1 - kept (query block, key block) pairs / all pairs."""
    return 1.0 - float(cnt.sum()) / (w.heads * w.n_blocks * w.n_kblocks)


def dense_flops(w):
    return 4.0 * w.head_dim * w.heads * float(w.N) * float(w.N)


def setup(name, mode=None, x=None, tau=None, select_impl="auto"):
    import torch

    import block_sparse_global_amd as bsg
    import synth
    w = synth.get_workload(name)
    if x is None:
        x = synth.make_inputs(w)
    to_t = (lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()) \
        if w.dtype == "bf16" else (lambda a: torch.from_numpy(a).cuda())
    q, k, v = to_t(x["q"]), to_t(x["k"]), to_t(x["v"])
    shape = bsg.Shape(*w.shape_args())
    if mode is None:
        mode = "drift" if w.score in ("drift", "both") else "prob"
    layer = bsg.BlockSparseGlobalAttention(shape, x["keep"], x["always"], mode=mode,
                                           rounds=w.rounds if mode == "drift" else 0,
                                           rho=w.rho, tau=tau, select_impl=select_impl)
    out = torch.empty_like(q)
    return w, x, shape, layer, (q, k, v), out


def hess_inputs(name):
    """Inputs of workload `name` with per-head budgets from stand-in head
    scores, allocated by ress_head_budgets (proportional with clipping) at
    the same total budget as the workload's own."""
    import block_sparse_global_amd as bsg
    import synth
    w = synth.get_workload(name)
    x = dict(synth.make_inputs(w))
    x["keep"] = bsg.ress_head_budgets(synth.make_head_scores(w.heads), w.n_kblocks,
                                      x["always"], int(np.sum(x["keep"])))
    return x


def attn_traffic(workload):
    """Counter-measured bytes of one attention launch, or None when the kernel
    source or the workload differs from the ones the counters were taken on."""
    import hashlib
    src = os.path.join(ROOT, "block_sparse_global_amd", "csrc", "attn.hip")
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if sha != ATTN_TRAFFIC["source_sha256"] or workload != ATTN_TRAFFIC["workload"]:
        return None
    return ATTN_TRAFFIC["read_bytes"] + ATTN_TRAFFIC["write_bytes"]


def time_events(fn, reps):
    """Mean ms per call over `reps` back-to-back calls (one event pair)."""
    import torch
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def time_median(fn, reps=20):
    """Median ms of `reps` calls, each between its own pair of HIP events on
    the launch stream (torch's current stream, which the binding passes)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev]))


def measured_peaks():
    """This GPU's measured bf16 matrix-core rate and HBM copy bandwidth, next
    to the published peaks: an MFMA loop (v_mfma_f32_32x32x16_bf16 on
    independent accumulators, two workgroups of four waves per CU) with the
    shader clock read from the core-cycle and 100 MHz counters, and a 2 GiB
    device-to-device copy (read + write bytes)."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "block_sparse_global_amd", "libress_probe.so")
    lib = ctypes.CDLL(path)
    lib.ress_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p]
    lib.ress_probe_mfma.restype = ctypes.c_int
    props = torch.cuda.get_device_properties(0)
    wgs = 2 * props.multi_processor_count
    iters = 20000
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
    st = torch.cuda.current_stream().cuda_stream

    def run():
        assert lib.ress_probe_mfma(wgs, iters, sink.data_ptr(), clocks.data_ptr(), st) == 0
    run()
    ms = time_median(run, 5)
    flops = wgs * 4 * iters * 8 * (32 * 32 * 16 * 2)
    cyc, ref = (int(v) for v in clocks.cpu().tolist())
    clock_ghz = cyc / (ref / 100e6) / 1e9 if ref > 0 else None
    nb = 1 << 31
    src = torch.empty(nb, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    cms = time_median(lambda: dst.copy_(src), 5)
    del dst
    lib.ress_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p]
    lib.ress_probe_hbm_read.restype = ctypes.c_int
    rwg = 8 * props.multi_processor_count
    rsink = torch.empty(rwg * 256, dtype=torch.int32, device="cuda")

    def read():
        assert lib.ress_probe_hbm_read(src.data_ptr(), nb, rwg, rsink.data_ptr(), st) == 0
    read()
    rms = time_median(read, 5)
    del src, sink, rsink
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": flops / (ms * 1e-3) / 1e12,
            "shader_clock_ghz_under_mfma": clock_ghz,
            "mfma_probe": f"{wgs} workgroups x 4 waves x {iters} x 8 independent "
                          f"v_mfma_f32_32x32x16_bf16, median of 5",
            "hbm_read_gbs": nb / (rms * 1e-3) / 1e9,
            "hbm_copy_gbs": 2 * nb / (cms * 1e-3) / 1e9,
            "hbm_probe": "2 GiB streaming read (non-temporal 16-byte loads, "
                         f"{rwg} workgroups) and a 2 GiB device-to-device copy (read + write "
                         "bytes), medians of 5",
            "published": {"mfma_bf16_tflops": PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS,
                          "clock_ghz": 2.4}}


def stage_breakdown(layer, qkv, out, reps):
    """Median ms per stage over `reps` steps, HIP events between the stages on
    the launch stream."""
    import torch
    q, k, v = qkv
    names = ["pool", "score", "select", "refine", "attend"]
    acc = {n: [] for n in names}
    for _ in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        ev[0].record()
        layer.pool(q, k, v); ev[1].record()
        layer.score(); ev[2].record()
        layer.select(); ev[3].record()
        layer.refine(); ev[4].record()
        layer.attend(q, k, v, out); ev[5].record()
        torch.cuda.synchronize()
        for i, n in enumerate(names):
            acc[n].append(ev[i].elapsed_time(ev[i + 1]))
    return {n: float(np.median(acc[n])) for n in names}


def scoring_memory(layer):
    """Device bytes the selection step keeps besides Q, K, V and the output,
    by buffer (the page's Table 1 reports the same quantity as scoring
    memory): pooled blocks, the block map P and the key, the pooled output
    and V^T M V, the keep lists, J, and the refinement workspace."""
    parts = {}
    for name in ("qpool", "kpool", "vpool", "P", "key", "vout", "vmv", "kept_idx", "kept_cnt",
                 "J_init", "J_final", "workspace"):
        t = getattr(layer, name, None)
        if t is not None:
            parts[name] = int(t.numel() * t.element_size())
    total = sum(parts.values())
    # the fused refinement keeps its per-row state on chip: no workspace; the
    # one-pass selection with refinement also keeps P, the key and vout on
    # chip
    res = {"bytes": total, "by_buffer": parts,
           "bytes_with_fused_refinement": total - parts.get("workspace", 0)}
    if "workspace" in parts:
        res["bytes_one_pass"] = total - sum(parts.get(b, 0) for b in ("P", "key", "vout",
                                                                      "workspace"))
    return res


def select_paths(names=("views8", "views32"), reps=20):
    """Score + top-k by the split calls (block map and key written, then
    read back) and by the fused pass (ress_select_fused), median ms on the
    same pooled blocks, with whether the two keep lists agree."""
    import torch
    res = {}
    for name in names:
        w, x, shape, a, qkv, _ = setup(name, select_impl="unfused")
        _, _, _, b, _, _ = setup(name, x=x, select_impl="fused")
        entry = {}
        for impl, L in (("unfused", a), ("fused", b)):
            L.pool(*qkv)

            def run(L=L):
                L.score()
                L.select()
            run()
            entry[impl] = time_median(run, reps)
        torch.cuda.synchronize()
        entry["identical_lists"] = bool(torch.equal(a.kept_idx, b.kept_idx)
                                        and torch.equal(a.kept_cnt, b.kept_cnt))
        entry["key_blocks"] = shape.nk
        res[name] = entry
        del a, b, qkv
        torch.cuda.empty_cache()
    return res


def budget_sweep(name, budgets, x=None, reps=10):
    """The attention kernel alone at one workload's token count with a
    uniform budget of c kept key blocks per row (probability top-k, the
    always-kept blocks included), for each c: median ms and TFLOP/s, and a
    least-squares line ms = fixed + per_block * c, which separates the cost
    of one more kept block in every row from what a launch costs regardless
    of the budget (reading Q, writing O, launch and ramp)."""
    import torch

    import synth
    w = synth.get_workload(name)
    if x is None:
        x = synth.make_inputs(w)
    pts = []
    for c in budgets:
        x2 = dict(x)
        x2["keep"] = np.full(w.heads, int(c), dtype=np.int32)
        _, _, _, lay, (q, k, v), out = setup(name, mode="prob", x=x2)
        lay(q, k, v, out)
        ms = time_median(lambda: lay.attend(q, k, v, out), reps)
        kf = kept_flops(w, lay.kept_idx.cpu().numpy(), lay.kept_cnt.cpu().numpy())
        pts.append({"keep": int(c), "attn_ms": ms, "tflops": kf / (ms * 1e-3) / 1e12})
        del lay, q, k, v, out
        torch.cuda.empty_cache()
    cs = np.array([p["keep"] for p in pts], dtype=np.float64)
    ms = np.array([p["attn_ms"] for p in pts])
    per_block, fixed = np.polyfit(cs, ms, 1)
    return {"workload": name, "points": pts, "fit_fixed_ms": float(fixed),
            "fit_ms_per_kept_block": float(per_block),
            "rows": int(w.heads * w.n_blocks)}


def torch_sdpa(names=("views8", "views32", "views100"), reps=5):
    """Outside context for the attention kernel: torch's own fused
    scaled_dot_product_attention (dense, bf16, [1][H][N_pad][64]) on the same
    GPU, restricted to its flash and memory-efficient kernels (never the
    unfused math path); median ms and TFLOP/s on N_pad^2 (padding included),
    next to this library's dense kernel at the same shape. None for a shape
    torch has no fused kernel for."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel

    import block_sparse_global_amd as bsg
    import synth
    res = {}
    for name in names:
        w = synth.get_workload(name)
        H, Np = w.heads, w.N_pad
        g = torch.Generator(device="cuda").manual_seed(5)
        q, k, v = (torch.randn((1, H, Np, 64), generator=g, device="cuda",
                               dtype=torch.float32).to(torch.bfloat16) for _ in range(3))
        flop = 4.0 * 64 * H * float(Np) * float(Np)
        entry = {"N_pad": Np}
        for label, backend in (("flash", SDPBackend.FLASH_ATTENTION),
                               ("efficient", SDPBackend.EFFICIENT_ATTENTION)):
            try:
                with sdpa_kernel([backend]):
                    f = lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v)  # noqa: E731
                    f()
                    torch.cuda.synchronize()
                    ms = time_median(f, reps)
                entry[label] = {"ms": ms, "tflops": flop / (ms * 1e-3) / 1e12}
            except RuntimeError as e:
                entry[label] = {"error": str(e).splitlines()[0][:120]}
        shape = bsg.Shape(H, Np, Np, 64, w.block)
        q3, k3, v3 = (t.view(H, Np, 64) for t in (q, k, v))
        o3 = torch.empty_like(q3)
        fd = lambda: bsg.dense_attention(q3, k3, v3, shape, o3)  # noqa: E731
        fd()
        ms = time_median(fd, reps)
        entry["libress_dense"] = {"ms": ms, "tflops": flop / (ms * 1e-3) / 1e12}
        res[name] = entry
        del q, k, v, q3, k3, v3, o3
        torch.cuda.empty_cache()
    return res


def projections(w, reps=20):
    """The linear maps around the attention call at this workload's token
    count with a 1024-wide model (16 heads x 64): the QKV projection and the
    output projection with the residual add, on synthetic bf16 weights;
    median ms and TFLOP/s (2 N_pad d_model 3 H D and 2 N_pad d_model H D)."""
    import torch

    import block_sparse_global_amd as bsg
    import synth
    dm = 1024
    shape = bsg.Shape(*w.shape_args())
    L = synth.make_sublayer(w.N_pad, w.heads, w.head_dim, dm, seed=11)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(  # noqa: E731
        torch.bfloat16).cuda()
    x, wq, bq, wo, bo = (t(L[n]) for n in ("x", "w_qkv", "b_qkv", "w_o", "b_o"))
    q, k, v = (torch.empty((w.heads, w.N_pad, w.head_dim), dtype=torch.bfloat16, device="cuda")
               for _ in range(3))
    y = torch.empty_like(x)
    f_qkv = lambda: bsg.ress_qkv_project(x, wq, bq, shape, q, k, v)  # noqa: E731
    f_out = lambda: bsg.ress_out_project(q, wo, bo, x, shape, y)  # noqa: E731
    f_qkv()
    f_out()
    a, b = time_median(f_qkv, reps), time_median(f_out, reps)
    fa = 2.0 * w.N_pad * dm * 3 * w.heads * w.head_dim
    fb = 2.0 * w.N_pad * dm * w.heads * w.head_dim
    res = {"d_model": dm, "qkv_ms": a, "qkv_tflops": fa / (a * 1e-3) / 1e12,
           "out_ms": b, "out_tflops": fb / (b * 1e-3) / 1e12}
    res["qkv_frac_of_peak"] = res["qkv_tflops"] / PEAK_BF16_TFLOPS
    res["out_frac_of_peak"] = res["out_tflops"] / PEAK_BF16_TFLOPS
    del x, wq, bq, wo, bo, q, k, v, y
    torch.cuda.empty_cache()
    return res


def refine_paths_ms(w, x, shape, layer, reps):
    """The refinement step by both library paths on the same top-k lists:
    kernels per round (the layer's) and the fused kernel; None without
    refinement or for rows longer than the fused kernel takes."""
    import torch

    import block_sparse_global_amd as bsg
    if layer.rounds <= 0 or shape.nk > bsg.REFINE_FUSED_MAX_BLOCKS:
        return None
    fused = bsg.BlockSparseGlobalAttention(shape, x["keep"], x["always"], mode=layer.mode,
                                           rounds=layer.rounds, rho=layer.rho, M=layer.M,
                                           refine_impl="fused")
    for buf in ("P", "key", "vpool", "vout"):  # the same score outputs
        setattr(fused, buf, getattr(layer, buf))
    layer.select()  # the top-k lists both paths start from
    idx0, cnt0 = layer.kept_idx.clone(), layer.kept_cnt.clone()
    res = {}
    for name, L in (("rounds", layer), ("fused", fused)):
        def run():
            L.kept_idx.copy_(idx0)
            L.kept_cnt.copy_(cnt0)
            L.refine()
        run()
        res[name] = time_events(run, reps)
    same = all(torch.equal(getattr(layer, f), getattr(fused, f))
               for f in ("kept_idx", "kept_cnt", "J_init", "J_final"))
    layer.kept_idx.copy_(idx0)
    layer.kept_cnt.copy_(cnt0)
    layer.refine()
    res["identical"] = bool(same)
    res["note"] = "includes restoring the top-k lists before each call"
    return res


def one_pass_selection_ms(w, x, shape, layer, qkv, reps):
    """Scoring, top-k and refinement by the split calls (the layer's: map,
    key and the refinement workspace in HBM) against the one-pass call
    (ress_select_refine_fused, map and key on chip), median ms from the same
    pooled blocks, with how many rows' keep lists differ; None without
    refinement or for rows longer than the one-pass kernel takes."""
    import torch

    import block_sparse_global_amd as bsg
    if layer.rounds <= 0 or shape.nk > bsg.SELECT_REFINE_FUSED_MAX_BLOCKS:
        return None
    one = bsg.BlockSparseGlobalAttention(shape, x["keep"], x["always"], mode=layer.mode,
                                         rounds=layer.rounds, rho=layer.rho, M=layer.M,
                                         select_impl="fused")
    assert one.select_impl == "fused"
    res = {}
    for name, L in (("split", layer), ("one_pass", one)):
        L.pool(*qkv)

        def run(L=L):
            L.score()
            L.select()
            L.refine()
        run()
        res[name] = time_median(run, reps)
    torch.cuda.synchronize()
    differ = torch.any(layer.kept_idx != one.kept_idx, dim=-1) | (layer.kept_cnt != one.kept_cnt)
    res["rows_differ"] = int(differ.sum().item())
    res["rows"] = int(differ.numel())
    del one
    torch.cuda.empty_cache()
    return res


def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def _oracle_attention_rate(w, x, idx, cnt, budget_s, seed=11):
    """The oracle's masked attention on random query blocks of w with the
    GPU's kept lists, until about budget_s seconds: (TFLOP/s, blocks, s)."""
    import oracle
    import synth
    rng = np.random.default_rng(seed)
    n, B = w.n_blocks, w.block
    qf = synth.as_f64(x["q"], w.dtype)
    kf = synth.as_f64(x["k"], w.dtype)
    vf = synth.as_f64(x["v"], w.dtype)
    vq = _valid_tokens(w.N, B, n)
    vk = _valid_tokens(w.N, w.kblock, w.n_kblocks)
    flops, spent, blocks = 0.0, 0.0, 0
    while spent < budget_s and blocks < w.heads * n:
        h, i = int(rng.integers(w.heads)), int(rng.integers(n))
        kept = np.zeros((1, n, w.n_kblocks), bool)
        kept[0, i, idx[h, i, : cnt[h, i]]] = True
        t0 = time.perf_counter()
        oracle.masked_attention(qf[h:h + 1], kf[h:h + 1], vf[h:h + 1], kept, w.N, B,
                                1.0 / math.sqrt(w.head_dim), blocks=[(0, i)], Bk=w.kblock)
        spent += time.perf_counter() - t0
        flops += 4.0 * w.head_dim * vq[i] * vk[idx[h, i, : cnt[h, i]]].sum()
        blocks += 1
    return flops / spent / 1e12, blocks, spent


def _oracle_selection_rate(w, x, rows_max=64, seed=12):
    """The oracle's selection (pool -> map -> key -> top-k -> refine) for a
    sample of query-block rows of w: pooling is timed over the whole tensors,
    the per-row steps on the sampled rows. Returns seconds for the whole
    workload (scaled from the sample) and the sample description."""
    import oracle
    import synth
    rng = np.random.default_rng(seed)
    f = lambda a: synth.as_f64(a, w.dtype)  # noqa: E731
    t0 = time.perf_counter()
    qp = oracle.block_pool(f(x["q"]), w.N, w.block)
    kp = oracle.block_pool(f(x["k"]), w.N, w.kblock)
    vp = oracle.block_pool(f(x["v"]), w.N, w.kblock) if w.score != "prob" else None
    t_pool = time.perf_counter() - t0
    H, n = w.heads, w.n_blocks
    rows = sorted({(int(rng.integers(H)), int(rng.integers(n))) for _ in range(rows_max)})
    t0 = time.perf_counter()
    for h, i in rows:
        P = oracle.block_map(qp[h:h + 1, i:i + 1], kp[h:h + 1], 1.0 / math.sqrt(w.head_dim))
        if w.score == "prob":
            key = P
        else:
            key, vout, _ = oracle.drift_key(P, vp[h:h + 1], None)
        kept, _ = oracle.select_topk(key, x["keep"][h:h + 1], x["always"])
        if w.rounds > 0 and w.score != "prob":
            oracle.refine_dropset(P, vp[h:h + 1], vout, None, x["keep"][h:h + 1], x["always"],
                                  kept, w.rounds, w.rho)
    t_rows = time.perf_counter() - t0
    total = t_pool + t_rows * (H * n) / len(rows)
    return total, (f"pooling of all tokens ({t_pool:.1f} s) plus map, key, top-k"
                   f"{' and refinement' if w.rounds else ''} of {len(rows)} random rows "
                   f"({t_rows:.1f} s), scaled to all {H * n} rows")


def cpu_baseline(w, x, idx, cnt, extra=(), budget_s=12.0):
    """The oracle timed on the host: masked attention on a bounded sample of
    query blocks of w (the headline figure, TFLOP/s on kept FLOPs), the
    selection step scaled from a row sample, attention of the other
    workloads in `extra` [(w, x, idx, cnt)], and a one-thread run on the
    tiny and 8-view workloads."""
    from threadpoolctl import threadpool_limits
    threads = _oracle_threads()
    rate, blocks, spent = _oracle_attention_rate(w, x, idx, cnt, budget_s)
    sel_s, sel_what = _oracle_selection_rate(w, x)
    res = {"value": rate, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
           "sample": f"float64 numpy oracle, masked attention of {blocks} random query blocks "
                     f"(kept lists from the GPU selection) of {w.name}, {spent:.1f} s",
           "selection_s_full_workload": sel_s, "selection_sample": sel_what,
           "per_workload": {}}
    for w2, x2, i2, c2 in extra:
        r2, b2, s2 = _oracle_attention_rate(w2, x2, i2, c2, 4.0)
        entry = {"attention_tflops": r2, "blocks": b2, "seconds": s2}
        if w2.name in ("tiny", "views8"):
            with threadpool_limits(1):
                r1, b1, s1 = _oracle_attention_rate(w2, x2, i2, c2, 3.0)
                entry["attention_tflops_1_thread"] = r1
                entry["selection_s_1_thread"] = _oracle_selection_rate(w2, x2, rows_max=16)[0]
        res["per_workload"][w2.name] = entry
    return res


def residual_drift_report(w, x, shape, qkv, out, dense_out):
    """Realised residual drift (mean over heads and query blocks of the
    per-token ||o_sparse - o_dense||^2, M = I) of this workload's selection
    and of the probability and drift top-k selections at the same budgets;
    outside any timed region."""
    import torch

    import block_sparse_global_amd as bsg
    q, k, v = qkv
    dr = torch.empty((shape.H, shape.nq), dtype=torch.float64, device="cuda")
    res = {"measure": "mean over heads and query blocks of per-token ||o_sparse - o_dense||^2"}

    def one(o):
        bsg.ress_residual_drift(o, dense_out, shape, dr)
        torch.cuda.synchronize()
        return float(dr.mean().item())

    res["this_selection"] = one(out)
    for name, mode, rounds in (("prob_topk", "prob", 0), ("drift_topk", "drift", 0)):
        lay = bsg.BlockSparseGlobalAttention(shape, x["keep"], x["always"], mode=mode,
                                             rounds=rounds, rho=w.rho)
        o2 = torch.empty_like(q)
        lay(q, k, v, o2)
        res[name] = one(o2)
        del lay, o2
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="views100")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the 8/32-view layer-vs-dense lines")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the dense-attention timing (profiling runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="also run one device-to-device copy of BYTES bytes, whose "
                         "HBM counters calibrate FETCH_SIZE / WRITE_SIZE")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the "
              "multi-GPU head sharding of this path is a design note, not a run.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    peaks = measured_peaks()
    w, x, shape, layer, qkv, out = setup(args.workload)
    q, k, v = qkv
    step = lambda: layer(q, k, v, out)  # noqa: E731
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ms_step = time_events(step, args.steps)
    t_wall = (time.perf_counter() - t_wall) / args.steps * 1e3
    ms_step_median = time_median(step, max(20, args.steps))

    idx = layer.kept_idx.cpu().numpy()
    cnt = layer.kept_cnt.cpu().numpy()
    kf = kept_flops(w, idx, cnt)
    objective = None
    if layer.rounds > 0:
        J0, J1 = layer.J_init.cpu().numpy(), layer.J_final.cpu().numpy()
        objective = {"J_init_mean": float(J0.mean()), "J_final_mean": float(J1.mean()),
                     "J_final_over_J_init_mean": float(np.mean(J1 / J0)),
                     "rows": int(J0.size)}
    stages = stage_breakdown(layer, qkv, out, max(20, args.steps))
    refine_paths = refine_paths_ms(w, x, shape, layer, max(3, args.steps // 2))
    one_pass = one_pass_selection_ms(w, x, shape, layer, qkv, max(5, args.steps // 2))
    attn_reps = max(20, args.steps)
    attn_ms = time_events(lambda: layer.attend(q, k, v, out), attn_reps)
    attn_median = time_median(lambda: layer.attend(q, k, v, out), attn_reps)
    mem = scoring_memory(layer)

    import block_sparse_global_amd as bsg
    df = dense_flops(w)
    dense_ms = float("nan")
    drift_report = None
    if not args.no_dense:
        dense_out = torch.empty_like(q)
        dense_reps = max(2, min(args.steps, 5))
        dense_ms = time_events(lambda: bsg.dense_attention(q, k, v, shape, dense_out),
                               dense_reps)
        if not args.no_sweep:
            drift_report = residual_drift_report(w, x, shape, qkv, out, dense_out)
        del dense_out
    if args.copy_calibration > 0:
        nb = int(args.copy_calibration)
        src = torch.empty(nb, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    proj = None if args.no_sweep else projections(w)
    sel_paths = None if args.no_sweep else select_paths()
    sdpa = None if args.no_sweep else torch_sdpa()

    sweep = {}
    budgets = None
    cpu_extra = []
    if not args.no_sweep:
        # 8 / 32 / 100 views (the headline lines) and 200 views with both
        # scores; each line: layer time, dense time, the attention kernel alone
        lines = [("views8", None), ("views32", None), ("views100", None),
                 ("views100", "cdf"), ("views100", "hess"), ("views100-k64", None),
                 ("views200", "prob"), ("views200", "drift")]
        x200 = None
        for name, mode in lines:
            key = name if mode is None else f"{name}-{mode}"
            if name == args.workload and mode is None and not args.no_dense:
                sweep[key] = {"layer_ms": ms_step, "dense_ms": dense_ms, "attn_ms": attn_ms,
                              "select_ms": stages["select"],
                              "score_select_ms": stages["score"] + stages["select"],
                              "select_impl": layer.select_impl, "kept_flop": kf,
                              "realised_sparsity": sparsity_of(w, cnt)}
            else:
                if name == "views200" and x200 is None:
                    import synth
                    x200 = synth.make_inputs(synth.get_workload(name))
                # "cdf": probability score, cumulative threshold CDF_TAU with
                # the workload's budget as the cap. "hess": per-head budgets
                # from head scores (the HeSS allocation), same total budget
                x_in = x200 if name == "views200" else None
                if mode == "hess":
                    x_in = hess_inputs(name)
                w2, x2, shape2, layer2, (q2, k2, v2), out2 = setup(
                    name, "prob" if mode == "cdf" else (None if mode == "hess" else mode),
                    x_in, tau=CDF_TAU if mode == "cdf" else None)
                for _ in range(3):
                    layer2(q2, k2, v2, out2)
                reps = 5 if name == "views200" else 20
                l_ms = time_median(lambda: layer2(q2, k2, v2, out2), reps)
                a_ms = time_median(lambda: layer2.attend(q2, k2, v2, out2), reps)
                s_ms = time_median(lambda: layer2.select(), reps)
                ss_ms = time_median(lambda: (layer2.score(), layer2.select()), reps)
                idx2 = layer2.kept_idx.cpu().numpy()
                cnt2 = layer2.kept_cnt.cpu().numpy()
                kf2 = kept_flops(w2, idx2, cnt2)
                if mode is None and name in ("views8", "views32"):
                    cpu_extra.append((w2, x2, idx2, cnt2))
                d2 = torch.empty_like(q2)
                d_ms = time_median(lambda: bsg.dense_attention(q2, k2, v2, shape2, d2),
                                   2 if name == "views200" else 5)
                sweep[key] = {"layer_ms": l_ms, "dense_ms": d_ms, "attn_ms": a_ms,
                              "select_ms": s_ms, "score_select_ms": ss_ms,
                              "select_impl": layer2.select_impl, "kept_flop": kf2,
                              "realised_sparsity": sparsity_of(w2, cnt2)}
                if mode == "hess":
                    sweep[key]["keep_per_head"] = [int(b) for b in x2["keep"]]
                del layer2, q2, k2, v2, out2, d2
                torch.cuda.empty_cache()
            e = sweep[key]
            e["speedup_vs_dense"] = e["dense_ms"] / e["layer_ms"]
            e["attn_tflops"] = e["kept_flop"] / (e["attn_ms"] * 1e-3) / 1e12
        x200 = None
        budgets = {"views8": budget_sweep("views8", (4, 8, 16, 32, 43, 64)),
                   "views100": budget_sweep("views100", (8, 16, 32, 64, 107, 215),
                                            x if args.workload == "views100" else None)}
        # the tiny workload (float32 inputs) for the oracle's one-thread line
        wt, xt, _, lt, qkvt, outt = setup("tiny")
        lt(*qkvt, outt)
        cpu_extra.insert(0, (wt, xt, lt.kept_idx.cpu().numpy(), lt.kept_cnt.cpu().numpy()))

    achieved = kf / (attn_ms * 1e-3) / 1e12
    res = {
        "metric": METRIC,
        "value": kf / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "views": w.views, "tokens": w.N, "padded_tokens": w.N_pad,
            "heads": w.heads, "head_dim": w.head_dim, "block": w.block, "key_block": w.kblock,
            "sparsity": list(w.sparsity), "score": layer.mode, "refine_rounds": layer.rounds,
            "seed": w.seed,
        },
        "roofline": {
            "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
            "traffic": attn_traffic(w.name), "traffic_unit": "bytes per launch (HBM, counters)",
            "kernel": "attn_kernel<128, 128> (ress_sparse_attn_fwd)",
            "flop_per_launch": kf, "avg_launch_ms": attn_ms, "median_launch_ms": attn_median,
            "launches_timed": attn_reps,
            "measured_peak": peaks["mfma_bf16_tflops"],
            "frac_of_measured_peak": achieved / peaks["mfma_bf16_tflops"],
        },
        "measured_peaks": peaks,
        "layer_ms": ms_step,
        "layer_ms_median": ms_step_median,
        "layer_ms_wall": t_wall,
        "dense_ms": None if args.no_dense else dense_ms,
        "dense_tflops": None if args.no_dense else df / (dense_ms * 1e-3) / 1e12,
        "speedup_vs_dense": None if args.no_dense else dense_ms / ms_step,
        "sparse_vs_dense_per_flop": None if args.no_dense else (kf / attn_ms) / (df / dense_ms),
        "attn_tflops": achieved,
        "kept_flop": kf,
        "realised_sparsity": sparsity_of(w, cnt),
        "stages_ms": stages,
        "selection_ms": sum(stages[n] for n in ("pool", "score", "select", "refine")),
        "refine_objective": objective,
        "scoring_memory": mem,
        "refine_paths_ms": refine_paths,
        "one_pass_selection_ms": one_pass,
        "projections": proj,
        "select_paths_ms": sel_paths,
        "budget_sweep": budgets,
        "torch_sdpa": sdpa,
        "views_sweep": sweep,
        "residual_drift": drift_report,
        "pages_context": PAGES_CONTEXT,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, x, idx, cnt, extra=cpu_extra)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
