"""ctypes binding of libress: the C ABI of include/ress.h, one Python function
per entry point with the same name.

This layer only marshals arguments: it checks device, dtype, contiguity and
shape of torch tensors, passes their device pointers and the current HIP
stream, and raises RessError on a negative status. Every step of the
computation runs in the library's HIP kernels. There is no fallback: if the
library is missing, importing this module raises.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libress.so")

RESS_OK = 0
RESS_ERR_INVALID_ARG = -1
RESS_ERR_UNSUPPORTED = -2
RESS_ERR_HIP = -3

RESS_DTYPE_BF16 = 0
RESS_DTYPE_F32 = 1
RESS_SCORE_PROB = 0
RESS_SCORE_DRIFT = 1
RESS_MAX_BLOCKS = 4096

ENTRY_POINTS = (
    "ress_block_pool",
    "ress_block_score",
    "ress_select_topk",
    "ress_select_cdf",
    "ress_select_fused",
    "ress_select_refine_fused",
    "ress_refine_dropset",
    "ress_refine_dropset_fused",
    "ress_refine_dropset_noalloc",
    "ress_refine_workspace_size",
    "ress_gram_from_wo",
    "ress_head_budgets",
    "ress_residual_drift",
    "ress_qkv_project",
    "ress_out_project",
    "ress_sparse_attn_fwd",
    "ress_last_error",
    "ress_version",
)


class RessError(RuntimeError):
    def __init__(self, func: str, code: int, msg: str):
        super().__init__(f"{func} failed with status {code}: {msg}")
        self.code = code


class ress_shape(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("N_pad", ctypes.c_int32), ("D", ctypes.c_int32),
                ("B", ctypes.c_int32), ("Bk", ctypes.c_int32)]


@dataclass(frozen=True)
class Shape:
    """Query blocks of B tokens, key blocks of Bk tokens (0: Bk = B)."""
    H: int
    N: int
    N_pad: int
    D: int
    B: int
    Bk: int = 0

    @property
    def kb(self) -> int:
        return self.Bk if self.Bk > 0 else self.B

    @property
    def n(self) -> int:
        """Query blocks (rows of the block maps)."""
        return self.N_pad // self.B

    @property
    def nq(self) -> int:
        return self.n

    @property
    def nk(self) -> int:
        """Key blocks (columns of the block maps)."""
        return -(-self.N // self.kb)

    def c(self) -> ress_shape:
        return ress_shape(self.H, self.N, self.N_pad, self.D, self.B, self.Bk)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libress is not built ({LIB_PATH} missing); run "
            "`python block_sparse_global_amd/build.py` first")
    lib = ctypes.CDLL(LIB_PATH)
    vp, dp, ip = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.ress_block_pool.argtypes = [vp, vp, vp, ctypes.c_int, ress_shape, dp, dp, dp, vp]
    lib.ress_block_score.argtypes = [dp, dp, dp, dp, ress_shape, ctypes.c_int,
                                     ctypes.c_double, ctypes.c_double, dp, dp, dp, dp, vp]
    lib.ress_select_topk.argtypes = [dp, ress_shape, ip, vp, i32, ip, ip, vp]
    lib.ress_select_cdf.argtypes = [dp, ress_shape, ip, vp, ctypes.c_double, i32, ip, ip, vp]
    lib.ress_select_fused.argtypes = [dp, dp, dp, dp, ress_shape, ctypes.c_int, ctypes.c_double,
                                      ctypes.c_double, ip, vp, i32, dp, ip, ip, vp]
    lib.ress_select_refine_fused.argtypes = [dp, dp, dp, dp, ress_shape, ctypes.c_double,
                                             ctypes.c_double, ip, vp, i32, ctypes.c_double, i32,
                                             dp, ip, ip, dp, dp, vp]
    lib.ress_refine_dropset.argtypes = [dp, dp, dp, dp, dp, ress_shape, ip, vp, i32,
                                        ctypes.c_double, ctypes.c_double, i32, ip, ip,
                                        dp, dp, vp, ctypes.c_size_t, vp]
    lib.ress_refine_dropset_fused.argtypes = [dp, dp, dp, dp, dp, ress_shape, ip, vp, i32,
                                              ctypes.c_double, ctypes.c_double, i32, ip, ip,
                                              dp, dp, vp]
    lib.ress_refine_dropset_noalloc.argtypes = [dp, dp, dp, dp, dp, ress_shape, ip, vp, i32,
                                                ctypes.c_double, ctypes.c_double, i32, ip, ip,
                                                dp, dp, vp]
    lib.ress_refine_workspace_size.argtypes = [ress_shape]
    lib.ress_refine_workspace_size.restype = ctypes.c_size_t
    lib.ress_sparse_attn_fwd.argtypes = [vp, vp, vp, ctypes.c_int, ress_shape, ip, ip, i32,
                                         ctypes.c_float, vp, vp, vp]
    lib.ress_gram_from_wo.argtypes = [vp, ctypes.c_int, i32, ress_shape, dp, vp]
    lib.ress_head_budgets.argtypes = [vp, i32, i32, vp, ctypes.c_int64, vp]
    lib.ress_residual_drift.argtypes = [vp, vp, ctypes.c_int, dp, ress_shape, dp, vp]
    lib.ress_qkv_project.argtypes = [vp, vp, vp, ctypes.c_int, i32, ress_shape, vp, vp, vp, vp]
    lib.ress_out_project.argtypes = [vp, vp, vp, vp, ctypes.c_int, i32, ress_shape, vp, vp]
    for f in ("ress_block_pool", "ress_block_score", "ress_select_topk",
              "ress_select_cdf", "ress_select_fused", "ress_select_refine_fused",
              "ress_refine_dropset", "ress_refine_dropset_fused",
              "ress_refine_dropset_noalloc", "ress_sparse_attn_fwd",
              "ress_gram_from_wo", "ress_head_budgets", "ress_residual_drift",
              "ress_qkv_project", "ress_out_project"):
        getattr(lib, f).restype = ctypes.c_int
    lib.ress_last_error.restype = ctypes.c_char_p
    lib.ress_last_error.argtypes = []
    lib.ress_version.restype = ctypes.c_int
    lib.ress_version.argtypes = []
    return lib


LIB = _load()


def _check(func: str, rc: int):
    if rc != RESS_OK:
        msg = LIB.ress_last_error().decode(errors="replace")
        raise RessError(func, rc, msg)


def _stream(stream) -> Optional[int]:
    if stream is None:
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, shape=None):
    """Device pointer of a contiguous tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor or None")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return RESS_DTYPE_BF16
    if t.dtype == torch.float32:
        return RESS_DTYPE_F32
    raise ValueError(f"unsupported token dtype {t.dtype}")


def _host_i32(a, name):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(a.cpu() if isinstance(a, torch.Tensor) else a,
                                          dtype=np.int32))
    return arr, arr.ctypes.data_as(ctypes.c_void_p)


def _host_u8(a, name):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(a.cpu() if isinstance(a, torch.Tensor) else a,
                                          dtype=np.uint8))
    return arr, arr.ctypes.data_as(ctypes.c_void_p)


def ress_version() -> int:
    return LIB.ress_version()


def ress_last_error() -> str:
    return LIB.ress_last_error().decode(errors="replace")


def ress_block_pool(q, k, v, shape: Shape, qpool, kpool, vpool, stream=None):
    ref = next(t for t in (q, k, v) if t is not None)
    dt = _dtype_code(ref)
    tok = (shape.H, shape.N_pad, shape.D)
    qblk = (shape.H, shape.nq, shape.D)
    kblk = (shape.H, shape.nk, shape.D)
    _check("ress_block_pool", LIB.ress_block_pool(
        _ptr(q, "q", ref.dtype, tok), _ptr(k, "k", ref.dtype, tok), _ptr(v, "v", ref.dtype, tok),
        dt, shape.c(),
        _ptr(qpool, "qpool", torch.float64, qblk), _ptr(kpool, "kpool", torch.float64, kblk),
        _ptr(vpool, "vpool", torch.float64, kblk), _stream(stream)))


def ress_block_score(qpool, kpool, vpool, M, shape: Shape, mode: int, scale: float,
                     eps: float, P, key, vout, vmv, stream=None):
    H, nq, nk, D = shape.H, shape.nq, shape.nk, shape.D
    f64 = torch.float64
    _check("ress_block_score", LIB.ress_block_score(
        _ptr(qpool, "qpool", f64, (H, nq, D)), _ptr(kpool, "kpool", f64, (H, nk, D)),
        _ptr(vpool, "vpool", f64, (H, nk, D)), _ptr(M, "M", f64, (H, D, D)),
        shape.c(), int(mode), float(scale), float(eps),
        _ptr(P, "P", f64, (H, nq, nk)), _ptr(key, "key", f64, (H, nq, nk)),
        _ptr(vout, "vout", f64, (H, nq, D)), _ptr(vmv, "vmv", f64, (H, nk)),
        _stream(stream)))


def ress_select_topk(key, shape: Shape, keep: Sequence[int], always_keep, k_max: int,
                     kept_idx, kept_cnt, stream=None):
    H, nq, nk = shape.H, shape.nq, shape.nk
    keep_arr, keep_p = _host_i32(keep, "keep")
    if keep_arr is not None and keep_arr.shape != (H,):
        raise ValueError(f"keep must have shape ({H},)")
    alw_arr, alw_p = _host_u8(always_keep, "always_keep")
    if alw_arr is not None and alw_arr.shape != (nk,):
        raise ValueError(f"always_keep must have shape ({nk},)")
    _check("ress_select_topk", LIB.ress_select_topk(
        _ptr(key, "key", torch.float64, (H, nq, nk)), shape.c(), keep_p, alw_p,
        int(k_max), _ptr(kept_idx, "kept_idx", torch.int32, (H, nq, k_max)),
        _ptr(kept_cnt, "kept_cnt", torch.int32, (H, nq)), _stream(stream)))


def ress_select_cdf(P, shape: Shape, keep: Sequence[int], always_keep, tau: float,
                    k_max: int, kept_idx, kept_cnt, stream=None):
    H, nq, nk = shape.H, shape.nq, shape.nk
    keep_arr, keep_p = _host_i32(keep, "keep")
    if keep_arr is not None and keep_arr.shape != (H,):
        raise ValueError(f"keep must have shape ({H},)")
    alw_arr, alw_p = _host_u8(always_keep, "always_keep")
    if alw_arr is not None and alw_arr.shape != (nk,):
        raise ValueError(f"always_keep must have shape ({nk},)")
    _check("ress_select_cdf", LIB.ress_select_cdf(
        _ptr(P, "P", torch.float64, (H, nq, nk)), shape.c(), keep_p, alw_p, float(tau),
        int(k_max), _ptr(kept_idx, "kept_idx", torch.int32, (H, nq, k_max)),
        _ptr(kept_cnt, "kept_cnt", torch.int32, (H, nq)), _stream(stream)))


# key blocks per row up to which ress_select_fused applies
SELECT_FUSED_MAX_BLOCKS = 2176


def ress_select_fused(qpool, kpool, vpool, M, shape: Shape, mode: int, scale: float, eps: float,
                      keep, always_keep, k_max: int, vmv, kept_idx, kept_cnt, stream=None):
    """Score and top-k in one pass per row tile, the map and key on chip;
    vmv [H][n_k] (drift) is written with V_j^T M V_j."""
    H, nq, nk, D = shape.H, shape.nq, shape.nk, shape.D
    f64 = torch.float64
    keep_arr, keep_p = _host_i32(keep, "keep")
    if keep_arr is not None and keep_arr.shape != (H,):
        raise ValueError(f"keep must have shape ({H},)")
    alw_arr, alw_p = _host_u8(always_keep, "always_keep")
    if alw_arr is not None and alw_arr.shape != (nk,):
        raise ValueError(f"always_keep must have shape ({nk},)")
    _check("ress_select_fused", LIB.ress_select_fused(
        _ptr(qpool, "qpool", f64, (H, nq, D)), _ptr(kpool, "kpool", f64, (H, nk, D)),
        _ptr(vpool, "vpool", f64, (H, nk, D)), _ptr(M, "M", f64, (H, D, D)), shape.c(),
        int(mode), float(scale), float(eps), keep_p, alw_p, int(k_max),
        _ptr(vmv, "vmv", f64, (H, nk)),
        _ptr(kept_idx, "kept_idx", torch.int32, (H, nq, k_max)),
        _ptr(kept_cnt, "kept_cnt", torch.int32, (H, nq)), _stream(stream)))


# key blocks per row up to which ress_select_refine_fused applies
SELECT_REFINE_FUSED_MAX_BLOCKS = 1088


def ress_select_refine_fused(qpool, kpool, vpool, M, shape: Shape, scale: float, eps: float,
                             keep, always_keep, rounds: int, rho: float, k_max: int, vmv,
                             kept_idx, kept_cnt, J_init=None, J_final=None, stream=None):
    """Drift scoring, top-k and the refinement in one pass per tile of rows,
    the map and key on chip (rows of at most SELECT_REFINE_FUSED_MAX_BLOCKS
    key blocks); vmv [H][n_k] is written with V_j^T M V_j."""
    H, nq, nk, D = shape.H, shape.nq, shape.nk, shape.D
    f64 = torch.float64
    keep_arr, keep_p = _host_i32(keep, "keep")
    if keep_arr is not None and keep_arr.shape != (H,):
        raise ValueError(f"keep must have shape ({H},)")
    alw_arr, alw_p = _host_u8(always_keep, "always_keep")
    if alw_arr is not None and alw_arr.shape != (nk,):
        raise ValueError(f"always_keep must have shape ({nk},)")
    _check("ress_select_refine_fused", LIB.ress_select_refine_fused(
        _ptr(qpool, "qpool", f64, (H, nq, D)), _ptr(kpool, "kpool", f64, (H, nk, D)),
        _ptr(vpool, "vpool", f64, (H, nk, D)), _ptr(M, "M", f64, (H, D, D)), shape.c(),
        float(scale), float(eps), keep_p, alw_p, int(rounds), float(rho), int(k_max),
        _ptr(vmv, "vmv", f64, (H, nk)),
        _ptr(kept_idx, "kept_idx", torch.int32, (H, nq, k_max)),
        _ptr(kept_cnt, "kept_cnt", torch.int32, (H, nq)),
        _ptr(J_init, "J_init", f64, (H, nq)), _ptr(J_final, "J_final", f64, (H, nq)),
        _stream(stream)))


def ress_refine_workspace_size(shape: Shape) -> int:
    nb = LIB.ress_refine_workspace_size(shape.c())
    if nb == 0:
        raise RessError("ress_refine_workspace_size", RESS_ERR_INVALID_ARG,
                        LIB.ress_last_error().decode(errors="replace"))
    return int(nb)


def ress_refine_dropset(P, key, vpool, vout, M, shape: Shape, keep, always_keep,
                        rounds: int, rho: float, eps: float, k_max: int, kept_idx,
                        kept_cnt, J_init=None, J_final=None, workspace=None, stream=None):
    """workspace: a device uint8 tensor of at least ress_refine_workspace_size
    bytes (allocated here when None)."""
    H, nq, nk, D = shape.H, shape.nq, shape.nk, shape.D
    if workspace is None:
        workspace = torch.empty(ress_refine_workspace_size(shape), dtype=torch.uint8,
                                device=kept_idx.device if isinstance(kept_idx, torch.Tensor)
                                else "cuda")
    ws_ptr = _ptr(workspace, "workspace", torch.uint8)
    f64 = torch.float64
    keep_arr, keep_p = _host_i32(keep, "keep")
    if keep_arr is not None and keep_arr.shape != (H,):
        raise ValueError(f"keep must have shape ({H},)")
    alw_arr, alw_p = _host_u8(always_keep, "always_keep")
    if alw_arr is not None and alw_arr.shape != (nk,):
        raise ValueError(f"always_keep must have shape ({nk},)")
    _check("ress_refine_dropset", LIB.ress_refine_dropset(
        _ptr(P, "P", f64, (H, nq, nk)), _ptr(key, "key", f64, (H, nq, nk)),
        _ptr(vpool, "vpool", f64, (H, nk, D)), _ptr(vout, "vout", f64, (H, nq, D)),
        _ptr(M, "M", f64, (H, D, D)), shape.c(), keep_p, alw_p, int(rounds), float(rho),
        float(eps), int(k_max), _ptr(kept_idx, "kept_idx", torch.int32, (H, nq, k_max)),
        _ptr(kept_cnt, "kept_cnt", torch.int32, (H, nq)),
        _ptr(J_init, "J_init", f64, (H, nq)), _ptr(J_final, "J_final", f64, (H, nq)),
        ws_ptr, workspace.numel(), _stream(stream)))


# key blocks per row up to which ress_refine_dropset_fused applies
REFINE_FUSED_MAX_BLOCKS = 1088


def ress_refine_dropset_fused(P, key, vpool, vout, M, shape: Shape, keep, always_keep,
                              rounds: int, rho: float, eps: float, k_max: int, kept_idx,
                              kept_cnt, J_init=None, J_final=None, stream=None):
    """ress_refine_dropset in one kernel per tile of rows, no workspace
    (rows of at most REFINE_FUSED_MAX_BLOCKS key blocks)."""
    H, nq, nk, D = shape.H, shape.nq, shape.nk, shape.D
    f64 = torch.float64
    keep_arr, keep_p = _host_i32(keep, "keep")
    if keep_arr is not None and keep_arr.shape != (H,):
        raise ValueError(f"keep must have shape ({H},)")
    alw_arr, alw_p = _host_u8(always_keep, "always_keep")
    if alw_arr is not None and alw_arr.shape != (nk,):
        raise ValueError(f"always_keep must have shape ({nk},)")
    _check("ress_refine_dropset_fused", LIB.ress_refine_dropset_fused(
        _ptr(P, "P", f64, (H, nq, nk)), _ptr(key, "key", f64, (H, nq, nk)),
        _ptr(vpool, "vpool", f64, (H, nk, D)), _ptr(vout, "vout", f64, (H, nq, D)),
        _ptr(M, "M", f64, (H, D, D)), shape.c(), keep_p, alw_p, int(rounds), float(rho),
        float(eps), int(k_max), _ptr(kept_idx, "kept_idx", torch.int32, (H, nq, k_max)),
        _ptr(kept_cnt, "kept_cnt", torch.int32, (H, nq)),
        _ptr(J_init, "J_init", f64, (H, nq)), _ptr(J_final, "J_final", f64, (H, nq)),
        _stream(stream)))


RESS_NOALLOC_SCRATCH_BYTES = 64 << 20


def ress_refine_dropset_noalloc(P, key, vpool, vout, M, shape: Shape, keep, always_keep,
                                rounds: int, rho: float, eps: float, k_max: int, kept_idx,
                                kept_cnt, J_init=None, J_final=None, stream=None):
    """ress_refine_dropset with its state in the library's fixed per-GPU
    scratch (no workspace, no allocation); calls on one GPU must not overlap."""
    H, nq, nk, D = shape.H, shape.nq, shape.nk, shape.D
    f64 = torch.float64
    keep_arr, keep_p = _host_i32(keep, "keep")
    if keep_arr is not None and keep_arr.shape != (H,):
        raise ValueError(f"keep must have shape ({H},)")
    alw_arr, alw_p = _host_u8(always_keep, "always_keep")
    if alw_arr is not None and alw_arr.shape != (nk,):
        raise ValueError(f"always_keep must have shape ({nk},)")
    _check("ress_refine_dropset_noalloc", LIB.ress_refine_dropset_noalloc(
        _ptr(P, "P", f64, (H, nq, nk)), _ptr(key, "key", f64, (H, nq, nk)),
        _ptr(vpool, "vpool", f64, (H, nk, D)), _ptr(vout, "vout", f64, (H, nq, D)),
        _ptr(M, "M", f64, (H, D, D)), shape.c(), keep_p, alw_p, int(rounds), float(rho),
        float(eps), int(k_max), _ptr(kept_idx, "kept_idx", torch.int32, (H, nq, k_max)),
        _ptr(kept_cnt, "kept_cnt", torch.int32, (H, nq)),
        _ptr(J_init, "J_init", f64, (H, nq)), _ptr(J_final, "J_final", f64, (H, nq)),
        _stream(stream)))


def ress_head_budgets(score, n_k: int, always_keep, total_keep: int) -> np.ndarray:
    """Per-head keep budgets from head scores (host only); returns int32 [H]."""
    sc = np.ascontiguousarray(np.asarray(score, dtype=np.float64))
    alw_arr, alw_p = _host_u8(always_keep, "always_keep")
    if alw_arr is not None and alw_arr.shape != (int(n_k),):
        raise ValueError(f"always_keep must have shape ({n_k},)")
    out = np.empty(sc.shape[0], dtype=np.int32)
    _check("ress_head_budgets", LIB.ress_head_budgets(
        sc.ctypes.data_as(ctypes.c_void_p), int(sc.shape[0]), int(n_k), alw_p,
        int(total_keep), out.ctypes.data_as(ctypes.c_void_p)))
    return out


def ress_residual_drift(out_sparse, out_dense, shape: Shape, drift, M=None, stream=None):
    """drift[h][i] = mean over block i's valid tokens of e^T M_h e,
    e = out_sparse - out_dense (||e||^2 when M is None)."""
    tok = (shape.H, shape.N_pad, shape.D)
    _check("ress_residual_drift", LIB.ress_residual_drift(
        _ptr(out_sparse, "out_sparse", out_sparse.dtype, tok),
        _ptr(out_dense, "out_dense", out_sparse.dtype, tok), _dtype_code(out_sparse),
        _ptr(M, "M", torch.float64, (shape.H, shape.D, shape.D)), shape.c(),
        _ptr(drift, "drift", torch.float64, (shape.H, shape.nq)), _stream(stream)))


def ress_gram_from_wo(w_o, shape: Shape, M, stream=None):
    """M[h] = W_O^h^T W_O^h for w_o of shape [d_model][H*D] (bf16 or float32)."""
    if w_o.dim() != 2 or w_o.shape[1] != shape.H * shape.D:
        raise ValueError(f"w_o must have shape [d_model][{shape.H * shape.D}]")
    _check("ress_gram_from_wo", LIB.ress_gram_from_wo(
        _ptr(w_o, "w_o", w_o.dtype, tuple(w_o.shape)), _dtype_code(w_o), int(w_o.shape[0]),
        shape.c(), _ptr(M, "M", torch.float64, (shape.H, shape.D, shape.D)), _stream(stream)))


def ress_sparse_attn_fwd(q, k, v, shape: Shape, kept_idx, kept_cnt, k_max: int,
                         scale: float, out, lse=None, stream=None):
    dt = _dtype_code(q)
    tok = (shape.H, shape.N_pad, shape.D)
    H, nq = shape.H, shape.nq
    _check("ress_sparse_attn_fwd", LIB.ress_sparse_attn_fwd(
        _ptr(q, "q", q.dtype, tok), _ptr(k, "k", q.dtype, tok), _ptr(v, "v", q.dtype, tok),
        dt, shape.c(),
        _ptr(kept_idx, "kept_idx", torch.int32, (H, nq, k_max)) if kept_idx is not None else None,
        _ptr(kept_cnt, "kept_cnt", torch.int32, (H, nq)) if kept_cnt is not None else None,
        int(k_max), float(scale), _ptr(out, "out", q.dtype, tok),
        _ptr(lse, "lse", torch.float32, (H, shape.N_pad)), _stream(stream)))


def ress_qkv_project(x, w_qkv, b_qkv, shape: Shape, q, k, v, stream=None):
    """q, k, v [H][N_pad][D] from x [N_pad][d_model] and a linear layer's weight
    w_qkv [3 H D][d_model] (optional bias [3 H D]); bf16 tensors."""
    if x.dim() != 2 or x.shape[0] != shape.N_pad:
        raise ValueError(f"x must have shape [N_pad={shape.N_pad}][d_model]")
    d_model = int(x.shape[1])
    HD = shape.H * shape.D
    tok = (shape.H, shape.N_pad, shape.D)
    bf = torch.bfloat16
    _check("ress_qkv_project", LIB.ress_qkv_project(
        _ptr(x, "x", bf), _ptr(w_qkv, "w_qkv", bf, (3 * HD, d_model)),
        _ptr(b_qkv, "b_qkv", bf, (3 * HD,)), _dtype_code(x), d_model, shape.c(),
        _ptr(q, "q", bf, tok), _ptr(k, "k", bf, tok), _ptr(v, "v", bf, tok), _stream(stream)))


def ress_out_project(o, w_o, b_o, residual, shape: Shape, y, stream=None):
    """y [N_pad][d_model] = residual + b_o + o W_O^T, with o [H][N_pad][D] read as
    [N_pad][H D] and W_O [d_model][H D]; y may be the residual tensor itself."""
    if w_o.dim() != 2 or w_o.shape[1] != shape.H * shape.D:
        raise ValueError(f"w_o must have shape [d_model][{shape.H * shape.D}]")
    d_model = int(w_o.shape[0])
    bf = torch.bfloat16
    _check("ress_out_project", LIB.ress_out_project(
        _ptr(o, "o", bf, (shape.H, shape.N_pad, shape.D)), _ptr(w_o, "w_o", bf),
        _ptr(b_o, "b_o", bf, (d_model,)),
        _ptr(residual, "residual", bf, (shape.N_pad, d_model)), _dtype_code(o), d_model,
        shape.c(), _ptr(y, "y", bf, (shape.N_pad, d_model)), _stream(stream)))
