"""Builds libress.so in-tree with hipcc for gfx950.

    python block_sparse_global_amd/build.py

Every HIP source under csrc/ is compiled and linked into one shared library
next to this file. Packed float32 VALU instructions are disabled for the
device code (-packed-fp32-ops); the host pass prints a harmless warning that
it does not know that feature.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libress.so")
ROOT = os.path.dirname(HERE)

SOURCES = ["api.hip", "pool.hip", "score.hip", "select.hip", "refine.hip", "refine_fused.hip",
           "attn.hip", "attn_f32.hip", "gram.hip", "drift.hip", "noalloc.hip", "proj.hip", "select_fused.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def command(out: str = LIB):
    return [
        hipcc(),
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-Wall",
        "-Wno-unused-function",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
        "-o", out,
    ] + [os.path.join(CSRC, s) for s in SOURCES]


PROBE_LIB = os.path.join(HERE, "libress_probe.so")
PROBE_SOURCES = [os.path.join("probe", "peak.hip")]


def probe_command(out: str = PROBE_LIB):
    """The benchmark's peak probe (libress_probe.so): not part of libress."""
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", out] + \
        [os.path.join(CSRC, s) for s in PROBE_SOURCES]


def build(verbose: bool = False) -> str:
    """Compiles the library (always) and returns its path."""
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(
        ln for ln in (res.stderr or "").splitlines()
        if "packed-fp32-ops" not in ln
    )
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{errs}")
    if verbose and errs.strip():
        print(errs, file=sys.stderr)
    os.replace(tmp, LIB)
    res = subprocess.run(probe_command(PROBE_LIB + ".tmp"), capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on the probe ({res.returncode}):\n{res.stderr}")
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
