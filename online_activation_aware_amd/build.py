"""Build libttq.so (HIP, gfx950 only) in-tree.

    python -m online_activation_aware_amd.build [source.hip ...]

Compiles every HIP source under csrc/ with hipcc for gfx950 and links them
into online_activation_aware_amd/libttq.so.  Objects go to _build/.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libttq.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["stats.hip", "quantize.hip", "quantize_lr.hip", "qgemm.hip", "qgemv.hip", "qgemv_gs.hip", "gemm_bf16.hip", "lowrank.hip", "factors.hip",
           "noalloc.hip", "ttq_api.cpp"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # IEEE behaviour: no contraction unless written as an explicit fma,
    # correctly rounded fp32 division/sqrt (hipcc's default), no fast-math.
    "-ffp-contract=off",
    # Keep the compiler from forming packed-fp32 (v_pk_*_f32) instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libttq)")


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + FLAGS + extra
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    noise = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(extra: list[str] | None = None, verbose: bool = True, only: list[str] | None = None) -> str:
    """Compile all sources (or only the named ones, reusing the other objects
    from an earlier build) and link libttq.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    extra = list(extra or [])
    todo = SOURCES if not only else [s for s in SOURCES if s in only]
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        list(ex.map(lambda s: _compile(s, extra), todo))
    objs = [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    # python -m online_activation_aware_amd.build [source.hip ...]: rebuild
    # only the named sources (others from _build/), then link.
    build(only=sys.argv[1:] or None)
