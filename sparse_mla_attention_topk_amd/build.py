"""Build the HIP library ``libsmla.so`` in-tree for gfx950 with hipcc.

``python -m sparse_mla_attention_topk_amd.build`` (or ``build_library()``) compiles every source
under ``csrc/`` and links the shared library next to this file.  It always recompiles.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libsmla.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["api.cpp", "topk.hip", "attention.hip", "cache_write.hip", "indexer.hip"]
ARCH = os.environ.get("SMLA_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def common_flags() -> list:
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        # keep packed-fp32 instructions out of the generated code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA accumulators in arch VGPRs: the rare online-softmax rescale then multiplies them in
        # place, and Q (the other MFMA operand) stays in AGPRs
        "-mllvm", "--amdgpu-mfma-vgpr-form",
        "-I", INCLUDE, "-I", CSRC,
        "-Wall", "-Wno-unused-result", "-Wno-inline-asm",
    ]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip() and verbose:
        print(out, flush=True)
    return obj


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}", flush=True)
    return LIB_PATH


if __name__ == "__main__":
    build_library(verbose="-v" in sys.argv)
