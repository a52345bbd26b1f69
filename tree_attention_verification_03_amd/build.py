"""Build libspectree.so (HIP, gfx950) in-tree with hipcc.

Usage: ``python -m tree_attention_verification_03_amd.build`` (or ``build()``).
Objects go to ``_build/`` at the repository root; the shared library lands
next to this file so the Python binding (and a copy of the tree shipped to a
GPU host) finds it without installation.
"""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libspectree.so")

ARCH = os.environ.get("SPEC_TREE_ARCH", "gfx950")
COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    f"--offload-arch={ARCH}",
    # keep the compiler from forming packed fp32 ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# translation units whose integer / fp64 results must be bit-exact: no FMA contraction
EXACT = {"tree_build.hip", "tree_verify.hip"}
SOURCES = ["api.cpp", "tree_build.hip", "tree_attention.hip", "tree_verify.hip", "kv_compact.hip"]


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libspectree)")


def _compile(src: str) -> str:
    hipcc = _hipcc()
    obj = os.path.join(OBJ, src + ".o")
    flags = list(COMMON)
    if src in EXACT:
        flags.append("-ffp-contract=off")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [hipcc, *lang, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _check_no_spills(src: str):
    """The attention kernel's pipelined loop counts its own outstanding loads (s_waitcnt vmcnt(n)), so
    scratch (spill) traffic would break its waits; the tree-build kernels are sized to stay resident
    (registers for several blocks per CU). A spilling build of either is rejected."""
    cmd = [_hipcc(), "-x", "hip", *COMMON, "--offload-device-only", "-c", os.path.join(CSRC, src), "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    sizes = re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", r.stderr)
    if r.returncode != 0 or not sizes or any(int(x) for x in sizes):
        raise RuntimeError(f"{src}: kernels must not spill to scratch (per-kernel scratch bytes/lane: {sizes})\n"
                           + r.stderr[-2000:])


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ, exist_ok=True)
    for src in ("tree_attention.hip", "tree_build.hip"):
        _check_no_spills(src)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
