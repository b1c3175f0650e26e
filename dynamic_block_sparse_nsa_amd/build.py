"""Build ``libnsa.so`` (the C-ABI library, HIP for gfx950) in-tree.

``python -m dynamic_block_sparse_nsa_amd.build`` compiles every source under ``csrc/``
with hipcc in parallel into ``_build/`` and links ``libnsa.so`` next to this file, then
builds ``libnsa_ceilings.so`` (the roofline microbenchmarks of ``ceilings/``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libnsa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

ARCH = "gfx950"
FLAGS = [
    "-O3", f"--offload-arch={ARCH}", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-result",
    # no packed-fp32 VALU instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


CEIL_SRC = os.path.join(HERE, "ceilings", "ceilings.hip")
CEIL_LIB = os.path.join(HERE, "libnsa_ceilings.so")


def build_ceilings(verbose: bool = False) -> str:
    """libnsa_ceilings.so: the roofline microbenchmarks (include/nsa_ceilings.h)."""
    tmp = CEIL_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-shared", CEIL_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {CEIL_SRC}:\n{r.stderr[-4000:]}")
    os.replace(tmp, CEIL_LIB)
    if verbose:
        print(f"built {CEIL_LIB}")
    return CEIL_LIB


if __name__ == "__main__":
    build(verbose=True)
    build_ceilings(verbose=True)
    sys.exit(0)
