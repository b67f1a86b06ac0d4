"""Build libdeltarule.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

Run as ``python -m delta_rule_linear_chunked_amd._build``; ``build()`` always
recompiles every source. Objects go to ``_build/`` at the repository root and
the shared library to ``delta_rule_linear_chunked_amd/lib/``.
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
OBJDIR = os.path.join(ROOT, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libdeltarule.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "plan.cpp", "scratch.hip", "decode.hip", "prefill.hip", "prefill_state.hip", "backward.hip",
           "backward_chunked.hip"]

# Packed-fp32 instructions are disabled for every device compile; hipcc's host
# pass does not know the feature and says so, which is harmless.
HIPFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


# Backend options per compilation unit, each measured on its kernels (results identical bit for
# bit): the ILP-first machine scheduler speeds up the latency-bound prefill state pass and
# backward walk but slows the preparation and decode kernels; MFMA accumulators in
# architectural VGPRs (rather than AGPRs) speed up both prefill passes.
_ILP = ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]
_MFMA_VGPR = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
FILE_FLAGS = {"prefill.hip": _MFMA_VGPR, "prefill_state.hip": _ILP + _MFMA_VGPR, "backward.hip": _ILP}


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith((".hip", ".cpp")) else []
    cmd = [_hipcc(), *HIPFLAGS, *FILE_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
