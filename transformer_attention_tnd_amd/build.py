"""Build libswa.so (HIP kernels + host C ABI) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libswa.so")
# source -> extra compiler flags
SOURCES = {
    "swa_host.cpp": [],
    "swa_fwd.hip": [],
    "swa_bwd.hip": [],
    # matrix-core results in ordinary vector registers: the softmax of the
    # bf16 backward kernels then reads them without accumulator-register copies
    "swa_bwd_kv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "swa_bwd_kv_gqa.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    # (the grouped build with dropout spills with that register form)
    "swa_bwd_kv_gqa_drop.hip": [],
    "swa_bwd_dq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "swa_noalloc.hip": [],
}
ARCH = os.environ.get("SWA_OFFLOAD_ARCH", "gfx950")


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; install ROCm or set HIPCC")


def common_flags():
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        # no packed fp32 VALU instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", os.path.join(ROOT, "include"),
    ]


def _compile(src, extra):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    # kernels: no NaN inputs are assumed, so max/min need no NaN-quieting
    # (infinities are kept); the host code validates arguments, NaN included
    kern = ["-fno-honor-nans"] if src.endswith(".hip") else []
    cmd = [hipcc()] + common_flags() + kern + extra + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose=True, extra=()):
    """Compile every source and link libswa.so; always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, SOURCES[s] + list(extra)), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
