"""Build libqgemv.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python block_quant_gemv_amd/build.py  (run as a script: importing the
package itself needs the built library).
Objects go to block_quant_gemv_amd/_build/, the library to
block_quant_gemv_amd/libqgemv.so.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqgemv.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

SOURCES = ["api.cpp", "launch_cache.cpp", "quant.hip", "gemv.hip", "kdirect.hip", "swiglu.hip", "moe.hip", "mfma.hip", "attn.hip", "s16.hip", "fact.hip", "noalloc.hip", "moe_fused.hip", "stream.hip"]

ARCH = "gfx950"
# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
COMMON = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
          f"-I{INCLUDE}", f"--offload-arch={ARCH}"]
DEVICE_ONLY = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source extras. mfma.hip: matrix-core results in ordinary VGPRs (gfx950
# has one register file), so the fp32 epilogue reads them without copies.
EXTRA = {"mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found; the library needs the ROCm toolchain")
    return h


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    cmd = [_hipcc(), *COMMON, "-c", path, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
        cmd += DEVICE_ONLY
    cmd += EXTRA.get(src, [])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 4)), 16)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
