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


# Host-sanitized variant for the host-only ABI tests: every host part built
# with AddressSanitizer and UndefinedBehaviorSanitizer (the device code is
# compiled as usual), loaded with the ASan runtime preloaded.
SAN_BUILD = os.path.join(HERE, "_build_san")
SAN_LIB = os.path.join(HERE, "_san", "libqgemv.so")
SAN_COMPILE = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer".split()
SAN_LINK = "-fsanitize=address -fsanitize=undefined -fno-gpu-sanitize".split()


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    cmd = [_hipcc(), *COMMON, "-c", path, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
        cmd += DEVICE_ONLY
    cmd += EXTRA.get(src, [])
    cmd += list(extra)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _build(build_dir: str, lib: str, compile_extra=(), link_extra=(), verbose: bool = False) -> str:
    os.makedirs(build_dir, exist_ok=True)
    os.makedirs(os.path.dirname(lib), exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 4)), 16)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, build_dir, compile_extra), SOURCES))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs, *link_extra]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def build(verbose: bool = False) -> str:
    return _build(BUILD, LIB, verbose=verbose)


def asan_runtime() -> str:
    """Path of the ASan runtime that a host-sanitized library needs preloaded."""
    clang = os.path.join(os.path.dirname(os.path.realpath(_hipcc())), "..", "lib", "llvm", "bin", "clang++")
    if not os.path.exists(clang):
        clang = shutil.which("clang++") or "clang++"
    r = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return r.stdout.strip()


def build_sanitized(verbose: bool = False) -> str:
    """The host-sanitized library (rebuilt only when a source is newer)."""
    if os.path.exists(SAN_LIB):
        newest = max(os.path.getmtime(p) for d in (CSRC, INCLUDE) for p in
                     (os.path.join(d, f) for f in os.listdir(d)))
        if os.path.getmtime(SAN_LIB) >= max(newest, os.path.getmtime(__file__)):
            return SAN_LIB
    return _build(SAN_BUILD, SAN_LIB, SAN_COMPILE, SAN_LINK, verbose=verbose)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
