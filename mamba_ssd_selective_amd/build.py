"""Build libm2ssd.so (the gfx950 HIP kernels + the C ABI) in-tree with hipcc.

Usage: python -m mamba_ssd_selective_amd.build   (or build() from Python).
Every source is compiled for gfx950 only; objects go to _build/ at the repo root
and the shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libm2ssd.so")
ARCH = "gfx950"

SOURCES = ["conv_rows.hip", "ssd_scan.hip", "ssd_chunked.hip", "gated_norm.hip", "decode_step.hip",
           "inproj.hip", "m2ssd_api.cpp"]

# Packed fp32 instructions are disabled for all device code (see the design notes).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libm2ssd.so)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd.insert(1, "-xhip")
    t = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in l and l.strip())
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{msgs}")
    if verbose:
        print(f"  compiled {src} in {time.time() - t:.1f}s" + (f"\n{msgs}" if msgs else ""), flush=True)
    return obj


def build(verbose: bool = True) -> str:
    """Compile every source for gfx950 and link libm2ssd.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"  linked {LIB}", flush=True)
    return LIB


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the C ABI
# layer, for the CPU tests of its argument checks: only m2ssd_api.cpp is
# rebuilt, its host code instrumented (each -fsanitize= applies to the host
# compilation only; the device code and the kernel objects are unchanged).
# Load it with the clang ASan runtime preloaded (asan_runtime()).
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_LIB = os.path.join(BUILD, "san", "libm2ssd_san.so")


def asan_runtime() -> str:
    """Path of clang's shared ASan runtime in the ROCm LLVM tree."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(_hipcc())))
    for cand in sorted(glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                              "libclang_rt.asan-x86_64.so")), reverse=True):
        return cand
    raise RuntimeError("clang ASan runtime not found under the ROCm LLVM tree")


def build_host_sanitized(verbose: bool = False) -> str:
    """Link libm2ssd_san.so: the kernel objects of build() plus m2ssd_api.cpp with
    host ASan/UBSan.  Returns its path."""
    os.makedirs(os.path.join(BUILD, "san"), exist_ok=True)
    kernels = [os.path.join(BUILD, s + ".o") for s in SOURCES if s != "m2ssd_api.cpp"]
    if not all(os.path.exists(o) for o in kernels):
        build(verbose)
    obj = os.path.join(BUILD, "san", "m2ssd_api.o")
    cmd = [_hipcc(), "-xhip", "-O1", "-g", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
           "-I", os.path.join(ROOT, "include"), *DEVICE_FLAGS, *SAN_FLAGS,
           "-c", os.path.join(CSRC, "m2ssd_api.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *SAN_FLAGS, "-shared-libasan",
           "-o", SAN_LIB, *kernels, obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    if verbose:
        print(f"  linked {SAN_LIB}", flush=True)
    return SAN_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
