"""Builds libgdn.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc."""

from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgdn.so")
ARCH = "gfx950"
SOURCES = ["recurrent.hip", "conv_prep.hip", "chunk_prefill.hip", "epilogue.hip", "gdn_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC]
# Packed fp32 instructions stay off: ordinary float code only. Matrix-core accumulators
# are kept in the ordinary vector registers when they fit, so the vector code that scales
# and packs them needs no copies from the accumulation registers.
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form=1"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + DEVICE + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC] + COMMON + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, r.stdout, r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every kernel for gfx950 and link libgdn.so next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


# The host side of the C ABI (argument checks, dispatch) under the address and undefined-
# behaviour sanitizers, linked with the kernels' objects from the last build(). The sanitizer
# flags reach the host compilation only. Load it with the sanitizer runtime preloaded
# (LD_PRELOAD=<SANITIZER_RUNTIME>) and GDN_LIBRARY=<the returned path>.
SANITIZED_LIB = os.path.join(BUILD_DIR, "libgdn_hostsan.so")
SANITIZER_RUNTIME = "/opt/rocm/lib/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so"
_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
        "-Xarch_host", "-fno-omit-frame-pointer"]


def build_host_sanitized() -> str:
    kernels = [os.path.join(BUILD_DIR, s + ".o") for s in SOURCES if s.endswith(".hip")]
    missing = [k for k in kernels if not os.path.exists(k)]
    if missing:
        raise RuntimeError("build() first: missing %s" % ", ".join(missing))
    obj = os.path.join(BUILD_DIR, "gdn_api.hostsan.o")
    cmd = [HIPCC, "-O1", "-g", "-std=c++17", "-fPIC", "-Wall", "-I", INCLUDE, "-I", CSRC] + _SAN + [
        "-c", os.path.join(CSRC, "gdn_api.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for gdn_api.cpp:\n%s\n%s" % (r.stdout, r.stderr))
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-shared-libasan"] + _SAN + kernels + [
        obj, "-o", SANITIZED_LIB]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (r.stdout, r.stderr))
    return SANITIZED_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
