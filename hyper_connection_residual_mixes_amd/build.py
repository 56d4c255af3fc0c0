"""Compile the HIP library libhc.so for gfx950, in-tree (next to this file)."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libhc.so")
SOURCES = [os.path.join(CSRC, "hc_kernels.hip"), os.path.join(CSRC, "hc_generic.hip"),
           os.path.join(CSRC, "hc_noalloc.hip"), os.path.join(CSRC, "hc_abi.cpp")]

# Packed-FP32 VALU forms are switched off for all device code.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def build(out: str = LIB_PATH, extra_flags=(), sources=None) -> str:
    """Always recompiles. Returns the path of the built shared library."""
    cmd = [hipcc(), *HIP_FLAGS, *extra_flags, "-shared",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           *(sources or SOURCES), "-o", out + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr}")
    os.replace(out + ".tmp", out)
    return out


# The MFMA-rate loop keeps its accumulators in VGPRs; in the accumulation-register
# form the compiler moves them between registers around every MFMA.
CEILINGS_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]


def build_bench_ceilings(out: str = os.path.join(ROOT, "bench_ceilings.so")) -> str:
    """The benchmark's ceiling kernels (plain copy, MFMA rate: bench_ceilings.hip at
    the repository root), a library of its own: it is measurement, not part of the
    C ABI."""
    return build(out=out, extra_flags=CEILINGS_FLAGS, sources=[os.path.join(ROOT, "bench_ceilings.hip")])


def build_host_sanitized(out: str) -> str:
    """The same library with AddressSanitizer and UndefinedBehaviorSanitizer on its
    host code only (the device code is built as usual); every finding aborts. For
    CPU tests of the C-ABI validation: load it with the clang ASan runtime
    preloaded (``sanitizer_runtime()``)."""
    flags = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=all", "-shared-libsan", "-fno-omit-frame-pointer"]
    return build(out=out, extra_flags=flags)


def sanitizer_runtime() -> str:
    """Path of the clang ASan runtime that a host-sanitized build needs preloaded."""
    r = subprocess.run([hipcc(), "--print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("clang ASan runtime not found")
    return path


if __name__ == "__main__":
    print(build())
