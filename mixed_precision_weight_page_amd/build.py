"""Build libpagedweight.so in-tree with hipcc for gfx950.

Every HIP source is compiled with the packed-fp32 feature switched off
(``-Xclang -target-feature -Xclang -packed-fp32-ops``) and without fast-math:
the quantizer relies on IEEE fp32 division, fma and fp64 division.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpagedweight.so")
ARCH = os.environ.get("PW_OFFLOAD_ARCH", "gfx950")

COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-I", os.path.join(PKG, "..", "include")]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = ["hipcc", *COMMON, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
            if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if msgs and os.environ.get("PW_BUILD_VERBOSE"):
        print("\n".join(msgs), file=sys.stderr)
    return obj


def build(extra=(), jobs: int = 8) -> str:
    """Compile every source and link libpagedweight.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), sources()))
    tmp = LIB + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


HOST_SOURCES = ("capi.cpp", "alloc.cpp", "budget.cpp")
SAN_BUILD = os.path.join(PKG, "_build_san")
SAN_LIB = os.path.join(SAN_BUILD, "libpagedweight_san.so")
# AddressSanitizer and UndefinedBehaviorSanitizer on the host code only:
# each -fsanitize= goes right after -Xarch_host, so no device code is built
# with a sanitizer
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer",
             "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined"]


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (to preload
    into an uninstrumented interpreter that loads the sanitized library)."""
    r = subprocess.run(["hipcc", "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip().splitlines()[-1] if r.stdout.strip() else ""
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("no shared AddressSanitizer runtime found")
    return path


def build_host_sanitized(jobs: int = 3) -> str:
    """The library with its host sources (C ABI, allocator, scheduler)
    instrumented by AddressSanitizer and UndefinedBehaviorSanitizer, the
    kernels as in the normal build; returns its path. Load it with
    PW_LIBRARY set to that path and the runtime of asan_runtime() preloaded."""
    os.makedirs(SAN_BUILD, exist_ok=True)

    def compile_one(src):
        name = os.path.basename(src)
        obj = os.path.join(SAN_BUILD, name + ".o")
        extra = SAN_FLAGS if name in HOST_SOURCES else []
        cmd = ["hipcc", *COMMON, *extra, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n" + r.stdout + r.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(compile_one, sources()))
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libsan",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-o", SAN_LIB, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    return SAN_LIB


if __name__ == "__main__":
    if sys.argv[1:] == ["sanitize"]:
        print(build_host_sanitized())
    else:
        print(build(extra=sys.argv[1:]))
