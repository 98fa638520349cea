"""Compile the gfx950 HIP library libmoe_hip.so in-tree with hipcc.

Every call compiles (no staleness check): ``python -m sparse_mixture_experts_gating_amd.build``.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libmoe_hip.so")
BUILD_DIR = os.path.join(PKG, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall", "-Werror",
    "-Wno-unused-command-line-argument",
    # packed FP32 (v_pk_*_f32) stays off: hipcc emits it from plain float code otherwise
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]

SOURCES = ["route.hip", "permute.hip", "gemm.hip", "combine.hip", "moe_api.cpp"]

# Host-only AddressSanitizer + UndefinedBehaviorSanitizer (the GPU code is
# built as usual): each -fsanitize applies to the host pass alone.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-g"]
SANITIZED_OUT = os.path.join(BUILD_DIR, "libmoe_hip_sanitized.so")


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime the sanitized build needs preloaded."""
    import glob
    found = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib", "clang", "*",
                                          "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not found:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found under the ROCm LLVM tree")
    return found[-1]


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + (".san.o" if sanitize else ".o"))
    cmd = [HIPCC, *FLAGS, *(SANITIZE_FLAGS if sanitize else []), "-x", "hip", "-c", os.path.join(CSRC, src),
           "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile and link libmoe_hip.so; sanitize=True builds _build/libmoe_hip_sanitized.so
    instead (host code under ASan/UBSan; the sanitizer entry points stay unresolved
    in the library and come from asan_runtime(), which the loader must preload)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
    out = SANITIZED_OUT if sanitize else OUT
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv)
    sys.exit(0)
