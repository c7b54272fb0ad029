"""Build libmoe.so (every HIP source under csrc/) for gfx950, in-tree.

    python -m mixture_experts_layer_28_amd.build            # libmoe.so
    python -m mixture_experts_layer_28_amd.build --sanitize # _build/asan/libmoe.so

Each .hip is compiled to an object under _build/ in parallel, then linked
into mixture_experts_layer_28_amd/libmoe.so. Always rebuilds.

--sanitize builds a copy whose host code of the C ABI (moe_abi.hip:
argument validation, workspace carving, dispatch) is instrumented with
AddressSanitizer and UndefinedBehaviorSanitizer; device code and the other
sources' host launch code are built as usual. It is loaded into a process
that preloads the sanitizer runtime (sanitizer_runtime()), for the CPU tests.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe.so")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    # packed fp32 arithmetic is disabled on purpose (plain float code only)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe)")


# host-only sanitizer flags: each -fsanitize= applies to the host pass only
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-g"]
SAN_SOURCES = ("moe_abi.hip",)


def _compile(src: str, hipcc: str, outdir: str = BUILD, extra=()) -> str:
    obj = os.path.join(outdir, os.path.basename(src) + ".o")
    cmd = [hipcc, *CFLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


def sanitizer_runtime() -> str:
    """The clang AddressSanitizer runtime (with UBSan) that a process loading
    the sanitized build preloads."""
    cands = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
                   + glob.glob("/opt/rocm/llvm/lib/clang/*/lib/x86_64-unknown-linux-gnu/libclang_rt.asan.so"))
    if not cands:
        raise RuntimeError("clang AddressSanitizer runtime not found under /opt/rocm/llvm")
    return cands[-1]


def build_sanitized(verbose: bool = False) -> str:
    """_build/asan/libmoe.so: the C ABI's host code under ASan + UBSan; the
    other objects are compiled as in build()."""
    hipcc = _hipcc()
    out = os.path.join(BUILD, "asan")
    os.makedirs(out, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def one(src):
        san = os.path.basename(src) in SAN_SOURCES
        return _compile(src, hipcc, out, SAN_FLAGS if san else ())
    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(one, srcs))
    lib_path = os.path.join(out, "libmoe.so")
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", lib_path, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(f"built {lib_path} (host ABI code sanitized)")
    return lib_path


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
