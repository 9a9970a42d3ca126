"""Build liblce.so for gfx950 with hipcc (in-tree, next to this file).

    python -m linear_cross_entropy_vocab_amd.build        # or build() from Python

Every HIP source under csrc/ is compiled with -O3 for gfx950 (packed-fp32 instructions
disabled) into _build/, then linked into linear_cross_entropy_vocab_amd/liblce.so.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblce.so")
ARCH = "gfx950"

FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build liblce.so)")


def _compile(hipcc: str, src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(hipcc, s), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host-sanitizer build: only the host code (the C ABI's argument checks, workspace carving
# and launch planning) compiled with AddressSanitizer and UndefinedBehaviorSanitizer, as
# relocatable host objects with no device code; it loads on a machine without a GPU and runs
# every host-side check of the ABI, never a kernel.  Loaded through LCE_LIBRARY with the
# sanitizer runtime preloaded (tests/test_host_sanitizers.py).
SAN_DIR = os.path.join(BUILD, "asan")
SAN_LIB = os.path.join(SAN_DIR, "liblce_asan.so")
SAN_HOST = ["-Xarch_host", "-fsanitize=address,undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_host_sanitized() -> str:
    hipcc = _hipcc()
    os.makedirs(SAN_DIR, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    common = ["-O1", "-g", "-std=c++17", "-fPIC", "-fgpu-rdc", "--offload-host-only", *SAN_HOST,
              "-I", INCLUDE, "-I", CSRC]

    def comp(src):
        obj = os.path.join(SAN_DIR, os.path.basename(src) + ".o")
        r = subprocess.run([hipcc, *common, "-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc (host sanitizer build) failed for {src}:\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(comp, srcs))
    r = subprocess.run([hipcc, "-shared", "-fPIC", "-fgpu-rdc", "--offload-host-only", *SAN_HOST[:2], "-shared-libsan",
                        *objs, "-o", SAN_LIB], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link (host sanitizer build) failed:\n{r.stderr}")
    return SAN_LIB


def sanitizer_runtime() -> str:
    """The clang AddressSanitizer runtime of the ROCm toolchain (preloaded into Python)."""
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return hits[-1]


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
