"""Build libmoe.so in-tree with hipcc for gfx950.

    python -m mixture_experts_ffn_05_amd.build

Compiles every csrc/*.hip translation unit to an object in parallel, then links
them into mixture_experts_ffn_05_amd/libmoe.so.  Always recompiles.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libmoe.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # keep the compiler from emitting packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libmoe needs ROCm's hipcc to build")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src).replace(".hip", ".o"))
    cmd = [hipcc(), *COMMON_FLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    noise = "not a recognized feature for this target"
    warn = "\n".join(l for l in res.stderr.splitlines() if l.strip() and noise not in l)
    if warn and verbose:
        print(warn, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    workers = min(len(sources), max(1, min(8, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), sources))
    tmp = LIB_PATH + ".tmp"
    # roctx (the stage ranges every call opens) from ROCm's profiler SDK
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-L/opt/rocm/lib",
           "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


# Host-only sanitizers for the C-ABI layer (argument validation, error strings,
# scratch bookkeeping): each -fsanitize= applies to the host pass only, so the
# gfx950 code is built exactly as in the library.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
SANITIZED_LIB = os.path.join(BUILD_DIR, "sanitized", "libmoe_sanitized.so")


def asan_runtime() -> str:
    """clang's shared AddressSanitizer runtime, which a process must preload to load SANITIZED_LIB."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang's AddressSanitizer runtime was not found under /opt/rocm/llvm")
    return hits[-1]


def build_sanitized(verbose: bool = False) -> str:
    """A copy of libmoe whose C-ABI layer (moe_api.hip) is built with AddressSanitizer
    and UndefinedBehaviorSanitizer on the host side, linked with the library's
    other objects as built by build().  For host-side tests only (no GPU needed)."""
    out_dir = os.path.dirname(SANITIZED_LIB)
    os.makedirs(out_dir, exist_ok=True)
    others = [os.path.join(BUILD_DIR, os.path.basename(s).replace(".hip", ".o"))
              for s in sorted(glob.glob(os.path.join(CSRC, "*.hip"))) if not s.endswith("moe_api.hip")]
    if not all(os.path.exists(o) for o in others):
        build(verbose)
    api_obj = os.path.join(out_dir, "moe_api_sanitized.o")
    cmd = [hipcc(), *COMMON_FLAGS, *SANITIZE_HOST, "-c", os.path.join(CSRC, "moe_api.hip"), "-o", api_obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on moe_api.hip (sanitized):\n{res.stdout}\n{res.stderr}")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *SANITIZE_HOST, "-shared-libsan", api_obj,
           *others, "-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib", "-o", SANITIZED_LIB]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed (sanitized):\n{res.stdout}\n{res.stderr}")
    return SANITIZED_LIB


if __name__ == "__main__":
    if "--sanitized" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
