"""Build libpa.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: ``python -m paged_kv_cache_185_amd.build`` or ``build_library()``.
Every call recompiles.  Objects go to ``_build/`` at the repository root;
the library lands next to this file as ``libpa.so``.
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
LIB = os.path.join(PKG, "libpa.so")

SOURCES = ["api.cpp", "pool.cpp", "cache_ops.hip", "decode.hip", "prefill.hip", "noalloc.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def common_flags():
    return [
        "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
        # never emit packed fp32 VALU ops (v_pk_fma_f32 and friends)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC, "-Wall", "-Wno-unused-function",
    ]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is noise
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


# ---- host sanitizer build ---------------------------------------------------
#
# The host code (page pool, argument checks, work planning) compiled with
# AddressSanitizer and UndefinedBehaviorSanitizer into a CPU-only test build of
# the library.  Only host code is instrumented: pool.cpp and api.cpp are
# compiled as plain C++ by clang, with no device pass, and linked with the
# kernels' objects from the normal build (never launched by the CPU tests).
# The library needs the sanitizer runtime loaded first in the process
# (sanitizer_runtime(), e.g. through LD_PRELOAD of a child process).

SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libasan"]
SAN_BUILD = os.path.join(BUILD, "host_sanitize")
SAN_LIB = os.path.join(SAN_BUILD, "libpa_host_sanitize.so")


def host_clang() -> str:
    for cand in (os.environ.get("PA_HOST_CLANG"), "/opt/rocm/llvm/bin/clang++", shutil.which("clang++")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("clang++ not found: the host sanitizer build needs it")


def sanitizer_runtime() -> str:
    """Path of the shared ASan runtime (which carries UBSan) of host_clang()."""
    r = subprocess.run([host_clang(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        r = subprocess.run([host_clang(), "-print-runtime-dir"], capture_output=True, text=True)
        path = os.path.join(r.stdout.strip(), "libclang_rt.asan-x86_64.so")
    if not os.path.exists(path):
        raise RuntimeError("shared AddressSanitizer runtime not found")
    return path


def build_host_sanitized(verbose: bool = False) -> str:
    """Build the host-sanitizer test library (SAN_LIB) and return its path."""
    os.makedirs(SAN_BUILD, exist_ok=True)
    kernel_objs = [os.path.join(BUILD, s + ".o") for s in SOURCES if s.endswith(".hip")]
    if not all(os.path.exists(o) for o in kernel_objs):
        os.makedirs(BUILD, exist_ok=True)
        with cf.ThreadPoolExecutor(max_workers=3) as ex:
            list(ex.map(_compile, [s for s in SOURCES if s.endswith(".hip")]))
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    flags = ["-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", "-fPIC", "-x", "c++",
             "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"), "-I", INCLUDE, "-I", CSRC] + SANITIZE

    def host_obj(src):
        obj = os.path.join(SAN_BUILD, src + ".o")
        r = subprocess.run([host_clang()] + flags + ["-c", os.path.join(CSRC, src), "-o", obj],
                           capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"sanitizer build of {src} failed:\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=2) as ex:
        objs = list(ex.map(host_obj, ["pool.cpp", "api.cpp"]))
    tmp = SAN_LIB + ".tmp"
    r = subprocess.run([host_clang(), "-shared", "-o", tmp] + objs + kernel_objs + SANITIZE +
                       ["-L", os.path.join(rocm, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib")],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("sanitizer link failed:\n" + r.stderr)
    os.replace(tmp, SAN_LIB)
    if verbose:
        print("built", SAN_LIB)
    return SAN_LIB


if __name__ == "__main__":
    build_library(verbose=True)
    if len(sys.argv) > 1 and sys.argv[1] == "--host-sanitize":
        build_host_sanitized(verbose=True)
