"""Builds libpa.so in-tree: host C++ with g++, device code with hipcc (gfx950).

Run as ``python -m paged_kv_cache_338_amd._build``.  Always recompiles.
It also builds ``libpa_floor.so``, the benchmark's floor kernels (a separate
library: nothing in libpa.so uses them).

``python -m paged_kv_cache_338_amd._build --sanitize`` builds a second copy,
``libpa_sanitize.so``, whose host sources (the allocator and the status
calls) are compiled by g++ with AddressSanitizer and UndefinedBehavior-
Sanitizer and linked by g++; the device sources are built as usual (the
sanitizers cover host code only).  The binding loads it when PA_LIBRARY
names it; the CPU tests of the allocator then run under the sanitizers
with the two runtimes preloaded:

    PA_LIBRARY=$PWD/paged_kv_cache_338_amd/libpa_sanitize.so \
    LD_PRELOAD="$(g++ -print-file-name=libasan.so):$(g++ -print-file-name=libubsan.so)" \
    ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \
    python -m pytest tests/test_capi_host.py -q -p no:cacheprovider

(leak checking is off because the Python interpreter itself keeps
allocations until exit).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpa.so")
SANITIZE_LIB = os.path.join(PKG, "libpa_sanitize.so")
# Measurement kernels for the decode's cost floor, loaded by bench.py only.
FLOOR_LIB = os.path.join(PKG, "libpa_floor.so")
FLOOR_SOURCE = "pa_floor.hip"

ARCH = "gfx950"
HOST_SOURCES = ["pa_status.cpp", "pa_allocator.cpp"]
DEVICE_SOURCES = ["pa_cache_ops.hip", "pa_decode.hip", "pa_prefill.hip"]
# Packed fp32 VALU instructions are disabled for all device code.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-command-line-argument"]
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]
# Host-only instrumentation for the --sanitize copy (g++ lines only).
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-g"]


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build step failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def _device_objects(verbose):
    """Compiles the device sources concurrently (the decode source, with its
    many kernel variants, takes minutes on its own)."""
    from concurrent.futures import ThreadPoolExecutor

    hipcc = _hipcc()
    jobs = []
    for src in DEVICE_SOURCES:
        obj = os.path.join(OBJ, src + ".o")
        jobs.append(([hipcc, *HIP_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj],
                     obj))
    with ThreadPoolExecutor(max_workers=len(jobs)) as pool:
        for f in [pool.submit(_run, cmd, verbose) for cmd, _ in jobs]:
            f.result()
    return [obj for _, obj in jobs]


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ, exist_ok=True)
    cxx = shutil.which("g++") or "g++"
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(OBJ, src + ".o")
        _run([cxx, *CXX_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, src), "-o", obj], verbose)
        objs.append(obj)
    objs += _device_objects(verbose)
    tmp = LIB + ".tmp"
    _run([_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    build_floor(verbose)
    return LIB


def build_floor(verbose: bool = True) -> str:
    """libpa_floor.so: the benchmark's floor kernels (not part of libpa.so)."""
    os.makedirs(OBJ, exist_ok=True)
    obj = os.path.join(OBJ, FLOOR_SOURCE + ".o")
    _run([_hipcc(), *HIP_FLAGS, "-c", os.path.join(CSRC, FLOOR_SOURCE), "-o", obj], verbose)
    tmp = FLOOR_LIB + ".tmp"
    _run([_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", obj, "-o", tmp], verbose)
    os.replace(tmp, FLOOR_LIB)
    return FLOOR_LIB


def build_sanitize(verbose: bool = True) -> str:
    """libpa_sanitize.so: sanitized host objects (g++), plain device objects,
    linked by g++ against the HIP runtime."""
    os.makedirs(OBJ, exist_ok=True)
    cxx = shutil.which("g++") or "g++"
    objs = []
    for src in HOST_SOURCES:
        obj = os.path.join(OBJ, src + ".san.o")
        _run([cxx, *CXX_FLAGS, *SANITIZE_FLAGS, "-I", INCLUDE, "-c", os.path.join(CSRC, src),
              "-o", obj], verbose)
        objs.append(obj)
    objs += _device_objects(verbose)
    rocm_lib = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    tmp = SANITIZE_LIB + ".tmp"
    _run([cxx, "-shared", *SANITIZE_FLAGS, *objs, "-L", rocm_lib, f"-Wl,-rpath,{rocm_lib}",
          "-lamdhip64", "-o", tmp], verbose)
    os.replace(tmp, SANITIZE_LIB)
    return SANITIZE_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitize(verbose="-q" not in sys.argv))
    else:
        build(verbose="-q" not in sys.argv)
        print(LIB)
