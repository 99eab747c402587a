"""Build libpa.so for gfx950 in-tree with hipcc.

``python paged_kv_cache_24_amd/build.py`` compiles every HIP source under
``csrc/`` (in parallel) and links ``paged_kv_cache_24_amd/libpa.so``, and beside
it ``libpa_debug.so``: the same kernels with the C ABI layer compiled with
PA_DEBUG_BOUNDS, which checks the device-resident indices of every call
(pa_debug_bounds in include/pa.h).  Run it as a script (or load it by path):
importing the package itself needs the library.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libpa.so")
DEBUG_LIB_PATH = os.path.join(PKG, "libpa_debug.so")
ARCH = "gfx950"

SOURCES = ["pa_api.hip", "reshape_and_cache.hip", "copy_blocks.hip", "decode.hip", "decode_fp8.hip", "prefill.hip",
           "debug_bounds.hip"]

COMPILE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # no packed-FP32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libpa.so")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is harmless
    out = "\n".join(line for line in res.stdout.splitlines() if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile and link libpa.so and libpa_debug.so; returns the path of
    libpa.so.  Always recompiles."""
    hipcc = _hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        jobs.append([hipcc, *COMPILE_FLAGS, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj])
    # the debug library differs in the C ABI layer only
    api_debug = os.path.join(BUILD_DIR, "pa_api_debug.o")
    jobs.append([hipcc, *COMPILE_FLAGS, *extra_flags, "-DPA_DEBUG_BOUNDS", "-c",
                 os.path.join(CSRC, "pa_api.hip"), "-o", api_debug])
    with ThreadPoolExecutor(min(len(jobs), os.cpu_count() or 1)) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    for path, lib_objs in ((LIB_PATH, objs), (DEBUG_LIB_PATH, [api_debug] + objs[1:])):
        tmp = path + ".tmp"
        _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *lib_objs], verbose)
        os.replace(tmp, path)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
