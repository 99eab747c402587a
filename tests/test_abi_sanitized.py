"""The C ABI layer built with AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

pa_api.hip is compiled with both sanitizers on its host code (the device code
is unchanged: the sanitizers apply to the host pass only), linked with the
kernels' objects of the normal build and with tests/abi_host_checks.cpp, which
drives every entry point through its refusals and the size queries through
their extremes.  The program must report every check passed with no
sanitizer finding; a finding aborts it (halt_on_error), so the exit status
carries it.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_24_amd", "csrc")
BUILD = os.path.join(ROOT, "_build")
OUT = os.path.join(BUILD, "sanitized")
KERNEL_OBJS = ["reshape_and_cache.o", "copy_blocks.o", "decode.o", "decode_fp8.o", "prefill.o",
               "debug_bounds.o"]
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("hipcc is not available")


def _run(cmd, **kw):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout[-4000:]}"
    return res.stdout


def test_abi_layer_under_asan_and_ubsan():
    hipcc = _hipcc()
    objs = [os.path.join(BUILD, o) for o in KERNEL_OBJS]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        pytest.fail(f"kernel objects missing ({missing}): run python paged_kv_cache_24_amd/build.py")
    os.makedirs(OUT, exist_ok=True)
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    api = os.path.join(OUT, "pa_api.o")
    _run([hipcc, *flags, *SAN, "-c", os.path.join(CSRC, "pa_api.hip"), "-o", api])
    drv = os.path.join(OUT, "abi_host_checks.o")
    _run([hipcc, "-x", "c++", "-O1", "-g", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"),
          "-c", os.path.join(ROOT, "tests", "abi_host_checks.cpp"), "-o", drv])
    exe = os.path.join(OUT, "abi_host_checks")
    _run([hipcc, "--offload-arch=gfx950", *SAN, drv, api, *objs, "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    out = _run([exe], env=env, timeout=120)
    assert "all host checks passed" in out, out
    assert "runtime error" not in out and "AddressSanitizer" not in out, out
