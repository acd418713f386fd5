"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The C-ABI source (argument validation, kept counts, random budgets, workspace
sizes) is compiled with the sanitizers on its host pass only (the device code
is built as usual), linked with a C++ driver that calls every host-side path
and every validation path that must refuse before any HIP call, and run on
the CPU.  Any sanitizer report fails the test."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "learned_token_pruning_05_amd")
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(ROOT, "_build", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd[:3])} ... failed:\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(not os.path.exists(CLANG), reason="ROCm clang++ not found")
def test_host_entry_points_under_asan_ubsan(lib):
    from learned_token_pruning_05_amd import build as _build
    os.makedirs(OUT, exist_ok=True)
    hipcc = _build._hipcc()
    others = [os.path.join(_build.BUILD_DIR, os.path.basename(f) + ".o")
              for f in sorted(os.listdir(CSRC)) if f.endswith(".hip") and f != "tg_api.hip"]
    if not all(os.path.exists(o) for o in others):
        _build.build_library()
    api_obj = os.path.join(OUT, "tg_api_sanitized.o")
    san = []
    for flag in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
                 "-fno-omit-frame-pointer"):
        san += ["-Xarch_host", flag]
    flags = [f for f in _build.HIP_FLAGS if f != "-O3"] + ["-O1", "-g"]
    _run([hipcc, *flags, *san, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, "tg_api.hip"), "-o", api_obj])
    drv_obj = os.path.join(OUT, "driver.o")
    _run([CLANG, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
          "-I", INCLUDE, "-c", os.path.join(ROOT, "tests", "host_sanitize", "driver.cpp"), "-o", drv_obj])
    exe = os.path.join(OUT, "host_driver")
    _run([CLANG, "-fsanitize=address,undefined", drv_obj, api_obj, *others, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, f"driver failed ({r.returncode}):\n{r.stdout[-3000:]}\n{r.stderr[-5000:]}"
    assert "clean under ASan/UBSan" in r.stdout
    shutil.rmtree(OUT, ignore_errors=True)
