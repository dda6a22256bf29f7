"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The C-ABI source (`rkv_api.hip`: schedule arithmetic, cache sizing, argument,
alignment and layout validation, the decode split hint, the scratch limit of
the allocation-free decode) is compiled with host-side instrumentation only
(`-Xarch_host` before each `-fsanitize=`; device code is built as usual) and
linked, with the kernel sources' objects of the ordinary build, into the C
program `host_asan/rkv_host_check.c`.  That program makes only calls that are
pure host arithmetic or that validation refuses before any device work, so it
runs without a GPU; a sanitizer report or a wrong status makes it exit
non-zero.  Leak detection is off: the HIP runtime keeps allocations for the
life of the process."""

import os
import shutil
import subprocess

import pytest

from conftest import ROOT

PKG = os.path.join(ROOT, "long_context_attention_rkv_amd")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
LLVM = "/opt/rocm/llvm/bin"
KERNEL_OBJS = ["k_decode.hip.o", "k_quantize.hip.o", "k_select.hip.o"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


@pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(f"{LLVM}/clang")),
                    reason="needs hipcc and the ROCm clang")
def test_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    if not all(os.path.exists(os.path.join(BUILD, o)) for o in KERNEL_OBJS):
        from long_context_attention_rkv_amd.build import build
        build(verbose=False)
    inc = os.path.join(ROOT, "include")
    api_o = str(tmp_path / "rkv_api.o")
    _run([HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-fPIC",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-fno-omit-frame-pointer", "-Wno-unused-command-line-argument", "-I", inc,
          "-c", os.path.join(PKG, "csrc", "rkv_api.hip"), "-o", api_o])
    check_o = str(tmp_path / "check.o")
    _run([f"{LLVM}/clang", "-O1", "-g", "-std=c11", "-Wall", "-Werror",
          "-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-I", inc,
          "-c", os.path.join(ROOT, "tests", "host_asan", "rkv_host_check.c"), "-o", check_o])
    exe = str(tmp_path / "rkv_host_check")
    _run([f"{LLVM}/clang++", "-fsanitize=address,undefined", check_o, api_o,
          *[os.path.join(BUILD, o) for o in KERNEL_OBJS],
          "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok "), r.stdout
    assert int(r.stdout.split()[1]) >= 100
    shutil.rmtree(tmp_path, ignore_errors=True)
