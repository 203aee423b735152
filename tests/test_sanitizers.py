"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the CPU code.

Two drivers under tests/sanitize/ run on the CPU, no GPU needed:

* oracle_driver.c exercises every routine of the C oracle on small shapes,
  with each buffer allocated at exactly the size the routine may touch;
* host_driver.cpp exercises the library's host code (handle creation,
  launch planning, plan descriptions, workspace sizing, every argument
  check), linked against api.hip compiled with a sanitized host pass.  No
  call in it reaches a kernel launch.

Any sanitizer report aborts the driver (-fno-sanitize-recover=all), so a
zero exit status means a clean run.  The public header is also compiled as
strict C and as C++.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN_DIR = os.path.join(ROOT, "tests", "sanitize")
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(ROOT, "gemm_scratch_nn_amd", "csrc")
BUILD = os.path.join(ROOT, "gemm_scratch_nn_amd", "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANGXX = "/opt/rocm/llvm/bin/clang++"
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")

need_gcc = pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not installed")
need_rocm = pytest.mark.skipif(not (os.path.exists(HIPCC) and os.path.exists(CLANGXX)),
                               reason="ROCm compilers not installed")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\nexit {r.returncode}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


@need_gcc
@pytest.mark.parametrize("std", ["c99", "c11"])
def test_header_compiles_as_strict_c(std):
    _run(["gcc", f"-std={std}", "-pedantic", "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
          "-x", "c", os.path.join(INCLUDE, "d4r_conv.h")])


@need_gcc
def test_header_compiles_as_cxx():
    _run(["g++", "-std=c++17", "-pedantic", "-Wall", "-Wextra", "-Werror", "-fsyntax-only",
          "-x", "c++", os.path.join(INCLUDE, "d4r_conv.h")])


@need_gcc
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fopenmp",
          os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(SAN_DIR, "oracle_driver.c"),
          "-lm", "-o", exe])
    r = _run([exe], env=dict(SAN_ENV, OMP_NUM_THREADS="2"), timeout=300)
    assert "all checks passed" in r.stdout


def _library_objects():
    """Objects of the regular build, rebuilt when a source is newer."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    deps = srcs + glob.glob(os.path.join(CSRC, "*.hpp")) + [os.path.join(INCLUDE, "d4r_conv.h")]
    objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in srcs]
    newest = max(os.path.getmtime(d) for d in deps)
    if any(not os.path.exists(o) or os.path.getmtime(o) < newest for o in objs):
        from gemm_scratch_nn_amd import build as b
        b.build()
    return objs


@need_rocm
def test_host_code_under_asan_ubsan(tmp_path):
    objs = [o for o in _library_objects() if not o.endswith("api.hip.o")]
    api_o = str(tmp_path / "api.o")
    drv_o = str(tmp_path / "driver.o")
    exe = str(tmp_path / "host_driver")
    # sanitizers on the host pass only: each flag follows -Xarch_host
    _run([HIPCC, "-O1", "-g", "-fno-omit-frame-pointer", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE,
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=all",
          "-c", os.path.join(CSRC, "api.hip"), "-o", api_o])
    _run([CLANGXX, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-Wall", "-Wextra",
          "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-I", INCLUDE,
          "-c", os.path.join(SAN_DIR, "host_driver.cpp"), "-o", drv_o])
    _run([CLANGXX, "-fsanitize=address,undefined", drv_o, api_o] + objs +
         ["-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    r = _run([exe], env=SAN_ENV, timeout=300)
    assert "all checks passed" in r.stdout
