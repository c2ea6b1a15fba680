"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two separate programs, built here with the host compilers and run as child
processes:
  * tests/native/api_sanitize.cpp against libgdn's C ABI, with the API source
    (argument validation, workspace sizing, launch planning, error text)
    compiled sanitized and the kernels' host objects linked as the library
    build left them; every call it makes returns before any HIP call;
  * tests/native/oracle_sanitize.c against the fp64 oracle's C source,
    compiled sanitized with OpenMP.
The two never link together: the oracle and the library share no code.
Sanitizer flags go to g++/gcc only; no GPU code is built with them.
"""
import os
import shutil
import subprocess

import pytest

from linear_attention_recurrence_deltanet_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
SAN = ["-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=undefined"]
ENV_UB = "halt_on_error=1:print_stacktrace=1"


def _need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not available")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def _kernel_objects():
    objs = [os.path.join(B.PKG, "_build", s + ".o") for s in B.HIP_SOURCES]
    srcs = [os.path.join(B.CSRC, s) for s in B.HIP_SOURCES]
    if not all(os.path.exists(o) for o in objs) or \
            any(os.path.getmtime(s) > os.path.getmtime(o) for s, o in zip(srcs, objs)):
        B.build(verbose=False)
    return objs


def test_api_under_asan_ubsan(tmp_path):
    _need("g++")
    objs = _kernel_objects()
    inc = ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", f"-I{B.INCLUDE}", f"-I{B.CSRC}"]
    api_o = str(tmp_path / "gdn_api.o")
    main_o = str(tmp_path / "api_sanitize.o")
    exe = str(tmp_path / "api_sanitize")
    _run(["g++", "-std=c++17", *SAN, *inc, "-c", os.path.join(B.CSRC, "gdn_api.cpp"), "-o", api_o])
    _run(["g++", "-std=c++17", *SAN, f"-I{B.INCLUDE}", "-c", os.path.join(NATIVE, "api_sanitize.cpp"),
          "-o", main_o])
    _run(["g++", *SAN, main_o, api_o, *objs, "-L/opt/rocm/lib", "-lamdhip64",
          "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    # leaks are not checked here: the HIP runtime's own allocations outlive main
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS=ENV_UB)
    r = _run([exe], env=env, timeout=300)
    assert "0 failures" in r.stdout, r.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    _need("gcc")
    exe = str(tmp_path / "oracle_sanitize")
    _run(["gcc", "-std=c99", *SAN, "-fopenmp", os.path.join(NATIVE, "oracle_sanitize.c"),
          os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS=ENV_UB,
               OMP_NUM_THREADS="4")
    r = _run([exe], env=env, timeout=300)
    assert "0 failures" in r.stdout, r.stdout
