"""AddressSanitizer and UndefinedBehaviorSanitizer builds of the host code,
run on the CPU (no GPU needed):

* the CPU oracle (oracle/oracle.cpp, g++) under a driver that calls every
  oracle function on small, ragged, NaN and non-SPD inputs with one and
  several threads (tests/sanitize/oracle_driver.cpp);
* the C ABI's host code (csrc/capi.hip; only its host part instrumented,
  launchers replaced by stand-ins) under a driver that makes every argument
  check fire (tests/sanitize/capi_driver.cpp).

Any sanitizer report ends the program with a non-zero status
(-fno-sanitize-recover=all); a clean exit passes.  The builds go to
_build_sanitize/ and take about a minute."""

import os
import shutil
import subprocess

import pytest

from conftest import ROOT

BUILD = os.path.join(ROOT, "_build_sanitize")
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "block_tridiagonal_pcg_bdmv_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ROCM = "/opt/rocm"


def _run(cmd, env=None, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)
    assert r.returncode == 0, "%s\n%s%s" % (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r


def _env(**extra):
    env = dict(os.environ)
    env.update(extra)
    return env


def test_oracle_under_asan_and_ubsan():
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    os.makedirs(BUILD, exist_ok=True)
    exe = os.path.join(BUILD, "oracle_sanitized")
    flags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-pthread",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    _run([gxx, *flags, os.path.join(ROOT, "oracle", "oracle.cpp"),
          os.path.join(SAN, "oracle_driver.cpp"), "-o", exe])
    r = _run([exe], env=_env(ASAN_OPTIONS="detect_leaks=1:halt_on_error=1",
                             UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1"))
    assert "oracle sanitizer driver: done" in r.stdout


def test_capi_host_checks_under_asan_and_ubsan():
    hipcc = os.path.join(ROCM, "bin", "hipcc")
    clang = os.path.join(ROCM, "llvm", "bin", "clang++")
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not available")
    os.makedirs(BUILD, exist_ok=True)
    capi_o = os.path.join(BUILD, "capi.o")
    # Only the host part is instrumented: each sanitizer flag applies to the
    # host compilation alone.
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host",
                "-fno-omit-frame-pointer"]
    _run([hipcc, "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-I" + INCLUDE,
          "-I" + CSRC, *host_san, "-c", os.path.join(CSRC, "capi.hip"), "-o", capi_o])
    cflags = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
              "-I" + os.path.join(ROCM, "include"), "-I" + INCLUDE,
              "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    objs = [capi_o]
    for src in ("capi_driver.cpp", "capi_stubs.cpp"):
        o = os.path.join(BUILD, src[:-4] + ".o")
        _run([clang, *cflags, "-c", os.path.join(SAN, src), "-o", o])
        objs.append(o)
    exe = os.path.join(BUILD, "capi_sanitized")
    _run([clang, "-fsanitize=address,undefined", *objs, "-L" + os.path.join(ROCM, "lib"),
          "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-o", exe])
    # The HIP runtime's own allocations are not this code's: no leak report.
    r = _run([exe], env=_env(ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
                             UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1"))
    assert "capi sanitizer driver: 0 failures" in r.stdout
