"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The library's host side (argument checks, plan selection and the decision
  model: csrc/fgemm_api.cpp, csrc/model.cpp) is built with g++ and the sanitizers
  next to link stand-ins for the device launchers (tests/sanitize/device_stubs.cpp),
  and tests/sanitize/host_harness.cpp drives the host-only entry points over a grid
  of shapes, layouts, types, epilogues and model constants.
* The oracle (oracle/oracle.c) is built with gcc and the sanitizers, and the
  oracle pins run against that build (FGEMM_ORACLE_LIB, with the sanitizer runtime
  preloaded into the Python process).
Any sanitizer report fails the test.  No GPU code is built with a sanitizer."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT = os.path.join(ROOT, "_build", "sanitize")
CSRC = os.path.join(ROOT, "hgemm_strassen_type_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV_SAN = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=0:halt_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    return r


def _have(tool):
    return subprocess.run(["which", tool], capture_output=True).returncode == 0


@pytest.mark.skipif(not _have("g++") or not os.path.isdir("/opt/rocm/include"),
                    reason="needs g++ and the ROCm headers")
def test_host_library_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    inc = ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-I" + CSRC]
    srcs = [os.path.join(CSRC, "fgemm_api.cpp"), os.path.join(CSRC, "model.cpp"),
            os.path.join(ROOT, "tests", "sanitize", "device_stubs.cpp"),
            os.path.join(ROOT, "tests", "sanitize", "host_harness.cpp")]
    exe = os.path.join(OUT, "host_harness")
    _run(["g++", "-std=c++17", "-O1", "-g", *SAN, *inc, *srcs, "-o", exe,
          "-L/opt/rocm/lib", "-Wl,-rpath,/opt/rocm/lib", "-lamdhip64"])
    r = _run([exe], env={**os.environ, **ENV_SAN}, timeout=600)
    assert "0 failures" in r.stdout, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr


@pytest.mark.skipif(not _have("gcc"), reason="needs gcc")
def test_oracle_pins_under_sanitizers():
    os.makedirs(OUT, exist_ok=True)
    lib = os.path.join(OUT, "liboracle_san.so")
    _run(["gcc", "-O1", "-g", *SAN, "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-pthread", "-o", lib, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    asan = _run(["gcc", "-print-file-name=libasan.so"]).stdout.strip()
    ubsan = _run(["gcc", "-print-file-name=libubsan.so"]).stdout.strip()
    env = {**os.environ, **ENV_SAN, "FGEMM_ORACLE_LIB": lib, "LD_PRELOAD": f"{asan}:{ubsan}"}
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       capture_output=True, text=True, env=env, cwd=ROOT, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "runtime error" not in out and "ERROR: AddressSanitizer" not in out, out[-6000:]
