"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

* libmixer's host side (csrc/mixer_api.cpp: argument validation, size-overflow guards, the
  Latin-square scheduler, the layer runner), built with g++ against stand-in launchers that
  record each launch (tests/sanitize/host_stubs.cpp), driven by tests/sanitize/host_driver.cpp.
* The C oracle (oracle/oracle.c) with OpenMP, driven by tests/sanitize/oracle_driver.c.

Each driver exits 0 and prints "OK <checks>" only if every check holds and the sanitizers
found nothing (any report aborts the run).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
CSRC = os.path.join(ROOT, "heterogeneous_attention_mixer_amd", "csrc")
FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _compile(cmd, tmp_path):
    res = subprocess.run(cmd, cwd=tmp_path, capture_output=True, text=True, timeout=300)
    if res.returncode != 0:
        if "fsanitize" in res.stderr and ("cannot find" in res.stderr or
                                          "unrecognized" in res.stderr):
            pytest.skip("sanitizer runtime not available: " + res.stderr[-300:])
        raise AssertionError(res.stderr[-4000:])


def _run(exe):
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    out = res.stdout + res.stderr
    assert res.returncode == 0 and res.stdout.startswith("OK "), out[-4000:]
    return int(res.stdout.split()[1])


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_library_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_san")
    _compile(["g++", "-std=c++17", *FLAGS, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
              "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
              os.path.join(CSRC, "mixer_api.cpp"), os.path.join(SAN, "host_stubs.cpp"),
              os.path.join(SAN, "host_driver.cpp"), "-o", exe], tmp_path)
    assert _run(exe) > 100


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _compile(["gcc", "-std=c11", *FLAGS, "-fopenmp", os.path.join(ROOT, "oracle", "oracle.c"),
              os.path.join(SAN, "oracle_driver.c"), "-lm", "-o", exe], tmp_path)
    assert _run(exe) > 100
