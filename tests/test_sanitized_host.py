"""The host-side C++ of the library (argument checks and workspace geometry,
csrc/sv_host.cpp) and the C oracle, built with AddressSanitizer and
UndefinedBehaviorSanitizer by the host compilers and run on the CPU: the
drivers under tests/sanitize/ call every check and size query, and every
oracle entry point, with valid and invalid arguments (see their headers).
No GPU and no HIP compiler: g++ / gcc build the plain sources, with the HIP
runtime API header for the public stream type only."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "draft_token_verification_07_amd", "csrc")
ROCM_INC = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "include")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-Wall", "-Wextra", "-Werror"]


def _build_and_run(tmp_path, compiler, sources, flags, expect):
    if shutil.which(compiler) is None:
        pytest.skip("%s not found" % compiler)
    exe = str(tmp_path / "driver")
    cmd = [compiler] + flags + SAN + sources + ["-o", exe]
    if compiler == "gcc":
        cmd += ["-lm", "-lpthread"]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, "build failed:\n%s\n%s" % (" ".join(cmd), b.stderr[-4000:])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and expect in r.stdout, "driver failed (%d):\n%s\n%s" % (
        r.returncode, r.stdout[-2000:], r.stderr[-6000:])


def test_host_checks_sanitized(tmp_path):
    _build_and_run(tmp_path, "g++",
                   [os.path.join(HERE, "sanitize", "host_checks.cpp"), os.path.join(CSRC, "sv_host.cpp")],
                   ["-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INC, "-I", os.path.join(ROOT, "include"),
                    "-I", CSRC], "host ok")


def test_oracle_sanitized(tmp_path):
    _build_and_run(tmp_path, "gcc",
                   [os.path.join(HERE, "sanitize", "oracle_checks.c"), os.path.join(ROOT, "oracle", "spec_oracle.c")],
                   ["-std=c11"], "oracle ok")
