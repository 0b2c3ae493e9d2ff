"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
the C ABI's argument checks and workspace layout (the library's
host_checks.hpp, the code api.cpp runs before any launch) and the CPU
oracle, each driven by a small program under tests/sanitize/ on
exactly-sized buffers.  Any invalid access or undefined behaviour aborts the
program."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, exe, tmp_path):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_host_checks_sanitized(tmp_path):
    exe = str(tmp_path / "host_checks")
    cmd = ["g++", "-std=c++17"] + SAN + ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
                                          "-I", os.path.join(ROOT, "include"),
                                          "-I", os.path.join(ROOT, "routed_fp8_expert_amd", "csrc"),
                                          os.path.join(ROOT, "tests", "sanitize", "host_checks.cpp"), "-o", exe]
    assert "host checks OK" in _run(cmd, exe, tmp_path)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
def test_oracle_sanitized(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    cmd = ["gcc", "-std=c99"] + SAN + ["-I", os.path.join(ROOT, "oracle"),
                                        os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
                                        os.path.join(ROOT, "oracle", "moe_oracle.c"), "-lm", "-o", exe]
    assert "oracle OK" in _run(cmd, exe, tmp_path)
