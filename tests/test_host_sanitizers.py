"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The oracle (oracle/oracle.c) runs every function on exactly-sized heap
  buffers, ragged shapes, both formats, both input dtypes, both scale rules and
  every GEMM layout (tests/sanitize/oracle_driver.c).
- The C ABI's argument validation (api.cpp) runs with its HIP launchers and
  hipGetLastError replaced by recording stubs: valid calls must reach their
  launcher with the right extents, invalid ones must return the documented
  status (tests/sanitize/abi_driver.cpp).

Both are built with gcc / g++ (no GPU code), -fsanitize=address,undefined and
no recovery, so any report fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _build_and_run(tmp_path, cmd, exe):
    if shutil.which(cmd[0]) is None:
        pytest.skip("%s not available" % cmd[0])
    proc = subprocess.run(cmd + ["-o", str(exe)], capture_output=True, text=True)
    assert proc.returncode == 0, proc.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    report = run.stderr
    assert run.returncode == 0, report[-4000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
    return run.stdout


def test_oracle_under_asan_ubsan(tmp_path):
    out = _build_and_run(tmp_path, ["gcc", "-std=c11"] + SAN + [
        "-I", os.path.join(ROOT, "oracle"),
        os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"),
        "-lm"], tmp_path / "oracle_driver")
    assert "all checks passed" in out


def test_abi_validation_under_asan_ubsan(tmp_path):
    if not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("HIP headers not available")
    out = _build_and_run(tmp_path, ["g++", "-std=c++17"] + SAN + [
        "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
        "-I", os.path.join(ROOT, "mx_block_scaled_x128_amd", "csrc"),
        os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"),
        os.path.join(ROOT, "mx_block_scaled_x128_amd", "csrc", "api.cpp")], tmp_path / "abi_driver")
    assert "all checks passed" in out
