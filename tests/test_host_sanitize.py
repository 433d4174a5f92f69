"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, CPU only
(no HIP code is built here):
- the argument checker: tests/host/validate_fuzz.cpp is built with g++
  together with csrc/gemv_validate.cpp and drives every checking entry point
  with random, extreme and malformed arguments;
- the CPU comparison GEMV: tests/host/cpu_fused_fuzz.c is built with gcc
  together with cpu/cpu_fused.c and runs random ragged shapes, every format
  and epilogue, fused and unfused, in place and not, over heap buffers of
  exactly the documented sizes;
- the oracle's C code: tests/host/oracle_fuzz.c is built with gcc together
  with oracle/gemv_oracle.c and calls every oracle routine over buffers of
  exactly the sizes the oracle documents.
See those files for the properties they check."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FLAGS = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all"]


def _build(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "validate_fuzz")
    cmd = [gxx, *FLAGS, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "decode_gemv_elementwise_amd", "csrc"),
           os.path.join(ROOT, "tests", "host", "validate_fuzz.cpp"),
           os.path.join(ROOT, "decode_gemv_elementwise_amd", "csrc", "gemv_validate.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if r.returncode != 0 and "sanitize" in r.stderr and ("cannot find" in r.stderr or "not supported" in r.stderr):
        pytest.skip("sanitizer runtime not available: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr[-3000:]
    return exe


def test_checker_under_sanitizers(tmp_path):
    exe = _build(tmp_path)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, "300000"], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.stdout.startswith("ok 300000 iterations")


def test_cpu_comparison_gemv_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    flags = open("/proc/cpuinfo").read() if os.path.exists("/proc/cpuinfo") else ""
    if not all(f in flags for f in (" avx2", " fma", " f16c")):
        pytest.skip("needs an AVX2/FMA/F16C host")
    exe = str(tmp_path / "cpu_fused_fuzz")
    cmd = [gcc, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-pthread", "-mavx2", "-mfma", "-mf16c", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "host", "cpu_fused_fuzz.c"),
           os.path.join(ROOT, "decode_gemv_elementwise_amd", "cpu", "cpu_fused.c"), "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, "400"], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.stdout.startswith("ok 400 iterations")


def test_oracle_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_fuzz")
    cmd = [gcc, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", os.path.join(ROOT, "tests", "host", "oracle_fuzz.c"),
           os.path.join(ROOT, "oracle", "gemv_oracle.c"), "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, "300"], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.stdout.startswith("ok 300 iterations")
