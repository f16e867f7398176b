"""Sanitizer builds of the host code (no GPU needed): the CPU oracle driven through every entry point,
cell and option (tests/sanitize/oracle_run.c), and the C ABI's argument validation and workspace queries
(tests/sanitize/abi_validation.cpp against the library source), each built with AddressSanitizer and
UndefinedBehaviorSanitizer and required to run clean.  The library build puts the sanitizers on the host
pass only: GPU code is built as usual."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(exe):
    p = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    out = p.stdout + p.stderr
    print(out[-3000:])
    assert p.returncode == 0, out[-3000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out
    return out


def test_oracle_runs_clean_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_run")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                           "-fno-omit-frame-pointer", "-o", exe, os.path.join(SAN, "oracle_run.c"), "-lm", "-lpthread"])
    assert "checks passed" in _run(exe)


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"), reason="no hipcc")
def test_abi_validation_runs_clean_under_host_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_validation")
    hipcc = "/opt/rocm/bin/hipcc" if os.path.exists("/opt/rocm/bin/hipcc") else "hipcc"
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "nonlinear_rnn_solve_amd", "csrc", "pararnn.hip"),
           os.path.join(SAN, "abi_validation.cpp"), "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=900)
    assert "checks passed" in _run(exe)
