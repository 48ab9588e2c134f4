"""CPU tier with sanitizers: the oracle and the library's host-side call planning are
built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc / g++, host code only)
and driven over small inputs, edge cases and argument errors by the two programs under
tests/sanitize/.  Any invalid access, leak or undefined operation fails the test."""
import os
import shutil
import subprocess

import pytest

TESTS = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(TESTS)
CSRC = os.path.join(ROOT, "linear_attention_video_gated_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]

pytestmark = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None,
                                reason="gcc / g++ not available")


def _run(exe, tmp_path):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="2")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, cwd=str(tmp_path), timeout=300)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    subprocess.run(["gcc", "-std=c99", "-fopenmp"] + SAN +
                   [os.path.join(ROOT, "oracle", "oracle_gdn.c"), os.path.join(TESTS, "sanitize", "oracle_check.c"),
                    "-o", exe, "-lm"], check=True)
    assert "ok" in _run(exe, tmp_path)


def test_host_plan_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_check")
    subprocess.run(["g++", "-std=c++17", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC] + SAN +
                   [os.path.join(CSRC, "gdn_plan.cpp"), os.path.join(TESTS, "sanitize", "plan_check.cpp"), "-o", exe],
                   check=True)
    assert "ok" in _run(exe, tmp_path)
