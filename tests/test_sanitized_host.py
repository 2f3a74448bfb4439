"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Two drivers are compiled with the host compilers (g++ / gcc, never the GPU
compiler) with -fsanitize=address,undefined and run:
  * tests/sanitize/host_checks.cpp: the library's planner and argument
    validation (paged_kv_decode_amd/csrc/planner.cpp, validate.cpp: pure
    C++, no HIP call) over seeded random and extreme sizes, checking every
    accepted plan against what the kernels rely on;
  * tests/sanitize/oracle_checks.c: the float64 oracle over seeded small
    problems with exactly sized buffers, direct against partitioned.
Any sanitizer report aborts the driver (-fno-sanitize-recover=all).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]


def _build_and_run(tmp_path, compiler, std, sources, includes, libs=()):
    if shutil.which(compiler) is None:
        pytest.skip("%s not found" % compiler)
    exe = str(tmp_path / "driver")
    cmd = [compiler, std] + SAN + ["-I" + os.path.join(ROOT, i) for i in includes] + \
        [os.path.join(ROOT, s) for s in sources] + ["-o", exe] + list(libs)
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "ERROR: AddressSanitizer" not in res.stderr
    assert "runtime error" not in res.stderr
    return res.stdout


def test_planner_and_validation_under_sanitizers(tmp_path):
    out = _build_and_run(tmp_path, "g++", "-std=c++17",
                         ["tests/sanitize/host_checks.cpp",
                          "paged_kv_decode_amd/csrc/planner.cpp",
                          "paged_kv_decode_amd/csrc/validate.cpp"],
                         ["include", "paged_kv_decode_amd/csrc"])
    assert "host checks passed" in out


def test_oracle_under_sanitizers(tmp_path):
    out = _build_and_run(tmp_path, "gcc", "-std=c11",
                         ["oracle/pa_oracle.c", "tests/sanitize/oracle_checks.c"], [], ["-lm"])
    assert "oracle checks passed" in out
