"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only): the oracle's pins run against an instrumented build of oracle.c, and
the library's host-side argument validation (plan.cpp, which has no HIP
dependency) runs over valid and invalid arguments in an instrumented driver.
Any out-of-bounds access, use after free or undefined behaviour aborts the
run."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]

needs_gcc = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="no gcc")


def _libasan():
    path = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("libasan not available")
    return path


@needs_gcc
def test_plan_checks_under_asan_ubsan(tmp_path):
    exe = tmp_path / "plan_san"
    csrc = os.path.join(ROOT, "differential_attention_amd", "csrc")
    subprocess.check_call(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"), "-I", csrc,
                           os.path.join(ROOT, "tests", "sanitize", "plan_driver.cpp"),
                           os.path.join(csrc, "plan.cpp"), "-o", str(exe)])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "plan checks ok" in r.stdout


@needs_gcc
def test_oracle_pins_under_asan_ubsan(tmp_path):
    lib = tmp_path / "liboracle_san.so"
    subprocess.check_call(["gcc", *SAN, "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                           "-std=c11", "-o", str(lib), os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    env = dict(os.environ, ORACLE_LIB=str(lib), LD_PRELOAD=_libasan(),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    # the instrumented build is the one loaded
    r = subprocess.run([sys.executable, "-c", "import oracle; print(oracle._load()._name)"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0 and r.stdout.strip() == str(lib), r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join("tests", "test_oracle.py")], cwd=ROOT, capture_output=True, text=True,
                       timeout=900, env=env)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert " passed" in r.stdout
