"""CPU AddressSanitizer + UndefinedBehaviorSanitizer build of the host code: the planner
(problem validation, variant tables, cost models, the chain planner) and the oracle, driven
over benchmark shapes, random valid and invalid problems, random chains and small oracle
evaluations by tests/sanitize/sanitize_driver.cpp.  Built with g++/gcc (no device code),
so no GPU is needed; any sanitizer report fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "depthwise_pointwise_convolution_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="needs g++ and gcc")
def test_planner_and_oracle_under_address_and_ub_sanitizers(tmp_path):
    oracle_o = str(tmp_path / "fcm_oracle.o")
    r = subprocess.run(["gcc", "-std=c11", "-ffp-contract=off", *SAN, "-c",
                        os.path.join(ROOT, "oracle", "fcm_oracle.c"), "-o", oracle_o],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    exe = str(tmp_path / "sanitize_driver")
    r = subprocess.run(["g++", "-std=c++17", *SAN, "-I" + os.path.join(ROOT, "include"),
                        "-I" + CSRC, os.path.join(ROOT, "tests", "sanitize", "sanitize_driver.cpp"),
                        os.path.join(CSRC, "plan.cpp"), oracle_o, "-o", exe, "-lm"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "sanitized run done" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
