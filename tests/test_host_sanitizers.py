"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The library's host plan builder (plan.cpp) and the serial C oracle are built
with -fsanitize=address,undefined into one driver (tests/native), which runs
them on small boxes and compares their PulseData. Any out-of-bounds access,
leak or undefined behaviour aborts the driver; GPU code is not involved.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "domain_decomposition_halo_fusedpackx_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="no host compiler")
def test_plan_builder_and_oracle_under_sanitizers(tmp_path):
    d = str(tmp_path)
    subprocess.check_call(["gcc", *SAN, "-std=c99", "-ffp-contract=off", "-c",
                           os.path.join(ROOT, "oracle", "halo_oracle.c"),
                           "-o", os.path.join(d, "oracle.o")])
    subprocess.check_call(["g++", *SAN, "-std=c++17", "-ffp-contract=off", "-pthread",
                           "-I", CSRC, os.path.join(ROOT, "tests", "native", "sanitize_driver.cpp"),
                           os.path.join(CSRC, "plan.cpp"), os.path.join(d, "oracle.o"),
                           "-o", os.path.join(d, "driver"), "-lm"])
    # verify_asan_link_order=0: the environment may preload a library ahead of
    # the ASan runtime; the driver is left to run with it
    env = dict(os.environ,
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([os.path.join(d, "driver")], capture_output=True, text=True, env=env,
                       timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "0 case(s) differ" in r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host compiler")
def test_epoch_bookkeeping_under_sanitizers(tmp_path):
    """The host's epoch count per kernel family moves only for launches that
    were enqueued, and a capture switches the plan to inferred epochs."""
    exe = os.path.join(str(tmp_path), "epoch_check")
    subprocess.check_call(["g++", *SAN, "-std=c++17", "-I", CSRC,
                           os.path.join(ROOT, "tests", "native", "epoch_check.cpp"), "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 epoch check(s) failed" in r.stdout
