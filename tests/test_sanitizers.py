"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The library's host-side validation and slot / size arithmetic
  (gated_deltanet_dual_amd/csrc/host_plan.cpp) built with g++
  -fsanitize=address,undefined together with tests/sanitize/host_plan_driver.cpp,
  which drives every check on valid and invalid batch descriptions.
* The fp64 oracle (oracle/flare_oracle.c) built the same way and run under
  its own pin tests in a child process that preloads libasan (the Python
  interpreter itself is not instrumented).
Any sanitizer report aborts the child and fails the test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gated_deltanet_dual_amd", "csrc")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _runtime(name):
    return subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True).stdout.strip()


def test_host_plan_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_plan_san")
    subprocess.run(["g++", "-std=c++17"] + SAN + ["-I", CSRC, os.path.join(CSRC, "host_plan.cpp"),
                                                  os.path.join(ROOT, "tests", "sanitize", "host_plan_driver.cpp"),
                                                  "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr


def test_oracle_pins_under_asan_ubsan():
    asan = _runtime("libasan.so")
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("libasan runtime not found")
    import oracle
    oracle.build(sanitized=True)
    env = dict(os.environ, FLARE_ORACLE_SANITIZED="1", LD_PRELOAD=asan,
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    tests = [os.path.join(ROOT, "tests", t) for t in ("test_oracle_pins.py", "test_oracle_grad.py",
                                                      "test_oracle_conv_bwd.py", "test_oracle_verify.py")]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"] + tests,
                       capture_output=True, text=True, env=env, cwd=ROOT)
    out = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, out
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, out
