"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only):
the oracle (oracle/zs_oracle.c) and the host step (csrc/zs_host.cpp), each
built with gcc/g++ together with a driver in tests/sanitize/ that walks every
routine over exactly-sized buffers.  A stray access or an undefined
operation aborts the driver, which fails the test."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


def _build_and_run(cmd, exe, env=None):
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600,
                       env=dict(os.environ, **(env or {})))
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    return r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_is_clean_under_sanitizers():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_driver")
        out = _build_and_run(["gcc", "-std=c99", "-ffp-contract=off", *SAN, "-o", exe,
                              os.path.join(ROOT, "oracle", "zs_oracle.c"),
                              os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-lm"],
                             exe)
    assert "clean" in out


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_step_is_clean_under_sanitizers():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "host_driver")
        out = _build_and_run(["g++", "-std=c++17", "-fopenmp", "-ffp-contract=off", *SAN,
                              "-I", os.path.join(ROOT, "include"), "-o", exe,
                              os.path.join(ROOT, "sharded_mixed_precision_shard_amd", "csrc",
                                           "zs_host.cpp"),
                              os.path.join(ROOT, "tests", "sanitize", "host_driver.cpp")],
                             exe, env={"OMP_NUM_THREADS": "4"})
    assert "clean" in out
