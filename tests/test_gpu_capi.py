"""The C ABI used from a plain C program (no Python, no torch in the step):
tests/capi/step_from_c.c is compiled with gcc against include/zs.h, linked to
libzs.so, the HIP runtime and the C oracle, and run on the GPU."""
import os
import subprocess
import tempfile

import pytest

import oracle
import sharded_mixed_precision_shard_amd as zs

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_step_from_c():
    lib_dir = os.path.dirname(zs.LIB_PATH)
    oracle_dir = os.path.dirname(os.path.abspath(oracle.__file__))
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "step_from_c")
        subprocess.run(["gcc", "-std=c11", "-O1", "-D__HIP_PLATFORM_AMD__",
                        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
                        "-o", exe, os.path.join(ROOT, "tests", "capi", "step_from_c.c"),
                        "-L", lib_dir, "-lzs", "-L", oracle_dir, "-lzs_oracle",
                        "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                        "-Wl,-rpath," + lib_dir, "-Wl,-rpath," + oracle_dir,
                        "-Wl,-rpath," + os.path.join(ROCM, "lib")],
                       check=True, capture_output=True, text=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "bitwise equal (separate and packed state, stochastic bf16 moments)" in r.stdout
