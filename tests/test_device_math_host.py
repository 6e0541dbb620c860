"""The dual update's correctly rounded square root and shared-reciprocal
quotients (tv_fgp_device.hpp), built for the CPU with estimates that may be
either faithful neighbour of the true value, against the host's IEEE sqrtf
and division (tests/device_math/seq.cpp; the GPU counterpart is
test_gpu_device_math.py)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
DM = os.path.join(HERE, "device_math")


def compiler():
    for c in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++")):
        if c and os.path.exists(c):
            return c
    pytest.skip("no clang++")


def test_sqrt_and_quotients_are_ieee(tmp_path):
    exe = str(tmp_path / "seq")
    subprocess.run([compiler(), "-std=c++17", "-O2", "-ffp-contract=off", "-I", DM,
                    "-I", os.path.join(HERE, "kernel_bounds", "shim"),
                    "-I", os.path.join(ROOT, "stencil_dual_update_amd", "csrc"),
                    "-I", os.path.join(ROOT, "include"), os.path.join(DM, "seq.cpp"), "-o", exe],
                   check=True, capture_output=True, text=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    lines = dict(l.split(" ", 1) for l in res.stdout.strip().splitlines())
    assert lines["sqrt"].startswith("0 of ")
    assert lines["div"].startswith("0 of ")
    assert lines["key"] == "0"
    # one Newton step from the lower estimate misses at the all-ones divisor
    # significand alone (the GPU test checks the hardware's result there)
    assert lines["recip"] == "rounded-estimate 0 (all-ones 0), other-estimate 0 (all-ones 1)"
