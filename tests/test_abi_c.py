"""The C ABI from a plain C program (no Python binding, no torch).

tests/abi_c/fgp_abi_c.c includes only include/tv_fgp.h and the HIP runtime
header, allocates device memory with hipMalloc and calls tv_fgp_run,
tv_primal and tv_fgp_duality_gap.  The CPU test checks that it compiles and
links against the built library; the GPU test runs it and compares p, r and z
with the CPU oracle bit for bit and the gap triple to fp64 summation error.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import phantoms

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIBDIR = os.path.join(ROOT, "stencil_dual_update_amd")
ROCM = "/opt/rocm"


def build(out):
    cc = shutil.which("gcc") or shutil.which("cc")
    if not cc or not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime_api.h")):
        pytest.skip("no C compiler or HIP headers")
    if not os.path.exists(os.path.join(LIBDIR, "libtvfgp.so")):
        pytest.fail("libtvfgp.so is not built")
    cmd = [cc, "-std=c11", "-O1", "-Wall", "-I", os.path.join(ROOT, "include"), "-I",
           os.path.join(ROCM, "include"), os.path.join(HERE, "abi_c", "fgp_abi_c.c"), "-o", out,
           "-L", LIBDIR, "-ltvfgp", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + LIBDIR + ":" + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


def test_c_program_builds(tmp_path):
    exe = build(str(tmp_path / "fgp_abi_c"))
    assert os.access(exe, os.X_OK)


@pytest.mark.gpu
@pytest.mark.parametrize("variant", [0, 6, 12], ids=["fused", "tb2", "tb3"])
def test_c_program_matches_oracle(tmp_path, variant):
    exe = build(str(tmp_path / "fgp_abi_c"))
    dims = (67, 45, 29)
    b, p0, r0 = phantoms.make_inputs(4, dims)
    d = str(tmp_path)
    b.tofile(os.path.join(d, "b.bin"))
    p0.tofile(os.path.join(d, "p.bin"))
    r0.tofile(os.path.join(d, "r.bin"))
    r = subprocess.run([exe, d, *map(str, dims), "0.003", "2", "5", str(variant)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
    pe, re = oracle.run(b, p0, r0, 0.003, 2, 5)
    ze = oracle.primal(b, pe, 0.003)
    for name, exp in (("p", pe), ("r", re), ("z", ze)):
        got = np.fromfile(os.path.join(d, name + "_out.bin"), np.float32).reshape(exp.shape)
        assert np.array_equal(got.view(np.uint32), exp.view(np.uint32)), name
    g, tv, fid = oracle.duality_gap(b, pe, 0.003)
    got = np.fromfile(os.path.join(d, "gap_out.bin"), np.float64)
    assert abs(got[0] - g) <= 1e-10 * 0.003 * tv, (got[0], g)
    assert abs(got[1] - tv) <= 1e-10 * tv, (got[1], tv)
    assert abs(got[2] - fid) <= 1e-10 * fid, (got[2], fid)
