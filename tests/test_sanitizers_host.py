"""The CPU oracle and the kernel sources under the host sanitizers (no GPU).

- AddressSanitizer + UndefinedBehaviorSanitizer on the oracle
  (oracle/tv_fgp_oracle.c) through tests/sanitize/oracle_driver.c, which calls
  every oracle entry point on small ragged volumes in buffers sized exactly.
- The same two sanitizers on the kernel headers compiled as host C++
  (tests/kernel_bounds/emul.cpp, every thread of every workgroup run in turn)
  on ragged shapes with the 32- and 64-bit index paths: UBSan flags any
  signed overflow or invalid shift in the index arithmetic that the guard
  pages of the plain bounds check cannot see.
- ThreadSanitizer on the threaded emulation (tests/kernel_bounds/func.cpp,
  one OS thread per GPU thread, the workgroup barrier a real one): a write to
  LDS that another thread reads without a barrier in between is reported as a
  data race, so this checks that every LDS exchange of the marching kernels is
  separated by the barriers it needs.

All three are plain host builds (gcc / clang++ of C and C++ sources; no GPU
code is built with a sanitizer).
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import phantoms

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
KB = os.path.join(HERE, "kernel_bounds")
CSRC = os.path.join(ROOT, "stencil_dual_update_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def cxx():
    for c in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++")):
        if c and os.path.exists(c):
            return c
    pytest.skip("no clang++")


def run_env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["TSAN_OPTIONS"] = "halt_on_error=1:second_deadlock_stack=1"
    return env


def test_oracle_under_asan_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("no gcc")
    exe = str(tmp_path / "oracle_driver")
    cmd = [gcc, "-std=c11", "-O1", "-g", "-ffp-contract=off"] + SAN + [
        os.path.join(ROOT, "oracle", "tv_fgp_oracle.c"),
        os.path.join(HERE, "sanitize", "oracle_driver.c"), "-lm", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=run_env())
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr[-3000:]


@pytest.fixture(scope="module")
def emul_san(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("emul_san") / "emul")
    cmd = [cxx(), "-std=c++17", "-O1", "-g"] + SAN + [
        "-I", os.path.join(KB, "shim"), "-I", CSRC, "-I", os.path.join(ROOT, "include"),
        os.path.join(KB, "emul.cpp"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


EMUL_VARIANTS = ["fused", "fused_h", "pair", "pair_h", "reg_march", "point", "two_kernel",
                 "lds_march", "lds_march_32x8", "primal", "gap", "gap_pair", "tb2", "tb2_h",
                 "tb3", "tb3_h", "cube", "cube_8x8x8"]


@pytest.mark.parametrize("variant", EMUL_VARIANTS)
def test_kernel_sources_under_asan_ubsan(emul_san, variant):
    failures = []
    for nx, ny, nz in [(1, 1, 1), (67, 9, 5), (130, 3, 4), (2, 11, 3), (140, 27, 20)]:
        for wide in (0, 1):
            planes = 8 if not variant.startswith("tb2") else 16
            args = [emul_san, variant, str(nx), str(ny), str(nz), str(wide), "0", "1",
                    str(planes)]
            r = subprocess.run(args, capture_output=True, text=True, timeout=600, env=run_env())
            if r.returncode != 0 or not r.stdout.startswith("ok"):
                failures.append((" ".join(args[1:]), r.returncode, r.stderr[-1500:]))
    assert not failures, failures


@pytest.fixture(scope="module")
def func_tsan(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("func_tsan") / "func")
    cmd = [cxx(), "-std=c++17", "-O1", "-g", "-fsanitize=thread", "-ffp-contract=off",
           "-pthread", "-DTVFGP_EMUL_THREADS", "-I", os.path.join(KB, "shim"), "-I", CSRC,
           "-I", os.path.join(ROOT, "include"), os.path.join(KB, "func.cpp"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


@pytest.mark.parametrize("kernel,dims", [
    ("fused", (70, 9, 6)), ("lds_march", (66, 5, 9)), ("lds_march_32x8", (40, 9, 6)),
    ("cube", (17, 9, 5)), ("pair", (130, 9, 6)), ("gap_pair", (130, 9, 6)), ("gap", (67, 9, 6)),
    ("tb2", (66, 10, 6)), ("tb3", (66, 10, 6)), ("tb3", (140, 27, 6))],
    ids=lambda c: str(c))
def test_lds_exchanges_race_free_under_tsan(func_tsan, tmp_path, kernel, dims):
    nx, ny, nz = dims
    b, p0, _ = phantoms.make_inputs(4, dims)
    r0 = (p0 + np.float32(0.2)).astype(np.float32)
    d = str(tmp_path)
    b.tofile(os.path.join(d, "b.bin"))
    p0.tofile(os.path.join(d, "p.bin"))
    r0.tofile(os.path.join(d, "r.bin"))
    args = [func_tsan, kernel, str(nx), str(ny), str(nz), "0.003", "0.3", "0.6", d, "0", "0",
            "0", "0.7"]
    r = subprocess.run(args, capture_output=True, text=True, timeout=900, env=run_env())
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stderr[-4000:]
    assert "WARNING: ThreadSanitizer" not in r.stderr, r.stderr[-4000:]
