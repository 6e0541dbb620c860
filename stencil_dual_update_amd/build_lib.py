"""Build the gfx950 shared library libtvfgp.so next to this file.

One hipcc invocation compiles the kernels and the C-ABI layer.  Flags:
  -ffp-contract=off        no fused multiply-add, so every variant and the
                           CPU reference round each operation the same way
  -Xclang -target-feature -Xclang -packed-fp32-ops
                           (with the leading minus) keeps the compiler from
                           emitting packed fp32 instructions
fp32 division and square root stay correctly rounded (hipcc's default); the
dual update's projection builds its own root and quotients from the same
instruction sequences (tv_fgp_device.hpp), which give the same bits.
"""
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libtvfgp.so")
ARCH = "gfx950"


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [
        os.path.join(CSRC, "tv_fgp_api.cpp")]


def flags():
    return [
        "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
        "-ffp-contract=off",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-command-line-argument",
        "-I", INCLUDE, "-I", CSRC,
    ]


def build(verbose=False, out=None, extra=()):
    out = out or LIB
    cmd = [hipcc()] + flags() + list(extra) + sources() + ["-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed (exit %d)" % res.returncode)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
