"""Build the CPU oracle shared library (test infrastructure only).

Compiles tv_fgp_oracle.c with gcc: -O2, no fast-math, no multiply-add
contraction, OpenMP over the outer z loop.  The result is
oracle/libtvoracle.so next to this file.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libtvoracle.so")


def build(verbose=False):
    src = os.path.join(HERE, "tv_fgp_oracle.c")
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared",
        "-ffp-contract=off", "-fno-fast-math", "-fno-unsafe-math-optimizations",
        "-fexcess-precision=standard", "-fopenmp",
        "-Wall", "-Wextra",
        src, "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, cwd=HERE)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
