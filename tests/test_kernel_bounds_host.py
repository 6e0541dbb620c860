"""CPU bounds check of the HIP kernel sources (no GPU needed).

tests/kernel_bounds/emul.cpp compiles the kernel headers as host C++ (at -O0,
so every load written in the source is executed) and
runs every thread of every workgroup on buffers placed against inaccessible
guard regions: any access outside a buffer, including a wrapped 32-bit
offset, faults.  Each case runs with the buffers flush against the guard at
their end and at their start, with the 32-bit and the 64-bit index paths, and
with the launch grid as well as a 7-workgroup grid that forces the tile loop.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "kernel_bounds")
CSRC = os.path.join(ROOT, "stencil_dual_update_amd", "csrc")

SHAPES = [(67, 45, 29), (1, 1, 1), (1, 1, 9), (9, 1, 1), (1, 7, 1), (130, 3, 70), (65, 5, 17),
          (63, 3, 2), (2, 2, 2), (64, 8, 4), (64, 8, 5), (64, 4, 16), (128, 16, 8),
          (1100, 10, 7), (2100, 20, 5), (3, 300, 5), (200, 9, 33), (2, 1, 1), (258, 17, 6),
          (126, 9, 4), (66, 10, 40), (130, 17, 33)]
VARIANTS = ["fused", "fused_nostream", "fused_h", "fused_nostream_h", "pair", "pair_nostream",
            "pair_h", "pair_nostream_h", "reg_march", "point", "two_kernel", "lds_march", "lds_march_32x4", "lds_march_32x8",
            "lds_march_32x16", "lds_march_64x8", "primal",
            "primal_h", "gap", "gap_pair", "tb2", "tb2_h", "tb3", "tb3_h", "cube", "cube_32x8x2", "cube_64x8x1", "cube_8x8x8",
            "cube_32x4x4"]
# shapes with tiles whose whole two- or three-step halo lies inside the
# volume (the three-step kernel runs those on a copy of its march with the x
# and y boundary rules folded), from fewer planes than the pipeline's depth
# to several slabs
INTERIOR_SHAPES = [(140, 27, 20), (200, 20, 3), (132, 20, 100)]
FOUR_PLANE = ("tb2", "tb2_h", "cube", "cube_32x8x2", "cube_64x8x1", "cube_8x8x8", "cube_32x4x4", "fused", "fused_nostream", "fused_h", "fused_nostream_h", "pair", "pair_nostream",
              "pair_h", "pair_nostream_h", "point", "gap", "gap_pair")


def compiler():
    for c in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++"), shutil.which("g++")):
        if c and os.path.exists(c):
            return c
    pytest.skip("no C++ compiler")


@pytest.fixture(scope="module")
def emul(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("kernel_bounds") / "emul")
    cmd = [compiler(), "-std=c++17", "-O0", "-I", os.path.join(SRC, "shim"), "-I", CSRC,
           "-I", os.path.join(ROOT, "include"), os.path.join(SRC, "emul.cpp"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


@pytest.mark.parametrize("variant", VARIANTS)
def test_every_access_in_bounds(emul, variant):
    failures = []
    shapes = SHAPES + (INTERIOR_SHAPES if variant.startswith(("tb2", "tb3")) else [])
    for nx, ny, nz in shapes:
        for wide in (0, 1):
            for end in (0, 1):
                for grid in ((0, 7) if wide else (0,)):
                    for planes in ((8, 16, 32) if variant.startswith("tb2") else
                                   (8, 16, 32, 96) if variant.startswith("tb3") else
                                   (8, 3) if variant not in FOUR_PLANE else (4,)):
                        args = [emul, variant, str(nx), str(ny), str(nz), str(wide), str(grid),
                                str(end), str(planes)]
                        r = subprocess.run(args, capture_output=True, text=True, timeout=120)
                        if r.returncode != 0 or not r.stdout.startswith("ok"):
                            failures.append((" ".join(args[1:]), r.returncode))
    assert not failures, failures
