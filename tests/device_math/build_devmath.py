"""Build libdevmath.so (the device-math test kernels) next to this file with
the library's own hipcc flags."""
import importlib.util
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
LIB = os.path.join(HERE, "libdevmath.so")


def build():
    spec = importlib.util.spec_from_file_location(
        "_tvfgp_build_lib", os.path.join(ROOT, "stencil_dual_update_amd", "build_lib.py"))
    bl = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bl)
    cmd = [bl.hipcc()] + bl.flags() + [os.path.join(HERE, "devmath.hip"), "-o", LIB + ".tmp"]
    res = subprocess.run(cmd, cwd=HERE, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed (exit %d)" % res.returncode)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build())
