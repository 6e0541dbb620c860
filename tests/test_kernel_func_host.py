"""CPU functional emulation of kernels that exchange data through LDS (no GPU).

tests/kernel_bounds/func.cpp compiles the kernel headers as host C++ with every
thread of a workgroup as an OS thread and a real barrier for __syncthreads(),
so the LDS rings and the barrier schedule are exercised as on the GPU.  The
arithmetic is IEEE binary32 without contraction on both sides, so the
emulated kernels must match the CPU oracle bit for bit.  This checks the
two-steps-per-pass kernel's pipeline (halo regions, ring slots, slab ends)
before any GPU run; the GPU parity tests then check the compiled code.
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
SRC = os.path.join(HERE, "kernel_bounds")
CSRC = os.path.join(ROOT, "stencil_dual_update_amd", "csrc")


def compiler():
    for c in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++")):
        if c and os.path.exists(c):
            return c
    pytest.skip("no clang++ (the kernels use clang vector extensions)")


@pytest.fixture(scope="module")
def func(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("kernel_func") / "func")
    cmd = [compiler(), "-std=c++17", "-O1", "-ffp-contract=off", "-pthread",
           "-DTVFGP_EMUL_THREADS", "-I", os.path.join(SRC, "shim"), "-I", CSRC, "-I",
           os.path.join(ROOT, "include"), os.path.join(SRC, "func.cpp"), "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


def emulate(func, tmp_path, kernel, b, p0, r0, lam, m1, m2, wide=0, grid=0, planes=0):
    nz, ny, nx = b.shape
    d = str(tmp_path)
    b.tofile(os.path.join(d, "b.bin"))
    p0.tofile(os.path.join(d, "p.bin"))
    r0.tofile(os.path.join(d, "r.bin"))
    r = subprocess.run([func, kernel, str(nx), str(ny), str(nz), repr(lam), repr(float(m1)),
                        repr(float(m2)), d, str(wide), str(grid), str(planes)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stderr
    pg = np.fromfile(os.path.join(d, "p_out.bin"), np.float32).reshape(p0.shape)
    rg = np.fromfile(os.path.join(d, "r_out.bin"), np.float32).reshape(p0.shape)
    return pg, rg


def inputs(dims, seed=7):
    b, p0, _ = phantoms.make_inputs(4, dims)
    rng = np.random.default_rng(seed)
    r0 = (p0 + 0.3 * rng.standard_normal(p0.shape)).astype(np.float32)
    return b, p0, r0


def assert_bits(got, exp, label):
    bad = np.count_nonzero(got.view(np.uint32) != exp.view(np.uint32))
    assert bad == 0, "%s: %d values differ" % (label, bad)


@pytest.mark.parametrize("dims", [(67, 19, 11), (65, 9, 6), (64, 8, 5), (1, 1, 1), (3, 17, 2)],
                         ids=lambda d: str(d))
def test_fused_one_step(func, tmp_path, dims):
    """The default kernel's single step equals the oracle's (tiles of 4 planes,
    ragged last tiles, a single voxel)."""
    b, p0, r0 = inputs(dims)
    pg, rg = emulate(func, tmp_path, "fused", b, p0, r0, 0.003, np.float32(0.4), 0.0)
    pe, re = oracle.step(b, p0, r0, 0.003, np.float32(0.4))
    assert_bits(pg, pe, "p")
    assert_bits(rg, re, "r")


@pytest.mark.parametrize("dims", [(130, 17, 11), (2, 1, 1), (128, 8, 8), (258, 9, 19), (4, 3, 2)],
                         ids=lambda d: str(d))
def test_pair_one_step(func, tmp_path, dims):
    """The two-voxels-per-lane kernel's single step equals the oracle's (8-plane
    tiles, ragged x, y and z tails)."""
    b, p0, r0 = inputs(dims)
    pg, rg = emulate(func, tmp_path, "pair", b, p0, r0, 0.003, np.float32(0.4), 0.0)
    pe, re = oracle.step(b, p0, r0, 0.003, np.float32(0.4))
    assert_bits(pg, pe, "p")
    assert_bits(rg, re, "r")


@pytest.mark.parametrize("dims", [(130, 17, 11), (2, 3, 9)], ids=lambda d: str(d))
def test_pair_one_step_binary16(func, tmp_path, dims):
    """The binary16 one-step kernel equals one step of the oracle's half mode."""
    b, p0, r0 = inputs(dims)
    ph, rh = oracle.f32_to_f16_bits(p0), oracle.f32_to_f16_bits(r0)
    pg, rg = emulate(func, tmp_path, "pair_h", b, oracle.f16_bits_to_f32(ph),
                     oracle.f16_bits_to_f32(rh), 0.003, np.float32(oracle.momentum(1)), 0.0)
    pe, re = oracle.run_half(b, ph, rh, 0.003, 1, 1)
    assert np.array_equal(oracle.f32_to_f16_bits(pg), pe)
    assert np.array_equal(oracle.f32_to_f16_bits(rg), re)


@pytest.mark.parametrize("kernel", ["cube", "cube_8x8x8", "lds_march"])
@pytest.mark.parametrize("dims", [(37, 19, 11), (16, 8, 4), (1, 1, 1), (70, 9, 19)],
                         ids=lambda d: str(d))
def test_lds_one_step(func, tmp_path, kernel, dims):
    b, p0, r0 = inputs(dims)
    pg, rg = emulate(func, tmp_path, kernel, b, p0, r0, 0.003, np.float32(0.4), 0.0)
    pe, re = oracle.step(b, p0, r0, 0.003, np.float32(0.4))
    assert_bits(pg, pe, "p")
    assert_bits(rg, re, "r")


@pytest.mark.parametrize("kernel,planes", [("lds_march_32x4", 32), ("lds_march_32x8", 2),
                                           ("lds_march_32x8", 8), ("lds_march_32x16", 16),
                                           ("lds_march_64x8", 8), ("lds_march", 16)],
                         ids=lambda c: str(c))
@pytest.mark.parametrize("dims", [(37, 19, 11), (70, 33, None), (1, 1, 1)], ids=lambda d: str(d))
def test_lds_march_shapes_one_step(func, tmp_path, kernel, planes, dims):
    """The marching kernel at the tile shapes of the page's sweep, one step
    against the oracle bit for bit (tiles and plane slabs ragged at the faces;
    nz None: one full slab of the shape's planes and a ragged one of 3)."""
    if dims[2] is None:
        dims = (dims[0], dims[1], planes + 3)
    b, p0, r0 = inputs(dims)
    pg, rg = emulate(func, tmp_path, kernel, b, p0, r0, 0.003, np.float32(0.4), 0.0,
                     planes=planes)
    pe, re = oracle.step(b, p0, r0, 0.003, np.float32(0.4))
    assert_bits(pg, pe, "p")
    assert_bits(rg, re, "r")


@pytest.mark.parametrize("kernel,dims,grid", [
    ("gap", (67, 19, 11), 0), ("gap", (130, 17, 9), 3), ("gap", (1, 1, 1), 0),
    ("gap_pair", (130, 17, 9), 0), ("gap_pair", (258, 9, 19), 5), ("gap_pair", (2, 1, 1), 0),
    ("gap_pair", (128, 8, 8), 0), ("gap_pair", (2, 11, 3), 0), ("gap_pair", (130, 9, 50), 0),
    ("gap_pair", (2, 3, 30), 2)], ids=lambda c: str(c))
def test_duality_gap(func, tmp_path, kernel, dims, grid):
    """The gap reduction's z exchange through LDS: sums within fp64 rounding of the oracle."""
    b, p0, r0 = inputs(dims)
    lam = 0.003
    d = str(tmp_path)
    nz, ny, nx = b.shape
    b.tofile(os.path.join(d, "b.bin"))
    p0.tofile(os.path.join(d, "p.bin"))
    r0.tofile(os.path.join(d, "r.bin"))
    r = subprocess.run([func, kernel, str(nx), str(ny), str(nz), repr(lam), "0", "0", d, "0",
                        str(grid)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    got = np.fromfile(os.path.join(d, "gap.bin"), np.float64)
    g, tv, fid = oracle.duality_gap(b, p0, lam)
    assert abs(got[0] - g) <= 1e-10 * lam * tv
    assert abs(got[1] - tv) <= 1e-10 * tv
    assert abs(got[2] - fid) <= 1e-10 * max(fid, 1e-300)


# (dims, 64-bit path, forced grid, slab length; 0 = as launched): slab ends,
# ragged x/y tails, nz below one slab, one voxel, tiles looped over by a short
# grid, each slab length the launcher picks
CASES = [((65, 9, 17), 0, 0, 0), ((64, 8, 48), 1, 0, 16), ((130, 17, 33), 0, 3, 0),
         ((1, 1, 40), 0, 0, 32), ((5, 70, 3), 0, 0, 0), ((63, 7, 15), 0, 0, 0), ((1, 1, 1), 0, 0, 0),
         ((66, 10, 18), 1, 2, 16), ((64, 8, 70), 0, 0, 32),
         # tiles whose whole halo lies inside the volume: several slabs, a
         # short grid, the 64-bit path, a shallow z
         ((140, 27, 20), 0, 0, 8), ((140, 27, 40), 1, 5, 16), ((140, 20, 2), 0, 0, 0)]


@pytest.mark.parametrize("dims,wide,grid,planes", CASES, ids=lambda c: str(c))
def test_two_steps_per_pass(func, tmp_path, dims, wide, grid, planes):
    b, p0, r0 = inputs(dims)
    m1, m2 = np.float32(0.3), np.float32(0.61)
    pg, rg = emulate(func, tmp_path, "tb2", b, p0, r0, 0.003, m1, m2, wide, grid, planes)
    pe, re = oracle.step(b, p0, r0, 0.003, m1)
    pe, re = oracle.step(b, pe, re, 0.003, m2)
    assert_bits(pg, pe, "p %s" % (dims,))
    assert_bits(rg, re, "r %s" % (dims,))


@pytest.mark.parametrize("dims,planes", [((65, 9, 17), 0), ((64, 8, 48), 16), ((5, 70, 3), 0),
                                         ((140, 20, 12), 8)],
                         ids=lambda c: str(c))
def test_two_steps_per_pass_binary16(func, tmp_path, dims, planes):
    """The binary16 two-step pass equals two steps of the oracle's half mode."""
    b, p0, r0 = inputs(dims)
    ph, rh = oracle.f32_to_f16_bits(p0), oracle.f32_to_f16_bits(r0)
    pg, rg = emulate(func, tmp_path, "tb2_h", b, oracle.f16_bits_to_f32(ph),
                     oracle.f16_bits_to_f32(rh), 0.003, np.float32(oracle.momentum(1)),
                     np.float32(oracle.momentum(2)), 0, 0, planes)
    pe, re = oracle.run_half(b, ph, rh, 0.003, 1, 2)
    assert np.array_equal(oracle.f32_to_f16_bits(pg), pe)
    assert np.array_equal(oracle.f32_to_f16_bits(rg), re)


# (dims, 64-bit path, forced grid, slab length; 0 = as launched) for the
# three-steps-per-pass kernel: slab ends, ragged tails, nz below a slab, one
# voxel, tiles looped over by a short grid, each slab length the launcher picks
# (dims, wide, grid, planes); the shapes from (140, 27, 20) on hold tiles
# whose whole halo lies inside the volume (the kernel's interior path, whose
# loads are unconditional and clamp their planes): fewer planes than the
# pipeline's depth, a long slab, several slabs over a short grid
CASES3 = [((65, 9, 17), 0, 0, 0), ((64, 8, 48), 1, 0, 16), ((130, 17, 33), 0, 3, 0),
          ((1, 1, 40), 0, 0, 32), ((5, 70, 3), 0, 0, 0), ((63, 7, 15), 0, 0, 8), ((1, 1, 1), 0, 0, 0),
          ((66, 10, 18), 1, 2, 16), ((64, 8, 200), 0, 0, 96), ((70, 13, 9), 0, 0, 8),
          ((140, 27, 20), 0, 0, 8), ((200, 20, 12), 1, 3, 8), ((140, 20, 3), 0, 0, 0),
          ((132, 20, 100), 0, 0, 96), ((140, 27, 40), 1, 5, 16)]


def emulate3(func, tmp_path, kernel, b, p0, r0, lam, m, wide=0, grid=0, planes=0):
    nz, ny, nx = b.shape
    d = str(tmp_path)
    b.tofile(os.path.join(d, "b.bin"))
    p0.tofile(os.path.join(d, "p.bin"))
    r0.tofile(os.path.join(d, "r.bin"))
    r = subprocess.run([func, kernel, str(nx), str(ny), str(nz), repr(lam), repr(float(m[0])),
                        repr(float(m[1])), d, str(wide), str(grid), str(planes), repr(float(m[2]))],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stderr
    pg = np.fromfile(os.path.join(d, "p_out.bin"), np.float32).reshape(p0.shape)
    rg = np.fromfile(os.path.join(d, "r_out.bin"), np.float32).reshape(p0.shape)
    return pg, rg


@pytest.mark.parametrize("dims,wide,grid,planes", CASES3, ids=lambda c: str(c))
def test_three_steps_per_pass(func, tmp_path, dims, wide, grid, planes):
    b, p0, r0 = inputs(dims)
    m = (np.float32(0.3), np.float32(0.61), np.float32(0.7))
    pg, rg = emulate3(func, tmp_path, "tb3", b, p0, r0, 0.003, m, wide, grid, planes)
    pe, re = oracle.step(b, p0, r0, 0.003, m[0])
    pe, re = oracle.step(b, pe, re, 0.003, m[1])
    pe, re = oracle.step(b, pe, re, 0.003, m[2])
    assert_bits(pg, pe, "p %s" % (dims,))
    assert_bits(rg, re, "r %s" % (dims,))


@pytest.mark.parametrize("dims,planes", [((65, 9, 17), 0), ((64, 8, 48), 16), ((5, 70, 3), 0),
                                         ((140, 20, 12), 8)],
                         ids=lambda c: str(c))
def test_three_steps_per_pass_binary16(func, tmp_path, dims, planes):
    """The binary16 instantiation equals three steps of the oracle's half mode."""
    b, p0, r0 = inputs(dims)
    ph, rh = oracle.f32_to_f16_bits(p0), oracle.f32_to_f16_bits(r0)
    m = [np.float32(oracle.momentum(k)) for k in (1, 2, 3)]
    pg, rg = emulate3(func, tmp_path, "tb3_h", b, oracle.f16_bits_to_f32(ph),
                      oracle.f16_bits_to_f32(rh), 0.003, m, 0, 0, planes)
    pe, re = oracle.run_half(b, ph, rh, 0.003, 1, 3)
    assert np.array_equal(oracle.f32_to_f16_bits(pg), pe)
    assert np.array_equal(oracle.f32_to_f16_bits(rg), re)


def slab_estimate(txy, nz, slots, c):
    """The three-step launcher's estimate of a pass with c-plane slabs, in
    plane steps: a tile of s planes takes s + 7; layers run one after another
    when one fills the slots, else side by side."""
    layers = (nz + c - 1) // c
    if txy >= slots:
        last = nz - (layers - 1) * c
        return ((txy + slots - 1) // slots) * ((layers - 1) * (c + 7) + last + 7)
    return ((txy * layers + slots - 1) // slots) * (min(c, nz) + 7)


@pytest.mark.parametrize("dims,slots,want", [
    ((512, 512, 512), 512, 96), ((1000, 777, 301), 512, 96), ((768, 768, 768), 512, 96),
    ((448, 448, 448), 512, 96), ((512, 512, 70), 512, 96), ((384, 384, 384), 512, 32),
    ((320, 320, 320), 512, 64), ((256, 256, 256), 512, 64), ((192, 192, 192), 512, 32),
    ((128, 128, 128), 512, 8), ((32, 32, 32), 512, 8), ((256, 256, 256), 160, 32),
    ((512, 512, 512), 160, 96), ((64, 8, 200), 512, 8)], ids=lambda c: str(c))
def test_three_step_slab_length(func, dims, slots, want):
    """tb3_planes takes, of 96, 64, 32, 16 and 8 planes, the slab with the least
    estimated pass time (the longer on a tie); the expected values are the
    measured best where the two rules differed (256^3, 320^3, 384^3, 192^3 and
    the 512 x 512 x 70 shard)."""
    nx, ny, nz = dims
    r = subprocess.run([func, "slabs", str(nx), str(ny), str(nz), str(slots)],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    got = int(r.stdout.split()[0])
    txy = ((nx + 63) // 64) * ((ny + 7) // 8)
    best = min((96, 64, 32, 16, 8), key=lambda c: (slab_estimate(txy, nz, slots, c), -c))
    assert got == best == want
    # once one slab layer fills the chip, the longest slab is always taken
    if txy >= slots:
        assert got == 96
