"""Seeded synthetic inputs for the FGP step: the volume b and the initial dual.

This module only draws random numbers and shapes them into volumes.  It holds
none of the method's arithmetic, and both the CPU oracle (in the tests) and the
GPU path take its arrays as plain inputs.

The page measures on a phantom of its own that is not available here; these
recipes stand in for it.  Five workloads are defined, from a small case the
oracle finishes in seconds to 512^3 and a non-power-of-two anisotropic volume:

  idx  dims (nx, ny, nz)  steps    lambda  b
  0    32 x 32 x 32       1 x 10   0.01    3 Gaussian blobs + N(0, 0.005)
  1    128^3              20 x 10  0.005   8 Gaussian blobs + N(0, 0.005)
  2    256^3              20 x 10  0.002   12 ellipsoids + N(0, 0.002)
  3    512^3              20 x 10  0.002   24 ellipsoids + N(0, 0.002)
  4    1000 x 777 x 301   20 x 10  0.003   U[0, 0.03] per voxel + 16 ellipsoids

Readings of the recipe where it leaves details open:
  - Gaussian blob: A * exp(-d^2 / (2 sigma^2)), A ~ U[0, 0.05], sigma in voxels,
    centre ~ U[0, n_a) per axis.
  - Ellipsoid: axis-aligned, centre ~ U[0.2 n_a, 0.8 n_a], semi-axes
    ~ U[0.05 n_a, 0.25 n_a], value offset ~ U[0, 0.02] added inside
    (offsets add up where ellipsoids overlap), zero background.
  - Noise parameter = standard deviation.
  - Workload 4: p starts as random vectors of norm <= 1 (uniform in the unit
    ball), with the component slots on each upper face set to zero, and
    r = p.  All other workloads start from p = r = 0.
  - Generator: numpy PCG64 seeded with the workload index; b is built in
    float64 and rounded once to float32.

Arrays are C-ordered with shape (nz, ny, nx), so x is the fastest index;
vector fields have shape (3, nz, ny, nx).
"""
import numpy as np

WORKLOADS = {
    0: dict(dims=(32, 32, 32), n_outer=1, n_inner=10, lam=0.01,
            kind="blobs", n_obj=3, sigma=(2.0, 6.0), noise=0.005, init="zero"),
    1: dict(dims=(128, 128, 128), n_outer=20, n_inner=10, lam=0.005,
            kind="blobs", n_obj=8, sigma=(4.0, 20.0), noise=0.005, init="zero"),
    2: dict(dims=(256, 256, 256), n_outer=20, n_inner=10, lam=0.002,
            kind="ellipsoids", n_obj=12, noise=0.002, init="zero"),
    3: dict(dims=(512, 512, 512), n_outer=20, n_inner=10, lam=0.002,
            kind="ellipsoids", n_obj=24, noise=0.002, init="zero"),
    4: dict(dims=(1000, 777, 301), n_outer=20, n_inner=10, lam=0.003,
            kind="uniform_ellipsoids", n_obj=16, noise=0.0, init="ball"),
}

BASE_NAMES = {
    0: "blobs 32^3",
    1: "blobs 128^3",
    2: "ellipsoids 256^3",
    3: "ellipsoids 512^3",
    4: "uniform+ellipsoids 1000x777x301",
}

NAMES = {
    0: "blobs 32^3, 10 steps",
    1: "blobs 128^3, 20x10 steps",
    2: "ellipsoids 256^3, 20x10 steps",
    3: "ellipsoids 512^3, 20x10 steps",
    4: "uniform+ellipsoids 1000x777x301, 20x10 steps",
}

_BLOB_AMP = (0.0, 0.05)
_ELL_OFFSET = (0.0, 0.02)
_UNIFORM = (0.0, 0.03)
_SLAB = 16  # planes drawn per chunk for the initial dual (fixes the draw order)


def workload(idx):
    """The recipe of workload ``idx`` (a copy)."""
    return dict(WORKLOADS[idx])


def _blobs(rng, dims, n_obj, sigma_rng):
    nx, ny, nz = dims
    out = np.zeros((nz, ny, nx))
    axes = [np.arange(n, dtype=np.float64) for n in (nx, ny, nz)]
    for _ in range(n_obj):
        amp = rng.uniform(*_BLOB_AMP)
        sigma = rng.uniform(*sigma_rng)
        centre = [rng.uniform(0.0, n) for n in (nx, ny, nz)]
        gx, gy, gz = [np.exp(-((ax - c) ** 2) / (2.0 * sigma * sigma))
                      for ax, c in zip(axes, centre)]
        out += amp * gz[:, None, None] * gy[None, :, None] * gx[None, None, :]
    return out


def _ellipsoids(rng, dims, n_obj, out):
    nx, ny, nz = dims
    for _ in range(n_obj):
        centre = [rng.uniform(0.2 * n, 0.8 * n) for n in (nx, ny, nz)]
        semi = [rng.uniform(0.05 * n, 0.25 * n) for n in (nx, ny, nz)]
        value = rng.uniform(*_ELL_OFFSET)
        lo = [max(int(np.floor(c - s)), 0) for c, s in zip(centre, semi)]
        hi = [min(int(np.ceil(c + s)) + 1, n) for c, s, n in
              zip(centre, semi, (nx, ny, nz))]
        ex, ey, ez = [((np.arange(l, h, dtype=np.float64) - c) / s) ** 2
                      for l, h, c, s in zip(lo, hi, centre, semi)]
        inside = (ez[:, None, None] + ey[None, :, None] + ex[None, None, :]) <= 1.0
        out[lo[2]:hi[2], lo[1]:hi[1], lo[0]:hi[0]] += value * inside
    return out


def make_b(idx, dims=None):
    """float32 volume b of workload ``idx``, optionally at other dims (nx, ny, nz)."""
    w = WORKLOADS[idx]
    dims = tuple(dims or w["dims"])
    nx, ny, nz = dims
    rng = np.random.Generator(np.random.PCG64(idx))
    if w["kind"] == "blobs":
        vol = _blobs(rng, dims, w["n_obj"], w["sigma"])
    elif w["kind"] == "ellipsoids":
        vol = _ellipsoids(rng, dims, w["n_obj"], np.zeros((nz, ny, nx)))
    elif w["kind"] == "uniform_ellipsoids":
        vol = rng.uniform(*_UNIFORM, size=(nz, ny, nx))
        vol = _ellipsoids(rng, dims, w["n_obj"], vol)
    else:
        raise ValueError(w["kind"])
    if w["noise"] > 0.0:
        vol += rng.normal(0.0, w["noise"], size=(nz, ny, nx))
    return vol.astype(np.float32)


def random_ball_field(dims, seed):
    """float32 (3, nz, ny, nx) field of vectors uniform in the unit ball.

    Direction from a normalised Gaussian 3-vector, radius U[0,1]^(1/3) kept
    below 1 - 1e-5 so float32 rounding cannot push the norm past 1.  Drawn
    and shaped in float32.  The slot of component a on the upper a-face is
    set to zero.
    """
    nx, ny, nz = dims
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.empty((3, nz, ny, nx), dtype=np.float32)
    for z0 in range(0, nz, _SLAB):
        z1 = min(z0 + _SLAB, nz)
        g = rng.standard_normal(size=(3, z1 - z0, ny, nx), dtype=np.float32)
        rad = rng.random(size=(z1 - z0, ny, nx), dtype=np.float32) ** np.float32(1.0 / 3.0)
        rad = np.minimum(rad, np.float32(1.0 - 1e-5))
        length = np.sqrt((g * g).sum(axis=0))
        length[length == 0.0] = 1.0
        out[:, z0:z1] = g * (rad / length)
    out[0, :, :, nx - 1] = 0.0
    out[1, :, ny - 1, :] = 0.0
    out[2, nz - 1, :, :] = 0.0
    return out


def make_uniform(dims, seed, lo, hi):
    """float32 volume (nz, ny, nx) of independent U[lo, hi) draws, drawn in float32."""
    nx, ny, nz = dims
    rng = np.random.Generator(np.random.PCG64(seed))
    out = np.empty((nz, ny, nx), dtype=np.float32)
    for z0 in range(0, nz, _SLAB):
        z1 = min(z0 + _SLAB, nz)
        out[z0:z1] = rng.random(size=(z1 - z0, ny, nx), dtype=np.float32)
    out *= np.float32(hi - lo)
    out += np.float32(lo)
    return out


def make_p0(idx, dims=None):
    """Initial dual p of workload ``idx`` (float32, (3, nz, ny, nx)); r starts equal."""
    w = WORKLOADS[idx]
    dims = tuple(dims or w["dims"])
    nx, ny, nz = dims
    if w["init"] == "zero":
        return np.zeros((3, nz, ny, nx), dtype=np.float32)
    return random_ball_field(dims, seed=1000 + idx)


def make_inputs(idx, dims=None):
    """(b, p0, r0) of workload ``idx``; r0 is a copy of p0."""
    b = make_b(idx, dims)
    p0 = make_p0(idx, dims)
    return b, p0, p0.copy()
