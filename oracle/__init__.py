"""CPU oracle of the FGP step on the 3D total-variation dual.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the GPU library ``stencil_dual_update_amd`` and never imports it.

The arithmetic lives in ``tv_fgp_oracle.c`` (plain C loops, compiled without
multiply-add contraction); this module only moves numpy arrays in and out.
It follows the page "TV solver: the FGP step on the GPU", section "What one
step does".  ``brute.py`` holds an independent fp64 brute force that builds
the forward-difference operator as an explicit matrix.

Array convention: a volume is a C-contiguous numpy array of shape
(nz, ny, nx), so x is the fastest index; a vector field is an array of shape
(3, nz, ny, nx) whose component 0 is along x, 1 along y and 2 along z.
"""
import ctypes
import os

import numpy as np

from .build_oracle import LIB as _LIB_PATH, build as _build

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        _build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.tv_oracle_momentum.restype = ctypes.c_double
    lib.tv_oracle_momentum.argtypes = [ctypes.c_int]
    lib.tv_oracle_set_threads.argtypes = [ctypes.c_int]
    lib.tv_oracle_get_threads.restype = ctypes.c_int
    for suf, real in (("f32", ctypes.c_float), ("f64", ctypes.c_double)):
        f = getattr(lib, "tv_oracle_run_" + suf)
        f.restype = ctypes.c_int
        f.argtypes = [P] * 7 + [real, ctypes.c_int, ctypes.c_int, I64, I64, I64]
        f = getattr(lib, "tv_oracle_step_" + suf)
        f.restype = ctypes.c_int
        f.argtypes = [P] * 10 + [real, real, I64, I64, I64]
        f = getattr(lib, "tv_oracle_adjoint_" + suf)
        f.restype = None
        f.argtypes = [P] * 4 + [I64, I64, I64]
        f = getattr(lib, "tv_oracle_gradient_" + suf)
        f.restype = None
        f.argtypes = [P] * 4 + [I64, I64, I64]
        f = getattr(lib, "tv_oracle_primal_readout_" + suf)
        f.restype = None
        f.argtypes = [P] * 4 + [real, P, I64, I64, I64]
        f = getattr(lib, "tv_oracle_duality_gap_" + suf)
        f.restype = ctypes.c_int
        f.argtypes = [P] * 4 + [real, I64, I64, I64, P]
    lib.tv_oracle_f16_to_f32.restype = ctypes.c_float
    lib.tv_oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.tv_oracle_f32_to_f16.restype = ctypes.c_uint16
    lib.tv_oracle_f32_to_f16.argtypes = [ctypes.c_float]
    lib.tv_oracle_f32_to_f16_array.restype = None
    lib.tv_oracle_f32_to_f16_array.argtypes = [P, P, I64]
    lib.tv_oracle_f16_to_f32_array.restype = None
    lib.tv_oracle_f16_to_f32_array.argtypes = [P, P, I64]
    lib.tv_oracle_run_h.restype = ctypes.c_int
    lib.tv_oracle_run_h.argtypes = [P] * 7 + [ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                               I64, I64, I64]
    _lib = lib
    return lib


def _suffix(dtype):
    dtype = np.dtype(dtype)
    if dtype == np.float32:
        return "f32", ctypes.c_float
    if dtype == np.float64:
        return "f64", ctypes.c_double
    raise TypeError("oracle runs in float32 or float64, not %s" % dtype)


def _ptr(a):
    assert a.flags.c_contiguous
    return ctypes.c_void_p(a.ctypes.data)


def _dims(vol):
    nz, ny, nx = vol.shape
    return nx, ny, nz


def set_threads(n):
    """Number of OpenMP threads the oracle uses (results do not depend on it)."""
    _load().tv_oracle_set_threads(int(n))


def get_threads():
    return int(_load().tv_oracle_get_threads())


def momentum(k):
    """m_k of the k-th step of an outer iteration, in double (k >= 1)."""
    return float(_load().tv_oracle_momentum(int(k)))


def momentum_f32(k):
    """m_k rounded once to float32."""
    return np.float32(momentum(k))


def adjoint(r):
    """L(r)(j) = sum_a r_a(j) - r_a(j - e_a), zero below the lower faces."""
    r = np.ascontiguousarray(r)
    suf, _ = _suffix(r.dtype)
    out = np.empty(r.shape[1:], dtype=r.dtype)
    getattr(_load(), "tv_oracle_adjoint_" + suf)(
        _ptr(r[0]), _ptr(r[1]), _ptr(r[2]), _ptr(out), *_dims(out))
    return out


def gradient(z):
    """g_a(i) = z(i) - z(i + e_a), zero at the upper a-face."""
    z = np.ascontiguousarray(z)
    suf, _ = _suffix(z.dtype)
    g = np.empty((3,) + z.shape, dtype=z.dtype)
    getattr(_load(), "tv_oracle_gradient_" + suf)(
        _ptr(z), _ptr(g[0]), _ptr(g[1]), _ptr(g[2]), *_dims(z))
    return g


def primal(b, p, lam):
    """z = max(b - lam*L(p), 0)."""
    b = np.ascontiguousarray(b)
    p = np.ascontiguousarray(p, dtype=b.dtype)
    suf, real = _suffix(b.dtype)
    z = np.empty_like(b)
    getattr(_load(), "tv_oracle_primal_readout_" + suf)(
        _ptr(b), _ptr(p[0]), _ptr(p[1]), _ptr(p[2]), real(lam), _ptr(z),
        *_dims(b))
    return z


def duality_gap(b, p, lam):
    """(G, TV(z), 1/2||z - b||^2) for z = max(b - lam L(p), 0), G in per-voxel form.

    G = lam * sum_i (|g(i)| - g(i).p(i)) with g = D z; see tv_fgp_oracle_body.h
    for why this equals the primal-dual gap P(z) - d(p).  z and g in b's
    precision, per-voxel terms and sums in double.
    """
    b = np.ascontiguousarray(b)
    suf, real = _suffix(b.dtype)
    p = np.ascontiguousarray(p, dtype=b.dtype)
    out = np.zeros(3, dtype=np.float64)
    rc = getattr(_load(), "tv_oracle_duality_gap_" + suf)(
        _ptr(b), _ptr(p[0]), _ptr(p[1]), _ptr(p[2]), real(lam), *_dims(b), _ptr(out))
    if rc != 0:
        raise MemoryError("oracle duality gap could not allocate scratch")
    return float(out[0]), float(out[1]), float(out[2])


def step(b, p, r, lam, m):
    """One FGP step with momentum coefficient m.  Returns (p_new, r_new)."""
    b = np.ascontiguousarray(b)
    suf, real = _suffix(b.dtype)
    p = np.array(p, dtype=b.dtype, copy=True, order="C")
    r = np.ascontiguousarray(r, dtype=b.dtype)
    rn = np.empty_like(r)
    rc = getattr(_load(), "tv_oracle_step_" + suf)(
        _ptr(b), _ptr(p[0]), _ptr(p[1]), _ptr(p[2]),
        _ptr(r[0]), _ptr(r[1]), _ptr(r[2]),
        _ptr(rn[0]), _ptr(rn[1]), _ptr(rn[2]),
        real(lam), real(m), *_dims(b))
    if rc != 0:
        raise MemoryError("oracle step could not allocate scratch")
    return p, rn


def run(b, p0, r0, lam, n_outer, n_inner, dtype=None):
    """n_outer outer iterations of n_inner FGP steps from (p0, r0).

    The momentum restarts at every outer iteration; p and r carry over.
    Returns copies (p, r) in ``dtype`` (default: b's dtype).
    """
    dtype = np.dtype(dtype or b.dtype)
    suf, real = _suffix(dtype)
    b = np.ascontiguousarray(b, dtype=dtype)
    p = np.array(p0, dtype=dtype, copy=True, order="C")
    r = np.array(r0, dtype=dtype, copy=True, order="C")
    assert p.shape == (3,) + b.shape and r.shape == p.shape
    rc = getattr(_load(), "tv_oracle_run_" + suf)(
        _ptr(b), _ptr(p[0]), _ptr(p[1]), _ptr(p[2]),
        _ptr(r[0]), _ptr(r[1]), _ptr(r[2]),
        real(lam), int(n_outer), int(n_inner), *_dims(b))
    if rc != 0:
        raise MemoryError("oracle run could not allocate scratch")
    return p, r


def f32_to_f16_bits(v):
    """binary16 bit patterns of float32 values (nearest, ties to even), same shape."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().tv_oracle_f32_to_f16_array(_ptr(v), _ptr(out), v.size)
    return out


def f16_bits_to_f32(h):
    """float32 values of binary16 bit patterns (exact), same shape."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    _load().tv_oracle_f16_to_f32_array(_ptr(h), _ptr(out), h.size)
    return out


def run_half(b, p0_bits, r0_bits, lam, n_outer, n_inner):
    """FGP with p and r stored as binary16 (uint16 bit patterns, (3, nz, ny, nx)).

    b is float32; arithmetic is float32; p and r are rounded to binary16 after
    every step.  Returns (p_bits, r_bits) copies.
    """
    b = np.ascontiguousarray(b, dtype=np.float32)
    p = np.array(p0_bits, dtype=np.uint16, copy=True, order="C")
    r = np.array(r0_bits, dtype=np.uint16, copy=True, order="C")
    assert p.shape == (3,) + b.shape and r.shape == p.shape
    rc = _load().tv_oracle_run_h(
        _ptr(b), _ptr(p[0]), _ptr(p[1]), _ptr(p[2]), _ptr(r[0]), _ptr(r[1]), _ptr(r[2]),
        float(lam), int(n_outer), int(n_inner), *_dims(b))
    if rc != 0:
        raise MemoryError("oracle half run could not allocate scratch")
    return p, r


def run_cone(b, p0, r0, lam, n_outer, n_inner, centre, radius=None):
    """Oracle result at one voxel of a large volume, from a sub-box around it.

    One FGP step makes r(i) depend on r at offsets of at most one voxel per
    axis (z at i and i + e_a, each from r at the voxel and its lower
    neighbours), so after K steps the value at a voxel depends only on the
    inputs within K voxels of it along each axis.  The sub-box is cut out to
    ``radius`` (default K + 1) voxels around ``centre`` and clipped at the
    true faces, where the boundary rule is the real one; at a cut face the
    artificial boundary reaches at most K voxels inward, so the centre is
    exact.  Returns (p[:, c], r[:, c], z_readout[c]) at the centre voxel.
    """
    nz, ny, nx = b.shape
    k = n_outer * n_inner
    rad = k + 1 if radius is None else radius
    cz, cy, cx = centre
    lo = (max(cz - rad, 0), max(cy - rad, 0), max(cx - rad, 0))
    hi = (min(cz + rad + 1, nz), min(cy + rad + 1, ny), min(cx + rad + 1, nx))
    sl = tuple(slice(a, e) for a, e in zip(lo, hi))
    bs = np.ascontiguousarray(b[sl])
    ps = np.ascontiguousarray(p0[(slice(None),) + sl])
    rs = np.ascontiguousarray(r0[(slice(None),) + sl])
    p, r = run(bs, ps, rs, lam, n_outer, n_inner)
    z = primal(bs, p, lam)
    loc = (cz - lo[0], cy - lo[1], cx - lo[2])
    return p[(slice(None),) + loc], r[(slice(None),) + loc], z[loc]
