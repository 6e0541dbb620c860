"""Pins of the CPU oracle to facts outside itself (no GPU needed).

Each test fixes part of the oracle against mathematics or a closed form, not
against a retyped copy of its own formulas:
  - adjoint identity <L r, z> = <r, D z> (L is the adjoint of D),
  - an fp64 brute force that builds D as a matrix from index pairs,
  - closed-form fixed points (two voxels, a 1D step edge), the 1D reduction
    and an independent bounded least-squares solve of the 1D problem,
  - the large-lambda limit and the duality gap (weak duality and its zero at
    the optimum), feasibility |p| <= 1, zero and constant inputs,
  - axis permutation, thread-count independence and the FISTA momentum's
    closed form at k = 2 (the golden ratio).
"""
import numpy as np
import pytest

from conftest import read_golden
from oracle import brute

RNG = np.random.default_rng(20261202)


def rand_admissible(shape, rng, scale=1.0):
    """Random dual field with the upper-face slot of each component zeroed."""
    nz, ny, nx = shape
    r = rng.uniform(-scale, scale, size=(3,) + shape)
    r[0, :, :, nx - 1] = 0.0
    r[1, :, ny - 1, :] = 0.0
    r[2, nz - 1, :, :] = 0.0
    return r


def zeros_field(shape, dtype=np.float64):
    return np.zeros((3,) + shape, dtype=dtype)


# --------------------------------------------------------------------------
# momentum

def test_momentum_closed_forms(oracle_mod):
    # t_1 = 1 gives m_1 = 0 exactly.
    assert oracle_mod.momentum(1) == 0.0
    # t_2 = (1 + sqrt 5)/2 is the golden ratio phi; t_3 = (1 + sqrt(1 + 4 phi^2))/2
    # and phi^2 = phi + 1, so m_2 = (phi - 1) / ((1 + sqrt(5 + 4 phi)) / 2).
    phi = (1.0 + 5.0 ** 0.5) / 2.0
    m2 = (phi - 1.0) / ((1.0 + (5.0 + 4.0 * phi) ** 0.5) / 2.0)
    assert abs(oracle_mod.momentum(2) - m2) < 1e-15
    ms = [oracle_mod.momentum(k) for k in range(1, 400)]
    assert all(0.0 <= a < b < 1.0 for a, b in zip(ms[1:], ms[2:]))
    # t_k = (k + 1)/2 + O(log k), so m_k = 1 - 3/k + O(log k / k^2).
    for k in (100, 200, 399):
        assert abs(oracle_mod.momentum(k) - (1.0 - 3.0 / k)) < 3.0 * np.log(k) / k ** 2
    # the brute force carries its own implementation of the sequence
    for k in range(1, 30):
        assert abs(oracle_mod.momentum(k) - brute.fista_momentum(k)) < 1e-15


# --------------------------------------------------------------------------
# P1: adjoint identity

SHAPES = [(8, 8, 8), (3, 7, 5), (9, 1, 1), (1, 1, 1000), (1, 1, 2), (1, 3, 4), (2, 2, 2)]


@pytest.mark.parametrize("shape", SHAPES)
def test_adjoint_identity(oracle_mod, shape):
    z = RNG.standard_normal(shape)
    r = rand_admissible(shape, RNG)
    lr = oracle_mod.adjoint(r)
    dz = oracle_mod.gradient(z)
    lhs = float(np.dot(lr.ravel(), z.ravel()))
    rhs = float(np.dot(r.ravel(), dz.ravel()))
    assert abs(lhs - rhs) <= 1e-6 * max(abs(lhs), abs(rhs), 1e-300)
    assert abs(lhs - rhs) <= 1e-12 * (np.abs(lr).sum() + 1.0)


@pytest.mark.parametrize("shape", [(8, 8, 8), (3, 7, 5), (1, 3, 4)])
def test_adjoint_defect_is_upper_face_sum(oracle_mod, shape):
    """With nonzero upper-face slots, <Lr,z> - <r,Dz> is the upper-face sum."""
    nz, ny, nx = shape
    z = RNG.standard_normal(shape)
    r = RNG.standard_normal((3,) + shape)
    lhs = float(np.dot(oracle_mod.adjoint(r).ravel(), z.ravel()))
    rhs = float(np.dot(r.ravel(), oracle_mod.gradient(z).ravel()))
    face = (float((r[0, :, :, nx - 1] * z[:, :, nx - 1]).sum())
            + float((r[1, :, ny - 1, :] * z[:, ny - 1, :]).sum())
            + float((r[2, nz - 1] * z[nz - 1]).sum()))
    assert abs((lhs - rhs) - face) < 1e-12 * (abs(face) + 1.0) * r.size


def test_gradient_matches_matrix(oracle_mod):
    """The stencil D equals the matrix built from index pairs (5x7x3)."""
    shape = (3, 7, 5)
    z = RNG.standard_normal(shape)
    d = brute.difference_matrix(5, 7, 3)
    assert np.array_equal(oracle_mod.gradient(z).ravel(), d @ z.ravel())
    r = rand_admissible(shape, RNG)
    assert np.allclose(oracle_mod.adjoint(r).ravel(), d.T @ r.ravel(), rtol=0, atol=1e-15)


# --------------------------------------------------------------------------
# P5: brute force

BRUTE_CASES = [
    ((8, 8, 8), 0.02, 2, 5, "zero"),
    ((3, 7, 5), 0.01, 3, 4, "ball"),
    ((9, 1, 1), 0.05, 1, 12, "zero"),
    ((4, 1, 3), 0.03, 2, 6, "ball"),
    ((2, 2, 2), 0.01, 1, 10, "rand"),
]


@pytest.mark.parametrize("shape,lam,n_outer,n_inner,init", BRUTE_CASES)
def test_brute_force_fp64(oracle_mod, shape, lam, n_outer, n_inner, init):
    b = RNG.uniform(-0.02, 0.08, size=shape)
    if init == "zero":
        p0 = zeros_field(shape)
        r0 = p0.copy()
    elif init == "ball":
        p0 = rand_admissible(shape, RNG, scale=0.5)
        r0 = p0.copy()
    else:  # r differs from p (mid-run state)
        p0 = rand_admissible(shape, RNG, scale=0.5)
        r0 = rand_admissible(shape, RNG, scale=0.5)
    p, r = oracle_mod.run(b, p0, r0, lam, n_outer, n_inner, dtype=np.float64)
    z = oracle_mod.primal(b, p, lam)
    pb, rb, zb = brute.run(b, p0, r0, lam, n_outer, n_inner)
    assert np.max(np.abs(p - pb)) < 1e-12
    assert np.max(np.abs(r - rb)) < 1e-12
    assert np.max(np.abs(z - zb)) < 1e-13


def test_brute_force_fp32_close(oracle_mod):
    shape = (8, 8, 8)
    b = RNG.uniform(-0.02, 0.08, size=shape)
    p0 = zeros_field(shape)
    p32, r32 = oracle_mod.run(b.astype(np.float32), p0.astype(np.float32),
                              p0.astype(np.float32), 0.02, 2, 10)
    pb, rb, _ = brute.run(b.astype(np.float32).astype(np.float64), p0, p0, 0.02, 2, 10)
    assert p32.dtype == np.float32
    assert np.max(np.abs(p32 - pb)) < 2e-6
    assert np.max(np.abs(r32 - rb)) < 2e-6


# --------------------------------------------------------------------------
# P2 feasibility, P3 zero, P4 constant

@pytest.mark.parametrize("dtype,tol", [(np.float32, 5e-7), (np.float64, 1e-14)])
def test_feasibility_every_step(oracle_mod, dtype, tol):
    shape = (12, 10, 14)
    import phantoms
    b = phantoms.make_b(1, dims=(14, 10, 12)).astype(dtype)
    p = zeros_field(shape, dtype)
    r = p.copy()
    worst = 0.0
    active = 0
    for o in range(3):
        for k in range(1, 11):
            p, r = oracle_mod.step(b, p, r, 0.005, dtype(oracle_mod.momentum(k)))
            n = np.sqrt((p.astype(np.float64) ** 2).sum(axis=0))
            worst = max(worst, float(n.max()))
            active += int((n > 1.0 - 1e-6).sum())
    assert worst <= 1.0 + tol
    assert active > 0  # the projection was exercised
    # admissibility is preserved: the upper-face slots stay exactly zero
    nz, ny, nx = shape
    assert not p[0, :, :, nx - 1].any() and not r[0, :, :, nx - 1].any()
    assert not p[1, :, ny - 1, :].any() and not r[1, :, ny - 1, :].any()
    assert not p[2, nz - 1].any() and not r[2, nz - 1].any()


@pytest.mark.parametrize("dtype", [np.float32, np.float64])
def test_zero_input_stays_zero(oracle_mod, dtype):
    shape = (6, 5, 7)
    b = np.zeros(shape, dtype)
    p, r = oracle_mod.run(b, zeros_field(shape, dtype), zeros_field(shape, dtype), 0.01, 2, 10)
    assert not p.any() and not r.any()
    assert not np.signbit(p).any() and not np.signbit(r).any()
    assert not oracle_mod.primal(b, p, 0.01).any()


@pytest.mark.parametrize("c", [0.0, 0.037, 1.5, -0.2])
def test_constant_input(oracle_mod, c):
    shape = (5, 6, 4)
    b = np.full(shape, c, np.float32)
    p, r = oracle_mod.run(b, zeros_field(shape, np.float32), zeros_field(shape, np.float32), 0.01, 2, 10)
    assert not p.any() and not r.any()
    z = oracle_mod.primal(b, p, 0.01)
    assert np.array_equal(z, np.full(shape, max(c, 0.0), np.float32))


# --------------------------------------------------------------------------
# P6: two voxels, P7: 1D reduction and step edge, independent 1D solve

@pytest.mark.parametrize("axis", [0, 1, 2])
@pytest.mark.parametrize("row", read_golden("two_voxel.txt"))
def test_two_voxel_closed_form(oracle_mod, axis, row):
    _, lam, b0, b1, z0, z1, pk = row[0], *map(float, row[1:])
    shape = [1, 1, 1]
    shape[2 - axis] = 2  # axis 0 = x = last array axis
    b = np.array([b0, b1]).reshape(shape)
    p, r = oracle_mod.run(b, zeros_field(tuple(shape)), zeros_field(tuple(shape)), lam, 1, 400,
                          dtype=np.float64)
    z = oracle_mod.primal(b, p, lam).ravel()
    assert np.allclose(z, [z0, z1], atol=1e-12, rtol=0)
    comp = p[axis].ravel()
    assert abs(comp[0] - pk) < 1e-12 and comp[1] == 0.0
    others = [a for a in range(3) if a != axis]
    assert not p[others].any()


def _embed_1d(signal, axis, other=(3, 2)):
    """A volume that varies along ``axis`` only (0 = x, 1 = y, 2 = z)."""
    n = len(signal)
    shape = [other[0], other[1]]
    shape.insert(2 - axis, n)
    shape = tuple(shape)
    view = [1, 1, 1]
    view[2 - axis] = n
    return np.broadcast_to(np.asarray(signal).reshape(view), shape).copy()


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_1d_reduction_exact(oracle_mod, axis):
    sig = RNG.uniform(-0.01, 0.06, size=11).astype(np.float32)
    b = _embed_1d(sig, axis)
    p, r = oracle_mod.run(b, zeros_field(b.shape, np.float32), zeros_field(b.shape, np.float32),
                          0.01, 2, 25)
    others = [a for a in range(3) if a != axis]
    assert not p[others].any() and not r[others].any()
    z = oracle_mod.primal(b, p, 0.01)
    # z is the same along the two other axes, bit for bit
    moved = np.moveaxis(z, 2 - axis, 0).reshape(z.shape[2 - axis], -1)
    assert (moved == moved[:, :1]).all()


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_step_edge_closed_form(oracle_mod, axis):
    nl, nr, a, c, lam = read_golden("step_edge_1d.txt")[0]
    nl, nr, a, c, lam = int(nl), int(nr), float(a), float(c), float(lam)
    sig = np.array([a] * nl + [c] * nr)
    b = _embed_1d(sig, axis)
    p, _ = oracle_mod.run(b, zeros_field(b.shape), zeros_field(b.shape), lam, 1, 4000,
                          dtype=np.float64)
    z = oracle_mod.primal(b, p, lam)
    ax = 2 - axis
    zline = np.moveaxis(z, ax, 0)[:, 0, 0]
    pline = np.moveaxis(p[axis], ax, 0)[:, 0, 0]
    z_exp = np.array([a - lam / nl] * nl + [c + lam / nr] * nr)
    p_exp = np.array([(j + 1) / nl for j in range(nl)] + [1.0 - k / nr for k in range(1, nr + 1)])
    assert np.max(np.abs(zline - z_exp)) < 1e-10
    assert np.max(np.abs(pline - p_exp)) < 1e-8


def test_1d_against_bounded_least_squares(oracle_mod):
    """Converged 1D z equals max(prox_TV(f), 0), prox from a bounded LSQ dual."""
    from scipy.optimize import lsq_linear
    n, lam = 14, 0.03
    f = RNG.uniform(-0.05, 0.15, size=n)
    d1 = np.eye(n)[:-1] - np.eye(n)[1:]  # (n-1) x n differences
    # prox_{lam TV}(f) = f - D1^T u with u = argmin_{|u| <= lam} ||D1^T u - f||^2
    u = lsq_linear(d1.T, f, bounds=(-lam, lam), method="bvls", tol=1e-14).x
    z_ref = np.maximum(f - d1.T @ u, 0.0)
    b = _embed_1d(f, 0)
    p, _ = oracle_mod.run(b, zeros_field(b.shape), zeros_field(b.shape), lam, 1, 20000,
                          dtype=np.float64)
    z = oracle_mod.primal(b, p, lam)[0, 0, :]
    assert np.max(np.abs(z - z_ref)) < 1e-8


# --------------------------------------------------------------------------
# P8 large lambda, P9 duality gap

@pytest.mark.parametrize("lo,hi", [(0.0, 1.0), (-1.0, 0.5)])
def test_large_lambda_limit(oracle_mod, lo, hi):
    shape = (6, 6, 6)
    b = RNG.uniform(lo, hi, size=shape)
    p, _ = oracle_mod.run(b, zeros_field(shape), zeros_field(shape), 100.0, 1, 20000,
                          dtype=np.float64)
    z = oracle_mod.primal(b, p, 100.0)
    assert np.max(np.abs(z - max(b.mean(), 0.0))) < 1e-9


def duality_gap(b, p, lam):
    """P(z) - d(p) for z = max(b - lam D^T p, 0), D built from index pairs.

    Primal P(z) = 1/2||z - b||^2 + lam sum_i ||(Dz)(i)||_2 over z >= 0.
    Dual d(p) = min_{z >= 0} 1/2||z - b||^2 + lam <D^T p, z> = 1/2||b||^2 - 1/2||z||^2,
    attained at z = max(b - lam D^T p, 0).  For |p(i)| <= 1 weak duality gives
    P(z) >= d(p), with equality only at a primal-dual optimum.
    """
    nz, ny, nx = b.shape
    n = b.size
    d = brute.difference_matrix(nx, ny, nz)
    bv = b.ravel()
    z = np.maximum(bv - lam * (d.T @ p.ravel()), 0.0)
    dz = (d @ z).reshape(3, n)
    primal = 0.5 * np.sum((z - bv) ** 2) + lam * np.sum(np.sqrt((dz ** 2).sum(axis=0)))
    dual = 0.5 * np.sum(bv ** 2) - 0.5 * np.sum(z ** 2)
    return primal - dual


def test_duality_gap_closes(oracle_mod):
    import phantoms
    b = phantoms.make_b(0, dims=(8, 8, 8)).astype(np.float64) * 4.0
    shape = b.shape
    lam = 0.01
    gaps = []
    for k in (1, 10, 100, 1000):
        p, _ = oracle_mod.run(b, zeros_field(shape), zeros_field(shape), lam, 1, k,
                              dtype=np.float64)
        assert np.sqrt((p ** 2).sum(axis=0)).max() <= 1.0 + 1e-14
        gaps.append(duality_gap(b, p, lam))
    assert all(g >= -1e-14 for g in gaps)
    assert gaps[0] > gaps[1] > gaps[2] > gaps[3]
    assert gaps[3] < 1e-6 * gaps[0]


def test_duality_gap_detects_anisotropic_projection(oracle_mod):
    """Control: clipping each component to [-1,1] (anisotropic) leaves a gap."""
    import phantoms
    b = phantoms.make_b(0, dims=(8, 8, 8)).astype(np.float64) * 4.0
    lam = 0.01
    nz, ny, nx = b.shape
    d = brute.difference_matrix(nx, ny, nz)
    p = np.zeros(3 * b.size)
    r = p.copy()
    for k in range(1, 1001):
        m = brute.fista_momentum(k)
        z = np.maximum(b.ravel() - lam * (d.T @ r), 0.0)
        pn = np.clip(r + (d @ z) / (12 * lam), -1.0, 1.0)
        pn3 = pn.reshape(3, -1)
        scale = np.maximum(1.0, np.sqrt((pn3 ** 2).sum(axis=0)))
        r = pn + m * (pn - p)
        p = pn
    # project to the ball so weak duality applies, then measure the gap
    p_ok = (p.reshape(3, -1) / scale).reshape(3, nz, ny, nx)
    p_ref, _ = oracle_mod.run(b, zeros_field(b.shape), zeros_field(b.shape), lam, 1, 1000,
                              dtype=np.float64)
    assert duality_gap(b, p_ok, lam) > 100 * duality_gap(b, p_ref, lam)


# --------------------------------------------------------------------------
# P10 axis permutation, P11 threads, fp32 vs fp64, cone helper

def test_axis_permutation(oracle_mod):
    b = RNG.uniform(-0.01, 0.07, size=(5, 6, 7))  # (nz, ny, nx)
    p0 = rand_admissible(b.shape, RNG, scale=0.3)
    lam = 0.02
    p, r = oracle_mod.run(b, p0, p0, lam, 2, 5, dtype=np.float64)
    # swap x and z: array axes 0 and 2; component 0 <-> 2
    bt = np.ascontiguousarray(b.transpose(2, 1, 0))
    pt0 = np.ascontiguousarray(p0[[2, 1, 0]].transpose(0, 3, 2, 1))
    pt, rt = oracle_mod.run(bt, pt0, pt0, lam, 2, 5, dtype=np.float64)
    back = pt[[2, 1, 0]].transpose(0, 3, 2, 1)
    assert np.max(np.abs(back - p)) < 1e-13
    backr = rt[[2, 1, 0]].transpose(0, 3, 2, 1)
    assert np.max(np.abs(backr - r)) < 1e-13


def test_thread_count_independence(oracle_mod):
    """The loops split the z planes over threads on volumes of at least 2^15
    voxels; this one (47 x 37 x 23 = 40,000) is above that."""
    import phantoms
    b, p0, r0 = phantoms.make_inputs(4, dims=(47, 37, 23))
    assert b.size >= 1 << 15
    old = oracle_mod.get_threads()
    try:
        oracle_mod.set_threads(1)
        p1, r1 = oracle_mod.run(b, p0, r0, 0.003, 2, 10)
        oracle_mod.set_threads(4)
        p4, r4 = oracle_mod.run(b, p0, r0, 0.003, 2, 10)
    finally:
        oracle_mod.set_threads(old)
    assert np.array_equal(p1.view(np.uint32), p4.view(np.uint32))
    assert np.array_equal(r1.view(np.uint32), r4.view(np.uint32))


def test_fp32_close_to_fp64(oracle_mod):
    import phantoms
    b, p0, r0 = phantoms.make_inputs(0)
    p32, r32 = oracle_mod.run(b, p0, r0, 0.01, 1, 10)
    p64, r64 = oracle_mod.run(b, p0, r0, 0.01, 1, 10, dtype=np.float64)
    assert np.max(np.abs(p32 - p64)) < 1e-5
    assert np.max(np.abs(r32 - r64)) < 1e-5


def test_cone_matches_full_run(oracle_mod):
    import phantoms
    b, p0, r0 = phantoms.make_inputs(4, dims=(40, 30, 20))
    p, r = oracle_mod.run(b, p0, r0, 0.003, 2, 3)
    z = oracle_mod.primal(b, p, 0.003)
    for c in [(0, 0, 0), (19, 29, 39), (10, 15, 20), (3, 28, 1), (19, 0, 37)]:
        pc, rc, zc = oracle_mod.run_cone(b, p0, r0, 0.003, 2, 3, c)
        assert np.array_equal(pc, p[(slice(None),) + c])
        assert np.array_equal(rc, r[(slice(None),) + c])
        assert zc == z[c]


# --------------------------------------------------------------------------
# duality gap in per-voxel form

def test_gap_per_voxel_form_equals_definition(oracle_mod):
    """In fp64 the oracle's per-voxel gap equals P(z) - d(p) from the definition."""
    import phantoms
    b = phantoms.make_b(0, dims=(9, 8, 7)).astype(np.float64) * 3.0
    lam = 0.01
    for k in (0, 1, 5, 40):
        p0 = zeros_field(b.shape)
        p, _ = oracle_mod.run(b, p0, p0, lam, 1, k, dtype=np.float64) if k else (p0, p0)
        g_pv, tv, fid = oracle_mod.duality_gap(b, p, lam)
        g_def = duality_gap(b, p, lam)  # matrix-built D, P(z) - d(p)
        assert abs(g_pv - g_def) <= 1e-12 * max(1.0, abs(g_def)) + 1e-15
        # the pieces: P(z) = fid + lam * tv
        nz, ny, nx = b.shape
        d = brute.difference_matrix(nx, ny, nz)
        z = np.maximum(b.ravel() - lam * (d.T @ p.ravel()), 0.0)
        dz = (d @ z).reshape(3, -1)
        assert abs(tv - np.sqrt((dz ** 2).sum(axis=0)).sum()) < 1e-12 * max(tv, 1.0)
        assert abs(fid - 0.5 * ((z - b.ravel()) ** 2).sum()) < 1e-12 * max(fid, 1.0)


def test_gap_nonnegative_and_closing(oracle_mod):
    import phantoms
    b, p0, r0 = phantoms.make_inputs(0, (12, 10, 9))
    lam = 0.01
    prev = None
    for k in (1, 10, 100, 400):
        p, _ = oracle_mod.run(b, p0, r0, lam, 1, k)
        g, tv, fid = oracle_mod.duality_gap(b, p, lam)
        assert g >= -1e-9 * lam * tv  # |p| <= 1 + 5e-7 in fp32
        if prev is not None:
            assert g < prev
        prev = g
    g1 = oracle_mod.duality_gap(b, oracle_mod.run(b, p0, r0, lam, 1, 1)[0], lam)[0]
    assert prev < 1e-3 * g1


@pytest.mark.parametrize("row", read_golden("two_voxel.txt"))
def test_gap_zero_at_two_voxel_optimum(oracle_mod, row):
    """At the closed-form optimum (p = +1 on the only slot) the gap is 0."""
    _, lam, b0, b1, z0, z1, pk = row[0], *map(float, row[1:])
    b = np.array([b0, b1]).reshape(1, 1, 2)
    p = zeros_field((1, 1, 2))
    p[0, 0, 0, 0] = pk
    g, tv, fid = oracle_mod.duality_gap(b, p, lam)
    assert abs(g) < 1e-15
    assert abs(tv - abs(z0 - z1)) < 1e-15
    assert abs(fid - 0.5 * ((z0 - b0) ** 2 + (z1 - b1) ** 2)) < 1e-15
