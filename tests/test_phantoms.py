"""Seeded input generators: determinism, shapes, value ranges, admissible p0."""
import numpy as np
import pytest

import phantoms


@pytest.mark.parametrize("idx", [0, 1, 2, 3, 4])
def test_recipe_fields(idx):
    w = phantoms.workload(idx)
    assert len(w["dims"]) == 3 and w["lam"] > 0
    assert w["n_outer"] * w["n_inner"] in (10, 200)


@pytest.mark.parametrize("idx,dims", [(0, None), (1, (40, 36, 30)), (2, (48, 40, 32)),
                                      (3, (64, 64, 64)), (4, (50, 39, 16))])
def test_b_deterministic_and_shaped(idx, dims):
    b1 = phantoms.make_b(idx, dims)
    b2 = phantoms.make_b(idx, dims)
    nx, ny, nz = dims or phantoms.workload(idx)["dims"]
    assert b1.shape == (nz, ny, nx) and b1.dtype == np.float32
    assert b1.flags.c_contiguous
    assert np.array_equal(b1.view(np.uint32), b2.view(np.uint32))
    assert np.isfinite(b1).all()


def test_b_differs_between_workloads():
    a = phantoms.make_b(2, (32, 32, 32))
    b = phantoms.make_b(3, (32, 32, 32))
    assert not np.array_equal(a, b)


def test_value_ranges():
    b0 = phantoms.make_b(0)
    # 3 blobs of amplitude <= 0.05 plus N(0, 0.005) noise
    assert b0.max() < 3 * 0.05 + 6 * 0.005 and b0.min() > -6 * 0.005
    assert 0.003 < b0.std() < 0.05
    b4 = phantoms.make_b(4, (60, 50, 20))
    assert b4.min() >= 0.0 and b4.max() <= 0.03 + 16 * 0.02
    assert (b4 > 0.03).any()  # the ellipsoids are there


def test_initial_dual_of_anisotropic_workload():
    dims = (37, 29, 21)
    nx, ny, nz = dims
    b, p0, r0 = phantoms.make_inputs(4, dims)
    assert p0.shape == (3, nz, ny, nx) and p0.dtype == np.float32
    assert np.array_equal(p0, r0) and p0 is not r0
    norm = np.sqrt((p0.astype(np.float64) ** 2).sum(axis=0))
    assert norm.max() <= 1.0
    assert norm.max() > 0.95 and norm.min() >= 0.0
    assert not p0[0, :, :, nx - 1].any()
    assert not p0[1, :, ny - 1, :].any()
    assert not p0[2, nz - 1].any()
    # seeded: a second draw is identical
    assert np.array_equal(p0, phantoms.make_p0(4, dims))


@pytest.mark.parametrize("idx", [0, 1, 2, 3])
def test_zero_initial_dual(idx):
    p0 = phantoms.make_p0(idx, (9, 8, 7))
    assert p0.shape == (3, 7, 8, 9) and not p0.any()
