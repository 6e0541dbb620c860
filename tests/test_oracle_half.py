"""Half-precision dual storage in the oracle: the binary16 conversions and the
half-storage iteration, pinned without a GPU.

The conversions are checked exhaustively (all 65536 binary16 patterns) and on
every rounding tie, against numpy's IEEE float16 conversion (a library routine
that implements the same round-to-nearest-even definition).
"""
import numpy as np
import pytest

from conftest import read_golden

RNG = np.random.default_rng(16)


def test_f16_to_f32_exhaustive(oracle_mod):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle_mod.f16_bits_to_f32(h)
    exp = h.view(np.float16).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), exp.view(np.uint32))


def test_f32_to_f16_ties_and_neighbours(oracle_mod):
    # every finite binary16 value, the exact midpoint to the next one (a tie
    # in binary32), and the binary32 values one ulp either side of it
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)  # ties are exact in binary32
    cand = np.concatenate([lo.astype(np.float32), mid, np.nextafter(mid, np.float32(0)),
                           np.nextafter(mid, np.float32(np.inf))])
    cand = np.concatenate([cand, -cand, np.float32([65504.0, 65519.996, 65520.0, np.inf, -np.inf])])
    got = oracle_mod.f32_to_f16_bits(cand)
    with np.errstate(over="ignore"):
        exp = cand.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, exp)


def test_f32_to_f16_random_bit_patterns(oracle_mod):
    x = RNG.integers(0, 1 << 32, size=4_000_000, dtype=np.uint64).astype(np.uint32)
    v = x.view(np.float32)
    v = v[~np.isnan(v)]  # NaN payloads: numpy keeps them, the oracle returns 0x7E00
    got = oracle_mod.f32_to_f16_bits(v)
    with np.errstate(over="ignore"):
        exp = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, exp)


def half(a):
    return np.asarray(a, np.float32).astype(np.float16).view(np.uint16)


def test_half_zero_and_constant(oracle_mod):
    shape = (5, 6, 7)
    for c in (0.0, 0.04, -0.3):
        b = np.full(shape, c, np.float32)
        z16 = np.zeros((3,) + shape, np.uint16)
        p, r = oracle_mod.run_half(b, z16, z16, 0.01, 2, 10)
        assert not p.any() and not r.any()


@pytest.mark.parametrize("row", read_golden("two_voxel.txt"))
def test_half_two_voxel_closed_form(oracle_mod, row):
    _, lam, b0, b1, z0, z1, pk = row[0], *map(float, row[1:])
    b = np.array([b0, b1], np.float32).reshape(1, 1, 2)
    z16 = np.zeros((3, 1, 1, 2), np.uint16)
    p, _ = oracle_mod.run_half(b, z16, z16, lam, 1, 400)
    pf = oracle_mod.f16_bits_to_f32(p)
    assert pf[0, 0, 0, 0] == np.float32(pk) and pf[0, 0, 0, 1] == 0.0  # +1 is exact in binary16
    z = oracle_mod.primal(b, pf, lam).ravel()
    assert np.allclose(z, [z0, z1], atol=1e-7, rtol=0)


def test_half_matches_single_step_definition(oracle_mod):
    """One half step = widen, one fp32 step, round (checked step by step)."""
    import phantoms
    b, p0, r0 = phantoms.make_inputs(4, (21, 17, 13))
    ph, rh = half(p0), half(r0)
    for k in range(1, 6):
        pw = oracle_mod.f16_bits_to_f32(ph)
        rw = oracle_mod.f16_bits_to_f32(rh)
        pe, re = oracle_mod.step(b, pw, rw, 0.003, oracle_mod.momentum_f32(k))
        ph2, rh2 = oracle_mod.run_half(b, ph, rh, 0.003, 1, 1) if k == 1 else (None, None)
        if k == 1:
            assert np.array_equal(ph2, half(pe)) and np.array_equal(rh2, half(re))
        ph, rh = half(pe), half(re)
    p5, r5 = oracle_mod.run_half(b, half(p0), half(r0), 0.003, 1, 5)
    assert np.array_equal(p5, ph) and np.array_equal(r5, rh)


def test_half_feasible_and_close_to_fp64(oracle_mod):
    """|p| <= 1 up to binary16 rounding; after 200 steps the half iterate stays
    close to the fp64 one.

    Rounding p to binary16 moves each component by at most 2^-12 (|p| <= 1), so
    one rounding shifts z = max(b - lam L(p), 0) by at most lam * 6 * 2^-12.
    The projection is non-expansive, so these shifts do not add up step by
    step; measured after 200 steps the z error is 1-12 times that one-step
    bound on the workload recipes.  The test allows 25 times, and the duality
    gap of the half iterate within 10% of the fp64 one.
    """
    import phantoms
    dims = (48, 40, 32)
    w = phantoms.workload(1)
    lam = w["lam"]
    b, p0, r0 = phantoms.make_inputs(1, dims)
    ph, rh = oracle_mod.run_half(b, half(p0), half(r0), lam, 20, 10)
    pf = oracle_mod.f16_bits_to_f32(ph).astype(np.float64)
    assert np.sqrt((pf ** 2).sum(axis=0)).max() <= 1.0 + 2.0 ** -10
    b64 = b.astype(np.float64)
    p64, _ = oracle_mod.run(b64, p0.astype(np.float64), r0.astype(np.float64), lam, 20, 10)
    z16 = oracle_mod.primal(b64, pf, lam)
    z64 = oracle_mod.primal(b64, p64, lam)
    assert np.max(np.abs(z16 - z64)) <= 25 * lam * 6 * 2.0 ** -12
    g16 = oracle_mod.duality_gap(b64, pf, lam)[0]
    g64 = oracle_mod.duality_gap(b64, p64, lam)[0]
    assert abs(g16 - g64) <= 0.1 * g64
