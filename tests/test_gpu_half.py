"""GPU FGP with the dual stored in binary16, against the CPU oracle's half mode.

Both sides widen p and r exactly, run the binary32 step in the same operation
order, and round p and r to binary16 (nearest, ties to even) after every
step; so the stored bit patterns must agree exactly, as must the binary32
primal read out from them.
"""
import numpy as np
import pytest

import oracle
import phantoms

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def tvf():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import stencil_dual_update_amd as m
    oracle.set_threads(16)
    return m


def half_inputs(workload, dims=None):
    b, p0, r0 = phantoms.make_inputs(workload, dims)
    return b, oracle.f32_to_f16_bits(p0), oracle.f32_to_f16_bits(r0)


def to_dev_half(bits):
    """uint16 bit patterns -> device float16 tensor holding the same bits."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")
    return t.view(torch.float16)


def to_host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def gpu_run_half(tvf, b, p_bits, r_bits, lam, n_outer, n_inner):
    bt = torch.from_numpy(np.ascontiguousarray(b)).to("cuda")
    p = to_dev_half(p_bits)
    ra = to_dev_half(r_bits)
    rb = torch.empty_like(ra)
    where = tvf.tv_fgp_run_h(bt, p, ra, rb, lam, n_outer, n_inner)
    torch.cuda.synchronize()
    return to_host_bits(p), to_host_bits(rb if where else ra), bt, p


def assert_bits_equal(got, exp, label):
    if not np.array_equal(got, exp):
        bad = np.argwhere(got != exp)
        i = tuple(bad[0])
        raise AssertionError("%s: %d binary16 values differ, first at %s: got %#06x expected "
                             "%#06x" % (label, len(bad), i, got[i], exp[i]))


@pytest.mark.parametrize("workload,n_outer,n_inner", [(0, 1, 1), (0, 2, 10), (1, 1, 10),
                                                      (4, 3, 4)])
def test_run_half_matches_oracle(tvf, workload, n_outer, n_inner):
    w = phantoms.workload(workload)
    b, p0, r0 = half_inputs(workload)
    pe, re = oracle.run_half(b, p0, r0, w["lam"], n_outer, n_inner)
    pg, rg, bt, pt = gpu_run_half(tvf, b, p0, r0, w["lam"], n_outer, n_inner)
    assert_bits_equal(pg, pe, "p")
    assert_bits_equal(rg, re, "r")
    z = torch.empty_like(bt)
    tvf.tv_primal_h(bt, pt, z, w["lam"])
    torch.cuda.synchronize()
    ze = oracle.primal(b, oracle.f16_bits_to_f32(pe), w["lam"])
    assert np.array_equal(z.cpu().numpy().view(np.uint32), ze.view(np.uint32))


# odd nx takes the one-voxel kernel, even nx the two-voxel one
RAGGED = [(1, 1, 1), (2, 1, 1), (1, 1, 7), (63, 9, 5), (64, 8, 4), (65, 9, 5), (67, 45, 29),
          (130, 3, 70), (1, 130, 3), (129, 1, 9), (1000, 7, 3), (33, 17, 1), (258, 17, 6),
          (126, 9, 4), (128, 8, 4), (2, 5, 9)]


@pytest.mark.parametrize("dims", RAGGED, ids=lambda d: "x".join(map(str, d)))
def test_run_half_ragged(tvf, dims):
    b, p0, r0 = half_inputs(4, dims)
    pe, re = oracle.run_half(b, p0, r0, 0.003, 2, 3)
    pg, rg, _, _ = gpu_run_half(tvf, b, p0, r0, 0.003, 2, 3)
    assert_bits_equal(pg, pe, "p %s" % (dims,))
    assert_bits_equal(rg, re, "r %s" % (dims,))


def test_step_half_nonzero_momentum(tvf):
    """One step with m != 0 from a state where p and r differ."""
    b, p0, r0 = half_inputs(4, (70, 33, 19))
    m = float(np.float32(oracle.momentum(4)))
    # the oracle's half run applies momentum(k) at step k; run 3 steps first on both
    # sides so that the fourth uses m = momentum(4)
    pe, re = oracle.run_half(b, p0, r0, 0.003, 1, 4)
    p3, r3 = oracle.run_half(b, p0, r0, 0.003, 1, 3)
    bt = torch.from_numpy(b).to("cuda")
    p = to_dev_half(p3)
    ri = to_dev_half(r3)
    ro = torch.empty_like(ri)
    tvf.tv_fgp_step_h(bt, p, ri, ro, 0.003, m)
    torch.cuda.synchronize()
    assert_bits_equal(to_host_bits(p), pe, "p")
    assert_bits_equal(to_host_bits(ro), re, "r")


def test_half_rounding_edges(tvf):
    """Values near the binary16 limits: subnormal p, r close to the largest finite 65504."""
    dims = (65, 9, 5)
    rng = np.random.default_rng(7)
    b = (rng.random(dims[::-1], dtype=np.float32) * 4.0e4).astype(np.float32)
    p0 = np.zeros((3,) + dims[::-1], dtype=np.float32)
    p0[0] = rng.standard_normal(dims[::-1]).astype(np.float32) * 1e-6  # subnormal range
    r0 = rng.uniform(-6.5e4, 6.5e4, (3,) + dims[::-1]).astype(np.float32)
    p0b, r0b = oracle.f32_to_f16_bits(p0), oracle.f32_to_f16_bits(r0)
    for lam in (1e-7, 2.0):
        pe, re = oracle.run_half(b, p0b, r0b, lam, 1, 6)
        pg, rg, _, _ = gpu_run_half(tvf, b, p0b, r0b, lam, 1, 6)
        assert_bits_equal(pg, pe, "p lam=%g" % lam)
        assert_bits_equal(rg, re, "r lam=%g" % lam)


def test_half_full_size_sampled(tvf):
    """Headline volume, 20 steps with binary16 storage; sampled voxels against
    the oracle on sub-boxes, and the ball constraint everywhere."""
    w = phantoms.workload(3)
    lam = w["lam"]
    b, p0, r0 = half_inputs(3)
    n_outer, n_inner = 2, 10
    pg, rg, _, _ = gpu_run_half(tvf, b, p0, r0, lam, n_outer, n_inner)
    pf = oracle.f16_bits_to_f32(pg).astype(np.float64)
    # rounding the projected p to binary16 can lift |p| above 1 by at most half an ulp
    # of 1 per component
    assert np.max(np.sqrt((pf ** 2).sum(axis=0))) <= 1.0 + 3 * 2.0 ** -11
    nz, ny, nx = b.shape
    rng = np.random.default_rng(3)
    K = n_outer * n_inner
    centres = [(0, 0, 0), (nz - 1, ny - 1, nx - 1), (nz // 2, 0, nx - 1)]
    centres += [tuple(int(rng.integers(0, s)) for s in (nz, ny, nx)) for _ in range(5)]
    for c in centres:
        sl = tuple(slice(max(0, ci - K - 1), min(s, ci + K + 2)) for ci, s in zip(c, b.shape))
        loc = tuple(ci - s.start for ci, s in zip(c, sl))
        pe, re = oracle.run_half(b[sl], p0[(slice(None),) + sl], r0[(slice(None),) + sl], lam,
                                 n_outer, n_inner)
        for a in range(3):
            assert pg[(a,) + c] == pe[(a,) + loc], ("p", a, c)
            assert rg[(a,) + c] == re[(a,) + loc], ("r", a, c)


def test_half_nan_input(tvf):
    """A NaN in b is handled as the oracle handles it (NaN patterns compared as a class)."""
    b, p0, r0 = half_inputs(4, (40, 20, 10))
    b = b.copy()
    b[5, 10, 20] = np.nan
    pe, re = oracle.run_half(b, p0, r0, 0.003, 1, 2)
    pg, rg, _, _ = gpu_run_half(tvf, b, p0, r0, 0.003, 1, 2)
    nan_e = (pe & 0x7C00) == 0x7C00
    nan_g = (pg & 0x7C00) == 0x7C00
    assert np.array_equal(nan_e & ((pe & 0x3FF) != 0), nan_g & ((pg & 0x3FF) != 0))
    keep = ~(nan_e | nan_g)
    assert np.array_equal(pg[keep], pe[keep])


@pytest.mark.parametrize("dims,guard", [((67, 9, 18), 4096), ((130, 9, 18), 4096),
                                        ((130, 9, 18), 4097)],
                         ids=["nx67", "nx130", "nx130_odd_offset"])
def test_half_nan_guard_bands(tvf, dims, guard):
    """binary16 volumes between NaN guard bands: no write may touch them, no
    read of them may reach a result.  An odd guard length leaves the volumes
    aligned to one element but not two."""
    nx, ny, nz = dims
    n = nx * ny * nz
    b, p0, r0 = half_inputs(4, dims)
    pe, re = oracle.run_half(b, p0, r0, 0.003, 1, 6)
    store = torch.full((9, n + 2 * guard), float("nan"), dtype=torch.float16, device="cuda")

    def vol(k, init=None):
        t = store[k, guard:guard + n].view(nz, ny, nx)
        if init is not None:
            t.copy_(to_dev_half(init))
        return t

    bt = torch.from_numpy(b).to("cuda")
    p = [vol(a, p0[a]) for a in range(3)]
    ra = [vol(3 + a, r0[a]) for a in range(3)]
    rb = [vol(6 + a) for a in range(3)]
    where = tvf.tv_fgp_run_h(bt, p, ra, rb, 0.003, 1, 6)
    torch.cuda.synchronize()
    r = rb if where else ra
    host = to_host_bits(store)
    nan = lambda h: ((h & 0x7C00) == 0x7C00) & ((h & 0x3FF) != 0)
    assert nan(host[:, :guard]).all() and nan(host[:, guard + n:]).all()
    assert_bits_equal(np.stack([to_host_bits(t) for t in p]), pe, "p")
    assert_bits_equal(np.stack([to_host_bits(t) for t in r]), re, "r")


def gpu_run2_half(tvf, b, p_bits, r_bits, lam, n_outer, n_inner):
    bt = torch.from_numpy(np.ascontiguousarray(b)).to("cuda")
    p = to_dev_half(p_bits)
    ra = to_dev_half(r_bits)
    rb = torch.empty_like(ra)
    ws = torch.empty_like(p)
    where = tvf.tv_fgp_run2_h(bt, p, ws, ra, rb, lam, n_outer, n_inner)
    torch.cuda.synchronize()
    return to_host_bits(p), to_host_bits(rb if where else ra)


@pytest.mark.parametrize("dims,n_outer,n_inner", [
    ((67, 45, 29), 2, 5), ((130, 17, 40), 1, 4), ((64, 8, 70), 1, 3), ((1, 1, 1), 1, 2),
    ((5, 70, 3), 3, 2), ((1000, 7, 3), 1, 6)], ids=lambda c: str(c))
def test_run2_half_matches_oracle(tvf, dims, n_outer, n_inner):
    """Two binary16 steps per pass against the oracle's half mode, odd and even inner counts."""
    b, p0, r0 = half_inputs(4, dims)
    pe, re = oracle.run_half(b, p0, r0, 0.003, n_outer, n_inner)
    pg, rg = gpu_run2_half(tvf, b, p0, r0, 0.003, n_outer, n_inner)
    assert_bits_equal(pg, pe, "p %s" % (dims,))
    assert_bits_equal(rg, re, "r %s" % (dims,))


def test_step2_half_equals_two_half_steps(tvf):
    b, p0, r0 = half_inputs(4, (70, 33, 19))
    m1, m2 = float(np.float32(oracle.momentum(3))), float(np.float32(oracle.momentum(4)))
    p2, r2 = oracle.run_half(b, p0, r0, 0.003, 1, 2)      # state after steps 1, 2
    pe, re = oracle.run_half(b, p0, r0, 0.003, 1, 4)      # then steps 3, 4
    bt = torch.from_numpy(b).to("cuda")
    pi, ri = to_dev_half(p2), to_dev_half(r2)
    po, ro = torch.empty_like(pi), torch.empty_like(ri)
    tvf.tv_fgp_step2_h(bt, pi, po, ri, ro, 0.003, m1, m2)
    torch.cuda.synchronize()
    assert_bits_equal(to_host_bits(po), pe, "p")
    assert_bits_equal(to_host_bits(ro), re, "r")
    assert np.array_equal(to_host_bits(pi), p2)


def test_run2_half_workload1_full(tvf):
    w = phantoms.workload(1)
    b, p0, r0 = half_inputs(1)
    pe, re = oracle.run_half(b, p0, r0, w["lam"], 2, 10)
    pg, rg = gpu_run2_half(tvf, b, p0, r0, w["lam"], 2, 10)
    assert_bits_equal(pg, pe, "p")
    assert_bits_equal(rg, re, "r")
