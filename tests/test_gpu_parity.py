"""GPU parity: the HIP kernels against the fp32 CPU oracle, element by element.

Gate (all variants): max |GPU - oracle| <= 1e-5 on p, r and z after the
full iteration count.  The kernels and the oracle evaluate the same fp32
operations in the same order without contraction, so the expected result is
bit-for-bit equality; the bitwise checks are separate tests so a one-ulp
difference is reported as such rather than hidden behind the tolerance.
Every call goes through the C ABI (libtvfgp.so via the ctypes binding).
"""
import numpy as np
import pytest

import oracle
import phantoms

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL = 1e-5
VARIANTS = ["fused", "lds_march", "two_kernel", "point", "reg_march", "pair", "tb2", "cube",
            "cube_32x8x2", "cube_64x8x1", "cube_8x8x8", "cube_32x4x4", "tb3"]


def run_workspace(tvf, v, like):
    """The workspace a run of variant v needs: z (two-kernel) or a second p (tb2, tb3)."""
    if v == tvf.TWO_KERNEL:
        return torch.empty_like(like)
    if v in (tvf.TB2, tvf.TB3):
        return torch.empty((3,) + tuple(like.shape), dtype=like.dtype, device=like.device)
    return None


@pytest.fixture(scope="module")
def tvf():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import stencil_dual_update_amd as m
    oracle.set_threads(16)
    return m


def gpu_solve(tvf, b, p0, r0, lam, n_outer, n_inner, variant="fused", stream=None):
    v = tvf.VARIANTS[variant]
    dev = torch.device("cuda")
    bt = torch.from_numpy(np.ascontiguousarray(b)).to(dev)
    p = torch.from_numpy(np.ascontiguousarray(p0)).to(dev)
    ra = torch.from_numpy(np.ascontiguousarray(r0)).to(dev)
    rb = torch.full_like(ra, float("nan"))
    ws = run_workspace(tvf, v, bt)
    where = tvf.tv_fgp_run(bt, p, ra, rb, lam, n_outer, n_inner, variant=v, z_ws=ws,
                           stream=stream)
    r = rb if where else ra
    z = torch.empty_like(bt)
    tvf.tv_primal(bt, p, z, lam, stream=stream)
    torch.cuda.synchronize()
    out = p.cpu().numpy(), r.cpu().numpy(), z.cpu().numpy()
    del bt, p, ra, rb, ws, z
    return out


def oracle_solve(b, p0, r0, lam, n_outer, n_inner):
    p, r = oracle.run(b, p0, r0, lam, n_outer, n_inner)
    return p, r, oracle.primal(b, p, lam)


def max_abs(a, e):
    return float(np.max(np.abs(a.astype(np.float64) - e.astype(np.float64)))) if a.size else 0.0


def assert_close(got, exp, label):
    for name, g, e in zip("prz", got, exp):
        assert g.shape == e.shape
        assert np.isfinite(g).all(), "%s %s: non-finite values" % (label, name)
        d = max_abs(g, e)
        assert d <= TOL, "%s %s: max abs %.3g > %g" % (label, name, d, TOL)


def assert_bitwise(got, exp, label):
    for name, g, e in zip("prz", got, exp):
        neq = int(np.count_nonzero(g.view(np.uint32) != e.view(np.uint32)))
        assert neq == 0, "%s %s: %d of %d elements differ in bits (max abs %.3g)" % (
            label, name, neq, g.size, max_abs(g, e))


_cache = {}


def reference(idx, dims=None, n_outer=None, n_inner=None):
    w = phantoms.workload(idx)
    n_outer = w["n_outer"] if n_outer is None else n_outer
    n_inner = w["n_inner"] if n_inner is None else n_inner
    key = (idx, dims, n_outer, n_inner)
    if key not in _cache:
        b, p0, r0 = phantoms.make_inputs(idx, dims)
        _cache.clear()
        _cache[key] = (b, p0, r0, w["lam"], n_outer, n_inner,
                       oracle_solve(b, p0, r0, w["lam"], n_outer, n_inner))
    return _cache[key]


# --------------------------------------------------------------------------
# small workloads, every variant

@pytest.mark.parametrize("variant", VARIANTS)
def test_workload0_blobs_32(tvf, variant):
    b, p0, r0, lam, no, ni, exp = reference(0)
    got = gpu_solve(tvf, b, p0, r0, lam, no, ni, variant)
    assert_close(got, exp, "blobs 32^3 " + variant)
    assert_bitwise(got, exp, "blobs 32^3 " + variant)


@pytest.mark.parametrize("variant", VARIANTS)
def test_workload1_blobs_128_full_200_steps(tvf, variant):
    b, p0, r0, lam, no, ni, exp = reference(1)
    got = gpu_solve(tvf, b, p0, r0, lam, no, ni, variant)
    assert_close(got, exp, "blobs 128^3 " + variant)
    assert_bitwise(got, exp, "blobs 128^3 " + variant)


RAGGED = [(67, 45, 29), (1, 1, 1), (1, 1, 9), (9, 1, 1), (1, 7, 1), (130, 3, 70),
          (65, 5, 17), (63, 3, 2), (1000, 7, 3), (2, 2, 2), (64, 4, 16), (64, 4, 17),
          (200, 9, 33), (3, 300, 5), (1100, 10, 6), (64, 70, 10), (2100, 20, 5),
          (258, 17, 6), (126, 9, 4), (2, 1, 3)]


@pytest.mark.parametrize("dims", RAGGED, ids=lambda d: "x".join(map(str, d)))
@pytest.mark.parametrize("idx", [0, 4])
def test_ragged_shapes_all_variants(tvf, dims, idx):
    b, p0, r0 = phantoms.make_inputs(idx, dims)
    lam = phantoms.workload(idx)["lam"]
    exp = oracle_solve(b, p0, r0, lam, 2, 5)
    for variant in VARIANTS:
        got = gpu_solve(tvf, b, p0, r0, lam, 2, 5, variant)
        label = "%s %s w%d" % (variant, dims, idx)
        assert_close(got, exp, label)
        assert_bitwise(got, exp, label)


@pytest.mark.parametrize("variant", VARIANTS)
def test_r_different_from_p(tvf, variant):
    """A mid-run state: r is not p (arbitrary admissible fields)."""
    dims = (70, 13, 21)
    b = phantoms.make_b(2, dims)
    p0 = phantoms.random_ball_field(dims, seed=7)
    r0 = phantoms.random_ball_field(dims, seed=8)
    exp = oracle_solve(b, p0, r0, 0.002, 3, 4)
    got = gpu_solve(tvf, b, p0, r0, 0.002, 3, 4, variant)
    assert_close(got, exp, "r != p " + variant)
    assert_bitwise(got, exp, "r != p " + variant)


@pytest.mark.parametrize("dims", [(77, 19, 11), (78, 19, 11)], ids=["nx77", "nx78"])
def test_single_step_with_explicit_momentum(tvf, dims):
    b, p0, r0 = phantoms.make_inputs(4, dims)
    m = np.float32(0.61803)
    pe, re = oracle.step(b, p0, r0, 0.003, m)
    dev = torch.device("cuda")
    bt = torch.from_numpy(b).to(dev)
    for variant in VARIANTS:
        v = tvf.VARIANTS[variant]
        p = torch.from_numpy(p0).to(dev)
        ri = torch.from_numpy(r0).to(dev)
        ro = torch.empty_like(ri)
        ws = run_workspace(tvf, v, bt) if v == tvf.TWO_KERNEL else None
        tvf.tv_fgp_step(bt, p, ri, ro, 0.003, float(m), variant=v, z_ws=ws)
        torch.cuda.synchronize()
        got = (p.cpu().numpy(), ro.cpu().numpy(), oracle.primal(b, p.cpu().numpy(), 0.003))
        exp = (pe, re, oracle.primal(b, pe, 0.003))
        assert_bitwise(got, exp, "single step " + variant)
        assert np.array_equal(ri.cpu().numpy(), r0), "r_in was modified"


STEP2_DIMS = [(67, 45, 29), (130, 17, 33), (64, 8, 16), (64, 8, 17), (1, 1, 1), (5, 70, 3),
              (1, 1, 40), (200, 3, 2), (129, 9, 47)]


@pytest.mark.parametrize("dims", STEP2_DIMS, ids=lambda d: "x".join(map(str, d)))
def test_step2_equals_two_oracle_steps(tvf, dims):
    """One two-steps-per-pass launch against two oracle steps, from a state with r != p."""
    b, p0, _ = phantoms.make_inputs(4, dims)
    rng = np.random.default_rng(17)
    r0 = (p0 + 0.3 * rng.standard_normal(p0.shape)).astype(np.float32)
    m1, m2 = np.float32(0.3), np.float32(0.61)
    pe, re = oracle.step(b, p0, r0, 0.003, m1)
    pe, re = oracle.step(b, pe, re, 0.003, m2)
    dev = torch.device("cuda")
    bt = torch.from_numpy(b).to(dev)
    pi = torch.from_numpy(p0).to(dev)
    ri = torch.from_numpy(r0).to(dev)
    po = torch.full_like(pi, float("nan"))
    ro = torch.full_like(ri, float("nan"))
    tvf.tv_fgp_step2(bt, pi, po, ri, ro, 0.003, float(m1), float(m2))
    torch.cuda.synchronize()
    got_p = po.cpu().numpy()
    assert_bitwise((got_p, ro.cpu().numpy(), oracle.primal(b, got_p, 0.003)),
                   (pe, re, oracle.primal(b, pe, 0.003)), "step2 %s" % (dims,))
    assert np.array_equal(pi.cpu().numpy(), p0) and np.array_equal(ri.cpu().numpy(), r0)


# --------------------------------------------------------------------------
# degenerate cases

@pytest.mark.parametrize("variant", VARIANTS)
def test_zero_input_stays_zero(tvf, variant):
    dims = (50, 9, 20)
    nx, ny, nz = dims
    b = np.zeros((nz, ny, nx), np.float32)
    p0 = np.zeros((3, nz, ny, nx), np.float32)
    p, r, z = gpu_solve(tvf, b, p0, p0, 0.01, 2, 10, variant)
    for a in (p, r, z):
        assert not a.any() and not np.signbit(a).any()


@pytest.mark.parametrize("variant", VARIANTS)
def test_negative_zero_in_b(tvf, variant):
    """b = -0 at some voxels: max(u, 0) must give +0 there, as (u > 0) ? u : +0 does
    (a max instruction may keep the sign of -0), and everything after bit for bit."""
    dims = (70, 9, 13)
    b, p0, r0 = phantoms.make_inputs(4, dims)
    b = b.copy()
    b.reshape(-1)[::7] = np.float32(-0.0)
    zero = np.zeros_like(p0)
    z_exp = oracle.primal(b, zero, 0.003)
    assert not np.signbit(z_exp[b == 0]).any()
    exp = oracle_solve(b, zero, zero, 0.003, 1, 4)
    got = gpu_solve(tvf, b, zero, zero, 0.003, 1, 4, variant)
    assert_bitwise(got, exp, "-0 in b " + variant)
    bt = torch.from_numpy(b).to("cuda")
    z = torch.empty_like(bt)
    tvf.tv_primal(bt, torch.from_numpy(zero).to("cuda"), z, 0.003)
    torch.cuda.synchronize()
    assert np.array_equal(z.cpu().numpy().view(np.uint32), z_exp.view(np.uint32))


@pytest.mark.parametrize("c", [0.0, 0.037, -0.2])
def test_constant_input(tvf, c):
    dims = (70, 6, 9)
    nx, ny, nz = dims
    b = np.full((nz, ny, nx), c, np.float32)
    p0 = np.zeros((3, nz, ny, nx), np.float32)
    for variant in VARIANTS:
        p, r, z = gpu_solve(tvf, b, p0, p0, 0.01, 2, 10, variant)
        assert not p.any() and not r.any()
        assert np.array_equal(z, np.full_like(b, max(c, 0.0)))


@pytest.mark.parametrize("dims", STEP2_DIMS + [(64, 8, 200), (70, 13, 9)],
                         ids=lambda d: "x".join(map(str, d)))
def test_step3_equals_three_oracle_steps(tvf, dims):
    """One three-steps-per-pass launch against three oracle steps, from a state with r != p."""
    b, p0, _ = phantoms.make_inputs(4, dims)
    rng = np.random.default_rng(19)
    r0 = (p0 + 0.3 * rng.standard_normal(p0.shape)).astype(np.float32)
    m = (np.float32(0.3), np.float32(0.61), np.float32(0.7))
    pe, re = p0, r0
    for mk in m:
        pe, re = oracle.step(b, pe, re, 0.003, mk)
    dev = torch.device("cuda")
    bt = torch.from_numpy(b).to(dev)
    pi = torch.from_numpy(p0).to(dev)
    ri = torch.from_numpy(r0).to(dev)
    po = torch.full_like(pi, float("nan"))
    ro = torch.full_like(ri, float("nan"))
    tvf.tv_fgp_step3(bt, pi, po, ri, ro, 0.003, *(float(x) for x in m))
    torch.cuda.synchronize()
    got_p = po.cpu().numpy()
    assert_bitwise((got_p, ro.cpu().numpy(), oracle.primal(b, got_p, 0.003)),
                   (pe, re, oracle.primal(b, pe, 0.003)), "step3 %s" % (dims,))
    assert np.array_equal(pi.cpu().numpy(), p0) and np.array_equal(ri.cpu().numpy(), r0)


@pytest.mark.parametrize("variant", ["tb2", "tb3"])
@pytest.mark.parametrize("no,ni", [(2, 5), (3, 4), (4, 1), (1, 7), (2, 11)],
                         ids=lambda c: str(c))
def test_multistep_runs_span_outer_iterations(tvf, variant, no, ni):
    """Passes of two or three steps may cover the end of one outer iteration and
    the start of the next (momentum restarted there); the run still equals the
    oracle's step-by-step run bit for bit."""
    b, p0, r0 = phantoms.make_inputs(4, (67, 21, 23))
    exp = oracle_solve(b, p0, r0, 0.003, no, ni)
    got = gpu_solve(tvf, b, p0, r0, 0.003, no, ni, variant)
    assert_bitwise(got, exp, "%s %dx%d" % (variant, no, ni))


@pytest.mark.parametrize("variant", ["tb2", "tb3", "fused"])
@pytest.mark.parametrize("no,ni", [(2, 10), (1, 7), (3, 4), (1, 3), (2, 1)], ids=lambda c: str(c))
def test_run_pp_leaves_p_where_it_ends(tvf, variant, no, ni):
    """tv_fgp_run_pp: p alternates with the workspace and is reported, not
    copied back; the p it names equals the oracle bit for bit, and the other
    buffer keeps the previous pass's p (multi-step variants) or stays
    untouched (one-step variants)."""
    b, p0, r0 = phantoms.make_inputs(4, (67, 21, 23))
    exp = oracle_solve(b, p0, r0, 0.003, no, ni)
    v = tvf.VARIANTS[variant]
    dev = torch.device("cuda")
    bt = torch.from_numpy(b).to(dev)
    p = torch.from_numpy(p0).to(dev)
    ra = torch.from_numpy(r0).to(dev)
    rb = torch.full_like(ra, float("nan"))
    ws = torch.full((3,) + tuple(bt.shape), float("nan"), device=dev)
    rw, pw = tvf.tv_fgp_run_pp(bt, p, ra, rb, 0.003, no, ni, variant=v,
                               z_ws=ws if v in (tvf.TB2, tvf.TB3) else None)
    torch.cuda.synchronize()
    if v not in (tvf.TB2, tvf.TB3):
        assert pw == 0
    pf = (ws if pw else p).cpu().numpy()
    rf = (rb if rw else ra).cpu().numpy()
    got = (pf, rf, oracle.primal(b, pf, 0.003))
    assert_bitwise(got, exp, "run_pp %s %dx%d" % (variant, no, ni))
    # the same run through tv_fgp_run ends with p in p: which buffer
    # tv_fgp_run_pp names follows the number of multi-step passes
    p2 = torch.from_numpy(p0).to(dev)
    ra2 = torch.from_numpy(r0).to(dev)
    rb2 = torch.empty_like(ra2)
    ws2 = torch.empty_like(ws)
    tvf.tv_fgp_run(bt, p2, ra2, rb2, 0.003, no, ni, variant=v,
                   z_ws=ws2 if v in (tvf.TB2, tvf.TB3) else ws2[0] if v == tvf.TWO_KERNEL else None)
    torch.cuda.synchronize()
    assert np.array_equal(p2.cpu().numpy().view(np.uint32), pf.view(np.uint32))


def test_no_steps_leaves_state(tvf):
    b, p0, r0 = phantoms.make_inputs(4, (40, 10, 6))
    for no, ni in ((0, 10), (3, 0)):
        p, r, z = gpu_solve(tvf, b, p0, r0, 0.003, no, ni)
        assert np.array_equal(p, p0) and np.array_equal(r, r0)
        assert np.array_equal(z, oracle.primal(b, p0, 0.003))


def test_odd_step_count_final_buffer(tvf):
    b, p0, r0 = phantoms.make_inputs(0, (33, 17, 9))
    exp = oracle_solve(b, p0, r0, 0.01, 1, 7)
    got = gpu_solve(tvf, b, p0, r0, 0.01, 1, 7)
    assert_bitwise(got, exp, "7 steps")


def test_non_default_stream(tvf):
    b, p0, r0, lam, no, ni, exp = reference(0)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        got = gpu_solve(tvf, b, p0, r0, lam, no, ni, "fused", stream=s)
    assert_bitwise(got, exp, "side stream")


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("dims,guard", [((67, 9, 18), 4096), ((130, 9, 18), 4096),
                                        ((130, 9, 18), 4097)],
                         ids=["nx67", "nx130", "nx130_odd_offset"])
def test_nan_guard_bands(tvf, variant, dims, guard):
    """Buffers sit between NaN guard bands: no write may touch them, no read
    of them may reach a result.  An odd guard length leaves the volumes
    aligned to one element but not two."""
    nx, ny, nz = dims
    n = nx * ny * nz
    b, p0, r0 = phantoms.make_inputs(4, dims)
    exp = oracle_solve(b, p0, r0, 0.003, 1, 6)
    dev = torch.device("cuda")
    v = tvf.VARIANTS[variant]
    store = torch.full((11, n + 2 * guard), float("nan"), device=dev)

    def vol(k, init=None):
        t = store[k, guard:guard + n].view(nz, ny, nx)
        if init is not None:
            t.copy_(torch.from_numpy(np.ascontiguousarray(init)))
        return t

    bt = vol(0, b)
    p = [vol(1 + a, p0[a]) for a in range(3)]
    ra = [vol(4 + a, r0[a]) for a in range(3)]
    rb = [vol(7 + a) for a in range(3)]
    ws = vol(10) if v == tvf.TWO_KERNEL else None
    ws_store = None
    if v in (tvf.TB2, tvf.TB3):  # three consecutive volumes between guard bands
        ws_store = torch.full((3 * n + 2 * guard,), float("nan"), device=dev)
        ws = ws_store[guard:guard + 3 * n].view(3, nz, ny, nx)
    where = tvf.tv_fgp_run(bt, p, ra, rb, 0.003, 1, 6, variant=v, z_ws=ws)
    torch.cuda.synchronize()
    r = rb if where else ra
    got_p = np.stack([t.cpu().numpy() for t in p])
    got_r = np.stack([t.cpu().numpy() for t in r])
    host = store.cpu().numpy()
    assert np.isnan(host[:, :guard]).all() and np.isnan(host[:, guard + n:]).all()
    if ws_store is not None:
        wh = ws_store.cpu().numpy()
        assert np.isnan(wh[:guard]).all() and np.isnan(wh[guard + 3 * n:]).all()
    assert_bitwise((got_p, got_r, oracle.primal(b, got_p, 0.003)), exp, "guard " + variant)


# --------------------------------------------------------------------------
# full-size workloads in the launch configuration the bench times
#
# The page's agreement tables ("Result at 256^3" and the 512^3 table) compare
# every variant after the full solve; here every variant is compared with the
# oracle at every voxel after the full 20 x 10 steps, bit for bit and within
# the 1e-5 gate.

def _all_variants_full(tvf, idx, label):
    b, p0, r0, lam, no, ni, exp = reference(idx)
    for variant in VARIANTS:
        print("%s %s: %d x %d steps" % (label, variant, no, ni), flush=True)
        got = gpu_solve(tvf, b, p0, r0, lam, no, ni, variant)
        assert_close(got, exp, "%s %s" % (label, variant))
        assert_bitwise(got, exp, "%s %s" % (label, variant))
        del got


def test_workload2_256_full_200_steps_all_variants(tvf):
    _all_variants_full(tvf, 2, "ellipsoids 256^3")


def test_workload3_512_full_200_steps_all_variants(tvf):
    """The headline volume: all 134M voxels after the full 20 x 10 steps."""
    _all_variants_full(tvf, 3, "ellipsoids 512^3")
    _cache.clear()


def test_workload4_anisotropic_full_200_steps(tvf):
    """1000 x 777 x 301 (rows of 1000 floats, not a multiple of a cache line;
    ragged tiles on every face): the whole volume after the full 20 x 10 steps,
    from a random admissible p with r = p, for every variant (the three-steps-
    per-pass run: 66 three-step passes, one two-step pass and the copy of p
    back from the workspace)."""
    b, p0, r0, lam, no, ni, exp = reference(4)
    assert b.shape == (301, 777, 1000)
    for variant in VARIANTS:
        print("1000x777x301 %s: %d x %d steps" % (variant, no, ni), flush=True)
        got = gpu_solve(tvf, b, p0, r0, lam, no, ni, variant)
        assert_close(got, exp, "1000x777x301 " + variant)
        assert_bitwise(got, exp, "1000x777x301 " + variant)
        del got
    p, r, z = exp
    # the invariants the oracle's result itself must show
    norm = np.sqrt((p.astype(np.float64) ** 2).sum(axis=0))
    assert norm.max() <= 1.0 + 5e-7
    nz, ny, nx = b.shape
    assert not p[0, :, :, nx - 1].any() and not p[1, :, ny - 1, :].any()
    assert not p[2, nz - 1].any()
    assert (z >= 0).all()
    _cache.clear()


def sample_points(dims, rng, n_random):
    nx, ny, nz = dims
    pts = set()
    for z in (0, nz - 1):
        for y in (0, ny - 1):
            for x in (0, nx - 1):
                pts.add((z, y, x))
    pts |= {(nz // 2, ny // 2, nx - 1), (nz - 1, ny // 2, nx // 2), (nz // 2, 0, nx // 2),
            (15, 3, 63), (16, 4, 64), (17, 5, 65), (nz - 2, ny - 2, nx - 2)}
    for _ in range(n_random):
        pts.add((int(rng.integers(nz)), int(rng.integers(ny)), int(rng.integers(nx))))
    return sorted(pts)


def test_workload4_anisotropic_sampled_10_steps(tvf):
    """1000 x 777 x 301, one outer iteration (10 steps) of the one-step
    kernel, on sampled voxels computed by the oracle from sub-boxes of the
    inputs (after K steps a voxel depends only on inputs within K voxels of
    it): a cross-check of the sub-box helper the >2^31-voxel test relies on."""
    dims = (1000, 777, 301)
    lam = phantoms.workload(4)["lam"]
    b, p0, r0 = phantoms.make_inputs(4, dims)
    rng = np.random.default_rng(4)
    p10, r10, z10 = gpu_solve(tvf, b, p0, r0, lam, 1, 10, "fused")
    for c in sample_points(dims, rng, 24):
        pe, re, ze = oracle.run_cone(b, p0, r0, lam, 1, 10, c)
        idx = (slice(None),) + c
        assert np.array_equal(p10[idx].view(np.uint32), pe.view(np.uint32)), c
        assert np.array_equal(r10[idx].view(np.uint32), re.view(np.uint32)), c
        assert z10[c] == ze, c


# --------------------------------------------------------------------------
# the marching kernel at every tile shape of the page's sweep ("TV solver:
# the FGP step on the GPU", section "What made the difference")

PAGE_MARCH_SHAPES = [(32, 8, 32), (32, 8, 16), (32, 8, 8), (32, 8, 4), (32, 8, 2), (32, 16, 16),
                     (32, 16, 8), (32, 4, 32), (64, 4, 16), (64, 8, 8), (64, 4, 8)]


def march_solve(tvf, b, p0, r0, lam, n_outer, n_inner, shape):
    """n_outer x n_inner steps with tv_fgp_step_march (momentum restarted per
    outer iteration, r ping-pong), then the read-out z."""
    tx, ty, planes = shape
    dev = torch.device("cuda")
    bt = torch.from_numpy(np.ascontiguousarray(b)).to(dev)
    p = torch.from_numpy(np.ascontiguousarray(p0)).to(dev)
    r = torch.from_numpy(np.ascontiguousarray(r0)).to(dev)
    rn = torch.full_like(r, float("nan"))
    for _ in range(n_outer):
        for k in range(1, n_inner + 1):
            tvf.tv_fgp_step_march(bt, p, r, rn, lam, tvf.momentum(k), tx, ty, planes)
            r, rn = rn, r
    z = torch.empty_like(bt)
    tvf.tv_primal(bt, p, z, lam)
    torch.cuda.synchronize()
    out = p.cpu().numpy(), r.cpu().numpy(), z.cpu().numpy()
    del bt, p, r, rn, z
    return out


@pytest.mark.parametrize("shape", PAGE_MARCH_SHAPES, ids=lambda s: "%dx%dx%d" % s)
def test_march_shapes_ragged(tvf, shape):
    for dims in [(67, 45, 29), (1, 1, 1), (33, 17, 40), (130, 3, 70), (2100, 20, 5)]:
        b, p0, r0 = phantoms.make_inputs(4, dims)
        exp = oracle_solve(b, p0, r0, 0.003, 2, 5)
        got = march_solve(tvf, b, p0, r0, 0.003, 2, 5, shape)
        label = "march %s %s" % (shape, dims)
        assert_close(got, exp, label)
        assert_bitwise(got, exp, label)


@pytest.mark.parametrize("idx", [1, 2], ids=["blobs128", "ellipsoids256"])
def test_march_shapes_full_200_steps(tvf, idx):
    b, p0, r0, lam, no, ni, exp = reference(idx)
    for shape in PAGE_MARCH_SHAPES:
        print("march %s workload %d: %d x %d steps" % (shape, idx, no, ni), flush=True)
        got = march_solve(tvf, b, p0, r0, lam, no, ni, shape)
        assert_close(got, exp, "march %s w%d" % (shape, idx))
        assert_bitwise(got, exp, "march %s w%d" % (shape, idx))
        del got


def test_march_rejects_other_shapes(tvf):
    b = torch.zeros((4, 5, 6), device="cuda")
    p = torch.zeros((3, 4, 5, 6), device="cuda")
    r = torch.zeros_like(p)
    ro = torch.zeros_like(p)
    for tx, ty, planes in [(16, 8, 8), (64, 16, 8), (32, 8, 0), (32, 8, 1025)]:
        with pytest.raises(tvf.TvFgpError) as e:
            tvf.tv_fgp_step_march(b, p, r, ro, 0.01, 0.0, tx, ty, planes)
        assert e.value.status == tvf.TV_ERR_PARAM
