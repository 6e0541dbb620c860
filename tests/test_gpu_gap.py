"""GPU duality gap and the convergence-checked solve, against the CPU oracle.

The gap kernel computes z and g = Dz in fp32 exactly as the oracle does (bit
for bit), the per-voxel terms in fp64 with the same roundings (multiply-adds
of exact products, the fidelity's 1/2 applied to its total), and sums them in
a different but fixed order; so the results agree to fp64 summation error
(relative 1e-10 is required) and repeated GPU calls agree bit for bit.
"""
import numpy as np
import pytest

import oracle
import phantoms

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

RTOL = 1e-10


@pytest.fixture(scope="module")
def tvf():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import stencil_dual_update_amd as m
    oracle.set_threads(16)
    return m


def gpu_gap(tvf, b, p, lam, b_offset=0):
    """Gap triple of the device kernels; b_offset > 0 places b that many
    elements into its allocation (misaligned for the pair pass when odd)."""
    nz, ny, nx = b.shape
    dev = torch.device("cuda")
    store = torch.zeros(b.size + b_offset, dtype=torch.float32, device=dev)
    bt = store[b_offset:].view(b.shape)
    bt.copy_(torch.from_numpy(np.ascontiguousarray(b)))
    pt = torch.from_numpy(np.ascontiguousarray(p)).to(dev)
    out = torch.full((3,), float("nan"), dtype=torch.float64, device=dev)
    ws = torch.empty(tvf.gap_workspace_bytes(nx, ny, nz) // 8, dtype=torch.float64, device=dev)
    tvf.tv_fgp_duality_gap(bt, pt, lam, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def assert_gap_close(got, exp, lam, label):
    g, tv, fid = exp
    scale_g = lam * tv + 1e-300
    assert abs(got[0] - g) <= RTOL * scale_g, (label, got[0], g)
    assert abs(got[1] - tv) <= RTOL * max(tv, 1e-300), (label, got[1], tv)
    assert abs(got[2] - fid) <= RTOL * max(fid, 1e-300), (label, got[2], fid)


@pytest.mark.parametrize("steps", [0, 1, 10])
def test_gap_workload0(tvf, steps):
    b, p0, r0 = phantoms.make_inputs(0)
    p = oracle.run(b, p0, r0, 0.01, 1, steps)[0] if steps else p0
    exp = oracle.duality_gap(b, p, 0.01)
    got = gpu_gap(tvf, b, p, 0.01)
    assert_gap_close(got, exp, 0.01, "w0 after %d" % steps)
    assert got[0] >= 0.0


@pytest.mark.parametrize("dims", [(67, 45, 29), (1, 1, 1), (2, 1, 1), (1, 1, 9), (130, 3, 70),
                                  (1100, 10, 7), (65, 5, 17)],
                         ids=lambda d: "x".join(map(str, d)))
def test_gap_ragged_random_dual(tvf, dims):
    b, p0, _ = phantoms.make_inputs(4, dims)
    exp = oracle.duality_gap(b, p0, 0.003)
    got = gpu_gap(tvf, b, p0, 0.003)
    assert_gap_close(got, exp, 0.003, str(dims))


@pytest.mark.parametrize("dims", [(130, 17, 9), (258, 9, 19), (2, 11, 3), (512, 64, 24)],
                         ids=lambda d: "x".join(map(str, d)))
def test_gap_pair_and_one_voxel_passes(tvf, dims):
    """Even nx with b and p aligned to two elements takes the two-voxels-per-
    lane first pass; b one element into its allocation takes the one-voxel
    pass.  Both agree with the oracle."""
    b, p0, _ = phantoms.make_inputs(4, dims)
    exp = oracle.duality_gap(b, p0, 0.003)
    assert_gap_close(gpu_gap(tvf, b, p0, 0.003), exp, 0.003, "pair %s" % (dims,))
    assert_gap_close(gpu_gap(tvf, b, p0, 0.003, b_offset=1), exp, 0.003, "one %s" % (dims,))


def test_gap_deterministic(tvf):
    b, p0, _ = phantoms.make_inputs(4, (150, 70, 40))
    a = gpu_gap(tvf, b, p0, 0.003)
    c = gpu_gap(tvf, b, p0, 0.003)
    assert np.array_equal(a.view(np.uint64), c.view(np.uint64))


def test_gap_full_size_512(tvf):
    """Headline volume after one outer iteration (10 steps), all voxels."""
    w = phantoms.workload(3)
    b, p0, r0 = phantoms.make_inputs(3)
    p, _ = oracle.run(b, p0, r0, w["lam"], 1, 10)
    exp = oracle.duality_gap(b, p, w["lam"])
    got = gpu_gap(tvf, b, p, w["lam"])
    assert_gap_close(got, exp, w["lam"], "512^3")


def oracle_trajectory(b, p0, r0, lam, n_outer, n_inner):
    """Oracle state and gap after 0, 1, ..., n_outer outer iterations."""
    states = []
    p, r = p0.copy(), r0.copy()
    for o in range(n_outer + 1):
        states.append((p.copy(), r.copy(), oracle.duality_gap(b, p, lam)))
        if o < n_outer:
            p, r = oracle.run(b, p, r, lam, 1, n_inner)
    return states


def gpu_solve(tvf, b, p0, r0, lam, max_outer, n_inner, tol, variant="fused"):
    nz, ny, nx = b.shape
    dev = torch.device("cuda")
    v = tvf.VARIANTS[variant]
    bt = torch.from_numpy(b).to(dev)
    p = torch.from_numpy(p0).to(dev)
    ra = torch.from_numpy(r0).to(dev)
    rb = torch.empty_like(ra)
    ws = torch.empty(tvf.gap_workspace_bytes(nx, ny, nz) // 8, dtype=torch.float64, device=dev)
    gd = torch.empty(3, dtype=torch.float64, device=dev)
    zws = (torch.empty_like(bt) if v == tvf.TWO_KERNEL else
           torch.empty_like(p) if v in (tvf.TB2, tvf.TB3) else None)
    done, where, gap = tvf.tv_fgp_solve(bt, p, ra, rb, lam, max_outer, n_inner, tol, ws, gd,
                                        variant=v, z_ws=zws)
    r = rb if where else ra
    return done, p.cpu().numpy(), r.cpu().numpy(), gap, gd.cpu().numpy()


@pytest.mark.parametrize("variant", ["fused", "two_kernel", "tb2", "tb3"])
def test_solve_stops_where_the_oracle_gap_says(tvf, variant):
    w = phantoms.workload(1)
    lam = w["lam"]
    b, p0, r0 = phantoms.make_inputs(1)
    traj = oracle_trajectory(b, p0, r0, lam, 8, 10)
    rel = [g / (fid + lam * tv) for _, _, (g, tv, fid) in traj]
    assert all(a > c for a, c in zip(rel[1:], rel[2:])), rel
    stop = 5
    tol = 0.5 * (rel[stop] + rel[stop - 1])  # reached first after `stop` outer iterations
    done, p, r, gap, gdev = gpu_solve(tvf, b, p0, r0, lam, 20, 10, tol, variant)
    assert done == stop
    pe, re, ge = traj[stop]
    assert np.array_equal(p.view(np.uint32), pe.view(np.uint32))
    assert np.array_equal(r.view(np.uint32), re.view(np.uint32))
    assert_gap_close(np.array(gap), ge, lam, "solve")
    assert np.array_equal(np.array(gap), gdev)


def test_solve_limits(tvf):
    b, p0, r0 = phantoms.make_inputs(0)
    # max_outer = 0: no step, only the gap of the initial p
    done, p, r, gap, _ = gpu_solve(tvf, b, p0, r0, 0.01, 0, 10, 1e-3)
    assert done == 0 and np.array_equal(p, p0)
    assert_gap_close(np.array(gap), oracle.duality_gap(b, p0, 0.01), 0.01, "initial")
    # negative tolerance: runs every outer iteration
    done, p, r, gap, _ = gpu_solve(tvf, b, p0, r0, 0.01, 3, 4, -1.0)
    assert done == 3
    pe, re = oracle.run(b, p0, r0, 0.01, 3, 4)
    assert np.array_equal(p.view(np.uint32), pe.view(np.uint32))
    assert np.array_equal(r.view(np.uint32), re.view(np.uint32))
    # a huge tolerance stops before the first iteration
    done, p, _, _, _ = gpu_solve(tvf, b, p0, r0, 0.01, 3, 4, 1e30)
    assert done == 0 and np.array_equal(p, p0)
