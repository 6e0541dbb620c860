"""GPU parity on a volume past 2^31 voxels (64-bit offset and index paths).

1400 x 1300 x 1200 = 2.18e9 voxels, 8.7 GB per volume.  At this size the
default kernel switches from 32-bit to 64-bit byte offsets, the ablation
kernels from int32 to int64 indices, and the grid is smaller than the tile
count, so workgroups loop over tiles.  Each variant runs three steps, so the
three-steps-per-pass run takes one three-step pass (and the two-steps-per-pass
run one two-step pass and one single step); sampled voxels (corners, faces,
interior, tile, slab and group edges, offsets past 4 GiB) are compared with
the CPU oracle on sub-boxes of the inputs (after K steps a voxel depends only
on inputs within K voxels of it, so a margin of K + 1 is exact).  The
duality-gap reduction is checked on the same volume against the oracle's gap
of the whole volume, and the binary16 runs (one and two steps per pass) on
sampled voxels against the oracle's half mode.
"""
import numpy as np
import pytest

import oracle
import phantoms

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

DIMS = (1400, 1300, 1200)
LAM = 0.01


def test_volume_past_2_31_voxels_all_variants():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import stencil_dual_update_amd as tvf
    nx, ny, nz = DIMS
    n = nx * ny * nz
    assert n > 2 ** 31
    free, _ = torch.cuda.mem_get_info()
    need = 14 * n * 4
    assert free > need, "needs %.0f GB of device memory, %.0f GB free" % (need / 1e9, free / 1e9)
    b = phantoms.make_uniform(DIMS, seed=11, lo=-0.01, hi=0.05)
    dev = torch.device("cuda")
    bt = torch.from_numpy(b).to(dev)
    p = torch.empty((3, nz, ny, nx), device=dev)
    ra = torch.empty_like(p)
    rb = torch.empty_like(p)
    ws3 = torch.empty_like(p)  # second p of the two-steps-per-pass variant
    ws = ws3[0]                 # z of the two-kernel variant, then the read-out
    # slabs of the multi-step kernels start at multiples of 96 or 32 planes,
    # tiles at multiples of 64 x 8; byte offsets pass 2^32 from plane 591 on
    pts = [(0, 0, 0), (nz - 1, ny - 1, nx - 1), (nz // 2, ny // 2, nx // 2), (7, 1299, 0),
           (1199, 0, 1399), (600, 8 * 81, 64 * 16), (601, 8 * 81 - 1, 64 * 16 - 1),
           (1100, 517, 1023), (3, 4, 1024), (1196, 1297, 700), (95, 7, 63), (96, 8, 64),
           (97, 9, 65), (1151, 1295, 1343), (1152, 1296, 1344), (1153, 1297, 1345),
           (767, 640, 1), (768, 639, 1398), (590, 1299, 1399), (591, 0, 0)]
    K = 3
    expected = {}
    for c in pts:
        lo = [max(v - K - 1, 0) for v in c]
        hi = [min(v + K + 2, s) for v, s in zip(c, (nz, ny, nx))]
        sub = np.ascontiguousarray(b[lo[0]:hi[0], lo[1]:hi[1], lo[2]:hi[2]])
        p0 = np.zeros((3,) + sub.shape, np.float32)
        pe, re, ze = oracle.run_cone(sub, p0, p0, LAM, 1, K,
                                     (c[0] - lo[0], c[1] - lo[1], c[2] - lo[2]))
        expected[c] = (pe, re, ze)
    for variant, v in tvf.VARIANTS.items():
        print("2.18e9 voxels: %s, %d steps" % (variant, K), flush=True)
        p.zero_()
        ra.zero_()
        where = tvf.tv_fgp_run(bt, p, ra, rb, LAM, 1, K, variant=v,
                               z_ws=ws if v == tvf.TWO_KERNEL else
                               ws3 if v in (tvf.TB2, tvf.TB3) else None)
        r = rb if where else ra
        tvf.tv_primal(bt, p, ws, LAM)
        torch.cuda.synchronize()
        for c, (pe, re, ze) in expected.items():
            gp = p[:, c[0], c[1], c[2]].cpu().numpy()
            gr = r[:, c[0], c[1], c[2]].cpu().numpy()
            gz = ws[c].item()
            assert np.array_equal(gp.view(np.uint32), pe.view(np.uint32)), (variant, c, gp, pe)
            assert np.array_equal(gr.view(np.uint32), re.view(np.uint32)), (variant, c, gr, re)
            assert np.float32(gz) == ze, (variant, c, gz, ze)
    del bt, p, ra, rb, ws, ws3
    torch.cuda.empty_cache()


def test_duality_gap_past_2_31_voxels():
    """Both first passes of the gap reduction (voxel pairs; one voxel, taken
    when b is misaligned) on their 64-bit offset paths, against the oracle's
    gap of the same p over the whole volume.  The oracle adds 2.2e9 terms
    one after another in fp64, so the comparison allows 1e-8 relative (its
    own rounding error is below n * 2^-53 ~ 2.4e-7 in the worst case and
    ~sqrt(n) * 2^-53 ~ 5e-12 typically)."""
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import stencil_dual_update_amd as tvf
    nx, ny, nz = DIMS
    n = nx * ny * nz
    free, _ = torch.cuda.mem_get_info()
    need = 12 * n * 4
    assert free > need, "needs %.0f GB of device memory, %.0f GB free" % (need / 1e9, free / 1e9)
    b = phantoms.make_uniform(DIMS, seed=12, lo=-0.01, hi=0.05)
    dev = torch.device("cuda")
    store = torch.empty(n + 1, dtype=torch.float32, device=dev)
    b_al = torch.from_numpy(b).to(dev)          # aligned: the pair pass
    b_mis = store[1:].view(nz, ny, nx)          # one element in: the one-voxel pass
    b_mis.copy_(b_al)
    p = torch.zeros((3, nz, ny, nx), device=dev)
    ra = torch.zeros_like(p)
    rb = torch.empty_like(p)
    tvf.tv_fgp_run(b_al, p, ra, rb, LAM, 1, 3)  # a dual field with |p| <= 1, not all zero
    del ra, rb
    ws = torch.empty(tvf.gap_workspace_bytes(nx, ny, nz) // 8, dtype=torch.float64, device=dev)
    got = []
    for bt in (b_al, b_mis):
        out = torch.full((3,), float("nan"), dtype=torch.float64, device=dev)
        tvf.tv_fgp_duality_gap(bt, p, LAM, out, ws)
        torch.cuda.synchronize()
        got.append(out.cpu().numpy())
    ph = p.cpu().numpy()
    del store, b_al, b_mis, p, ws
    torch.cuda.empty_cache()
    g, tv, fid = oracle.duality_gap(b, ph, LAM)
    assert tv > 0 and fid > 0
    for label, v in zip(("pair", "one voxel"), got):
        assert abs(v[0] - g) <= 1e-8 * LAM * tv, (label, v[0], g)
        assert abs(v[1] - tv) <= 1e-8 * tv, (label, v[1], tv)
        assert abs(v[2] - fid) <= 1e-8 * fid, (label, v[2], fid)
    # the two passes sum in different orders; both are far more accurate
    # than the tolerance above
    assert abs(got[0][1] - got[1][1]) <= 1e-11 * tv


@pytest.mark.parametrize("two_per_pass", [False, True], ids=["one_step", "two_steps"])
def test_binary16_past_2_31_voxels(two_per_pass):
    """The binary16 paths (the pair kernel and the two-steps-per-pass kernel)
    on their 64-bit offset paths: three steps from p = r = 0 (an odd count, so
    the two-step run also takes one single step), sampled voxels against the
    oracle's half mode on sub-boxes, bit for bit on the stored binary16."""
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import stencil_dual_update_amd as tvf
    nx, ny, nz = DIMS
    n = nx * ny * nz
    free, _ = torch.cuda.mem_get_info()
    need = n * 4 + 12 * n * 2
    assert free > need, "needs %.0f GB of device memory, %.0f GB free" % (need / 1e9, free / 1e9)
    b = phantoms.make_uniform(DIMS, seed=13, lo=-0.01, hi=0.05)
    dev = torch.device("cuda")
    bt = torch.from_numpy(b).to(dev)
    p = torch.zeros((3, nz, ny, nx), dtype=torch.float16, device=dev)
    ra = torch.zeros_like(p)
    rb = torch.empty_like(p)
    n_outer, n_inner = 1, 3
    if two_per_pass:
        ws = torch.empty_like(p)
        where = tvf.tv_fgp_run2_h(bt, p, ws, ra, rb, LAM, n_outer, n_inner)
    else:
        where = tvf.tv_fgp_run_h(bt, p, ra, rb, LAM, n_outer, n_inner)
    torch.cuda.synchronize()
    r = rb if where else ra
    K = n_outer * n_inner
    pts = [(0, 0, 0), (nz - 1, ny - 1, nx - 1), (nz // 2, ny // 2, nx // 2), (7, 1299, 0),
           (1199, 0, 1399), (600, 8 * 81, 64 * 16), (601, 8 * 81 - 1, 128 * 8 - 1),
           (1100, 517, 1023), (3, 4, 1024), (1196, 1297, 700)]
    for c in pts:
        sl = tuple(slice(max(0, ci - K - 1), min(s, ci + K + 2)) for ci, s in zip(c, b.shape))
        loc = tuple(ci - s.start for ci, s in zip(c, sl))
        sub = np.ascontiguousarray(b[sl])
        z0 = np.zeros((3,) + sub.shape, np.uint16)
        pe, re = oracle.run_half(sub, z0, z0, LAM, n_outer, n_inner)
        gp = p[:, c[0], c[1], c[2]].cpu().numpy().view(np.uint16)
        gr = r[:, c[0], c[1], c[2]].cpu().numpy().view(np.uint16)
        assert np.array_equal(gp, pe[(slice(None),) + loc]), ("p", c, gp, pe[(slice(None),) + loc])
        assert np.array_equal(gr, re[(slice(None),) + loc]), ("r", c, gr, re[(slice(None),) + loc])
    del bt, p, ra, rb
    torch.cuda.empty_cache()
