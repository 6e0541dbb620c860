"""The allocation-free duality gap against the workspace one, through the C ABI.

tv_fgp_duality_gap_noalloc runs the same two reduction kernels as
tv_fgp_duality_gap with the partial sums in the library's static device
array instead of a caller's workspace, so its output must be the same bits.
Two calls in a row, the second on a smaller volume (fewer partial sums: the
first call's leftovers in the array must not reach the result), for both
first passes (even nx: voxel pairs; odd nx: one voxel per lane), and each
against the oracle's gap within the reduction's rounding.
"""
import numpy as np
import pytest

import oracle
import phantoms

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


def _gap_both(tvf, b, p, lam):
    dev = torch.device("cuda")
    bt = torch.from_numpy(b).to(dev)
    pt = torch.from_numpy(p).to(dev)
    nz, ny, nx = b.shape
    ws = torch.full((tvf.gap_workspace_bytes(nx, ny, nz) // 8,), float("nan"),
                    dtype=torch.float64, device=dev)
    out_ws = torch.full((3,), float("nan"), dtype=torch.float64, device=dev)
    out_na = torch.full((3,), float("nan"), dtype=torch.float64, device=dev)
    tvf.tv_fgp_duality_gap(bt, pt, lam, out_ws, ws)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    tvf.tv_fgp_duality_gap_noalloc(bt, pt, lam, out_na)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return out_ws.cpu().numpy(), out_na.cpu().numpy()


@pytest.mark.parametrize("sizes", [((130, 70, 45), (66, 9, 18)), ((131, 70, 45), (67, 9, 18))],
                         ids=["pair_pass", "one_voxel_pass"])
def test_noalloc_gap_equals_workspace_gap(sizes):
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import stencil_dual_update_amd as tvf
    lam = 0.003
    for dims in sizes:  # the second call is on the smaller volume
        b, p0, _ = phantoms.make_inputs(4, dims)
        print("noalloc gap %s" % (dims,), flush=True)
        got_ws, got_na = _gap_both(tvf, b, p0, lam)
        assert np.isfinite(got_na).all()
        assert np.array_equal(got_ws.view(np.uint64), got_na.view(np.uint64)), (got_ws, got_na)
        g, tv, fid = oracle.duality_gap(b, p0, lam)
        assert abs(got_na[0] - g) <= 1e-10 * lam * tv
        assert abs(got_na[1] - tv) <= 1e-10 * tv
        assert abs(got_na[2] - fid) <= 1e-10 * fid


def test_noalloc_gap_rejects_before_launch():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import stencil_dual_update_amd as tvf
    L = tvf.lib
    b = torch.zeros((5, 6, 7), device="cuda")
    p = torch.zeros((3, 5, 6, 7), device="cuda")
    out = torch.zeros(3, dtype=torch.float64, device="cuda")
    import ctypes
    P3 = ctypes.c_void_p * 3
    pp = P3(*[p[a].data_ptr() for a in range(3)])
    assert L.tv_fgp_duality_gap_noalloc(b.data_ptr(), pp, 0.01, 7, 6, 5, None, None) == \
        tvf.TV_ERR_NULL
    assert L.tv_fgp_duality_gap_noalloc(b.data_ptr(), pp, 0.0, 7, 6, 5, out.data_ptr(),
                                        None) == tvf.TV_ERR_PARAM
    assert L.tv_fgp_duality_gap_noalloc(b.data_ptr(), pp, 0.01, 0, 6, 5, out.data_ptr(),
                                        None) == tvf.TV_ERR_DIMS
    # out inside p[0]
    assert L.tv_fgp_duality_gap_noalloc(b.data_ptr(), pp, 0.01, 7, 6, 5, p[0].data_ptr(),
                                        None) == tvf.TV_ERR_ALIAS
