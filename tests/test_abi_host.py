"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every function include/tv_fgp.h declares, and
reject every invalid call with its documented status before touching the HIP
runtime.  The momentum schedule is host logic and is compared with the
oracle's independent implementation.  Fake device addresses are used only on
paths that fail validation (or enqueue nothing), so no memory is accessed.
"""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

tvf = pytest.importorskip("stencil_dual_update_amd", reason="libtvfgp.so not built")
L = tvf.lib

NX, NY, NZ = 8, 6, 5
VOL = NX * NY * NZ * 4
BASE = 1 << 40  # fake, never dereferenced


def addr(k):
    """Address of the k-th fake volume (disjoint, 256-byte aligned)."""
    return BASE + k * ((VOL + 255) // 256 * 256 + 4096)


P3 = ctypes.c_void_p * 3


def field(*ks):
    return P3(*[None if k is None else addr(k) if isinstance(k, int) and k < 1000 else k
                for k in ks])


def step(b=0, p=(1, 2, 3), ri=(4, 5, 6), ro=(7, 8, 9), lam=0.01, m=0.0,
         dims=(NX, NY, NZ), variant=0, ws=None):
    bb = None if b is None else addr(b)
    pp = None if p is None else field(*p)
    rin = None if ri is None else field(*ri)
    rout = None if ro is None else field(*ro)
    return L.tv_fgp_step_ex(bb, pp, rin, rout, lam, m, *dims, variant,
                            None if ws is None else addr(ws), None)


def header_functions():
    text = open(os.path.join(ROOT, "include", "tv_fgp.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"\b(tv_\w+)\s*\(", text)


def test_exports_match_header():
    names = header_functions()
    assert names, "no declarations parsed"
    assert tuple(names) == tvf.EXPORTS
    for n in names:
        assert hasattr(L, n), n
        assert ctypes.cast(getattr(L, n), ctypes.c_void_p).value


def test_library_path_is_in_tree():
    assert os.path.dirname(tvf.LIB_PATH) == os.path.join(ROOT, "stencil_dual_update_amd")


def test_momentum_matches_oracle(oracle_mod):
    for k in range(1, 60):
        assert np.float32(tvf.momentum(k)) == oracle_mod.momentum_f32(k), k
    assert tvf.momentum(0) == 0.0 and tvf.momentum(-3) == 0.0


def test_status_strings_distinct():
    codes = [0, -1, -2, -3, -4, -5, -6, -7, -8]
    strs = [tvf.status_string(c) for c in codes]
    assert len(set(strs)) == len(strs)
    assert tvf.status_string(-99) == "unknown status"


def test_variant_names():
    for name, v in tvf.VARIANTS.items():
        assert tvf.variant_name(v) == name
    assert tvf.variant_name(13) is None
    assert tvf.variant_name(-1) is None


def test_workspace_bytes():
    assert tvf.workspace_bytes(tvf.TWO_KERNEL, 10, 20, 30) == 10 * 20 * 30 * 4
    for v in (tvf.FUSED, tvf.LDS_MARCH, tvf.POINT, tvf.REG_MARCH):
        assert tvf.workspace_bytes(v, 10, 20, 30) == 0
    assert tvf.workspace_bytes(tvf.TWO_KERNEL, 0, 20, 30) == 0
    assert tvf.workspace_bytes(tvf.TB2, 10, 20, 30) == 3 * 10 * 20 * 30 * 4
    assert tvf.workspace_bytes(tvf.TB3, 10, 20, 30) == 3 * 10 * 20 * 30 * 4
    assert tvf.workspace_bytes(tvf.PAIR, 10, 20, 30) == 0
    assert tvf.workspace_bytes(13, 10, 20, 30) == 0
    assert tvf.workspace_bytes(tvf.CUBE, 10, 20, 30) == 0
    assert tvf.workspace_bytes(tvf.TWO_KERNEL, 1 << 31, 1 << 31, 1 << 31) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(b=None), tvf.TV_ERR_NULL),
    (dict(p=None), tvf.TV_ERR_NULL),
    (dict(ri=None), tvf.TV_ERR_NULL),
    (dict(ro=None), tvf.TV_ERR_NULL),
    (dict(p=(1, None, 3)), tvf.TV_ERR_NULL),
    (dict(ro=(7, 8, None)), tvf.TV_ERR_NULL),
    (dict(dims=(0, NY, NZ)), tvf.TV_ERR_DIMS),
    (dict(dims=(NX, -1, NZ)), tvf.TV_ERR_DIMS),
    (dict(dims=(NX, NY, 0)), tvf.TV_ERR_DIMS),
    (dict(dims=(1 << 31, 1 << 31, 1 << 31)), tvf.TV_ERR_DIMS),
    (dict(dims=(1 << 62, 2, 1)), tvf.TV_ERR_DIMS),
    (dict(ro=(7, 8, 5)), tvf.TV_ERR_ALIAS),        # r_out aliases r_in
    (dict(ro=(7, 7, 9)), tvf.TV_ERR_ALIAS),        # two outputs alias
    (dict(p=(1, 2, 0)), tvf.TV_ERR_ALIAS),         # p aliases b
    (dict(p=(4, 2, 3)), tvf.TV_ERR_ALIAS),         # p aliases r_in
    (dict(ro=(7, 8, 1)), tvf.TV_ERR_ALIAS),        # r_out aliases p
    (dict(lam=0.0), tvf.TV_ERR_PARAM),
    (dict(lam=-0.01), tvf.TV_ERR_PARAM),
    (dict(lam=float("nan")), tvf.TV_ERR_PARAM),
    (dict(lam=float("inf")), tvf.TV_ERR_PARAM),
    (dict(lam=1e-45), tvf.TV_ERR_PARAM),           # 1/(12 lambda) overflows
    (dict(m=float("nan")), tvf.TV_ERR_PARAM),
    (dict(m=float("inf")), tvf.TV_ERR_PARAM),
    (dict(variant=13), tvf.TV_ERR_VARIANT),
    (dict(variant=-1), tvf.TV_ERR_VARIANT),
    (dict(variant=2), tvf.TV_ERR_WORKSPACE),       # two-kernel without z
    (dict(variant=2, ws=0), tvf.TV_ERR_ALIAS),     # workspace aliases b
])
def test_step_rejects(kw, code):
    assert step(**kw) == code


def test_partial_overlap_is_alias():
    pp = field(1, 2, 3)
    ri = field(4, 5, 6)
    ro = P3(addr(7), addr(8), addr(5) + 8)  # overlaps r_in[1] by all but 8 bytes
    assert L.tv_fgp_step_ex(addr(0), pp, ri, ro, 0.01, 0.0, NX, NY, NZ, 0, None, None) \
        == tvf.TV_ERR_ALIAS
    ro = P3(addr(7), addr(8), addr(5) + VOL - 4)  # last float of r_in[1]
    assert L.tv_fgp_step_ex(addr(0), pp, ri, ro, 0.01, 0.0, NX, NY, NZ, 0, None, None) \
        == tvf.TV_ERR_ALIAS


def test_misaligned_pointer():
    pp = P3(addr(1) + 2, addr(2), addr(3))
    assert L.tv_fgp_step_ex(addr(0), pp, field(4, 5, 6), field(7, 8, 9), 0.01, 0.0,
                            NX, NY, NZ, 0, None, None) == tvf.TV_ERR_ALIGN


def test_default_entry_point_validates():
    assert L.tv_fgp_step(None, field(1, 2, 3), field(4, 5, 6), field(7, 8, 9),
                         0.01, 0.0, NX, NY, NZ, None) == tvf.TV_ERR_NULL
    assert L.tv_fgp_step(addr(0), field(1, 2, 3), field(4, 5, 6), field(7, 8, 9),
                         0.01, 0.0, NX, NY, 0, None) == tvf.TV_ERR_DIMS


def run(b=0, p=(1, 2, 3), ra=(4, 5, 6), rb=(7, 8, 9), lam=0.01, n_outer=2, n_inner=3,
        dims=(NX, NY, NZ), variant=0, ws=None):
    where = ctypes.c_int(-7)
    st = L.tv_fgp_run(None if b is None else addr(b), field(*p), field(*ra), field(*rb),
                      lam, n_outer, n_inner, *dims, variant,
                      None if ws is None else addr(ws), None, ctypes.byref(where))
    return st, where.value


@pytest.mark.parametrize("kw,code", [
    (dict(b=None), tvf.TV_ERR_NULL),
    (dict(n_outer=-1), tvf.TV_ERR_PARAM),
    (dict(n_inner=-2), tvf.TV_ERR_PARAM),
    (dict(lam=0.0), tvf.TV_ERR_PARAM),
    (dict(rb=(7, 8, 4)), tvf.TV_ERR_ALIAS),        # r_b aliases r_a
    (dict(ra=(4, 5, 1)), tvf.TV_ERR_ALIAS),        # r_a aliases p
    (dict(dims=(NX, NY, -4)), tvf.TV_ERR_DIMS),
    (dict(variant=13), tvf.TV_ERR_VARIANT),
    (dict(variant=2), tvf.TV_ERR_WORKSPACE),
    (dict(variant=6), tvf.TV_ERR_WORKSPACE),       # two steps per pass without p workspace
    (dict(variant=6, ws=9), tvf.TV_ERR_ALIAS),     # first workspace volume is r_b[2]
])
def test_run_rejects(kw, code):
    st, where = run(**kw)
    assert st == code
    assert where == 0


@pytest.mark.parametrize("n_outer,n_inner", [(0, 10), (20, 0), (0, 0)])
def test_run_with_no_steps_enqueues_nothing(n_outer, n_inner):
    # valid arguments, zero steps: returns at once with r_final = 0 and never
    # reaches the HIP runtime (there is no GPU here)
    st, where = run(n_outer=n_outer, n_inner=n_inner)
    assert st == tvf.TV_OK and where == 0


def test_primal_rejects():
    pp = field(1, 2, 3)
    assert L.tv_primal(None, pp, addr(4), 0.01, NX, NY, NZ, None) == tvf.TV_ERR_NULL
    assert L.tv_primal(addr(0), pp, None, 0.01, NX, NY, NZ, None) == tvf.TV_ERR_NULL
    assert L.tv_primal(addr(0), None, addr(4), 0.01, NX, NY, NZ, None) == tvf.TV_ERR_NULL
    assert L.tv_primal(addr(0), pp, addr(2), 0.01, NX, NY, NZ, None) == tvf.TV_ERR_ALIAS
    assert L.tv_primal(addr(0), pp, addr(0), 0.01, NX, NY, NZ, None) == tvf.TV_ERR_ALIAS
    assert L.tv_primal(addr(0), pp, addr(4), -1.0, NX, NY, NZ, None) == tvf.TV_ERR_PARAM
    assert L.tv_primal(addr(0), pp, addr(4), 0.01, NX, 0, NZ, None) == tvf.TV_ERR_DIMS


def test_python_binding_raises():
    with pytest.raises(tvf.TvFgpError) as e:
        tvf.tv_fgp_step(addr(0), [addr(1), addr(2), addr(3)], [addr(4), addr(5), addr(6)],
                        [addr(7), addr(8), addr(5)], 0.01, 0.0, stream=0, dims=(NX, NY, NZ))
    assert e.value.status == tvf.TV_ERR_ALIAS
    assert tvf.tv_fgp_run(addr(0), [addr(1), addr(2), addr(3)], [addr(4), addr(5), addr(6)],
                          [addr(7), addr(8), addr(9)], 0.01, 0, 10, stream=0,
                          dims=(NX, NY, NZ)) == 0


def test_gap_workspace_bytes():
    assert 0 < tvf.gap_workspace_bytes(NX, NY, NZ) <= 24 * 1024
    assert tvf.gap_workspace_bytes(4096, 4096, 4096) == 3 * 8 * 1024
    assert tvf.gap_workspace_bytes(0, 1, 1) == 0


def gap(b=0, p=(1, 2, 3), lam=0.01, out=20, ws=21, ws_bytes=None, dims=(NX, NY, NZ)):
    wsb = tvf.gap_workspace_bytes(*dims) if ws_bytes is None else ws_bytes
    return L.tv_fgp_duality_gap(None if b is None else addr(b), field(*p), lam, *dims,
                                None if out is None else addr(out),
                                None if ws is None else addr(ws), wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(b=None), tvf.TV_ERR_NULL),
    (dict(out=None), tvf.TV_ERR_NULL),
    (dict(ws=None), tvf.TV_ERR_NULL),
    (dict(p=(1, None, 3)), tvf.TV_ERR_NULL),
    (dict(ws_bytes=8), tvf.TV_ERR_WORKSPACE),
    (dict(lam=0.0), tvf.TV_ERR_PARAM),
    (dict(dims=(NX, 0, NZ)), tvf.TV_ERR_DIMS),
    (dict(out=1), tvf.TV_ERR_ALIAS),   # out inside p[0]
    (dict(ws=0), tvf.TV_ERR_ALIAS),    # workspace inside b
    (dict(out=21), tvf.TV_ERR_ALIAS),  # out inside the workspace
])
def test_gap_rejects(kw, code):
    assert gap(**kw) == code


def test_gap_misaligned_out():
    assert L.tv_fgp_duality_gap(addr(0), field(1, 2, 3), 0.01, NX, NY, NZ, addr(20) + 4,
                                addr(21), tvf.gap_workspace_bytes(NX, NY, NZ), None) \
        == tvf.TV_ERR_ALIGN


def solve(max_outer=3, n_inner=5, tol=1e-3, ra=(4, 5, 6), rb=(7, 8, 9), gws=21, gdev=20,
          lam=0.01, host=True):
    where, done = ctypes.c_int(-5), ctypes.c_int(-5)
    gh = (ctypes.c_double * 3)()
    st = L.tv_fgp_solve(addr(0), field(1, 2, 3), field(*ra), field(*rb), lam, max_outer, n_inner,
                        tol, NX, NY, NZ, 0, None, addr(gws),
                        tvf.gap_workspace_bytes(NX, NY, NZ), addr(gdev), None,
                        ctypes.byref(where), ctypes.byref(done), gh if host else None)
    return st, where.value, done.value


@pytest.mark.parametrize("kw,code", [
    (dict(max_outer=-1), tvf.TV_ERR_PARAM),
    (dict(n_inner=-1), tvf.TV_ERR_PARAM),
    (dict(tol=float("nan")), tvf.TV_ERR_PARAM),
    (dict(lam=-1.0), tvf.TV_ERR_PARAM),
    (dict(host=False), tvf.TV_ERR_NULL),
    (dict(gdev=7), tvf.TV_ERR_ALIAS),      # gap output inside r_b[0]
    (dict(gws=4), tvf.TV_ERR_ALIAS),       # gap workspace inside r_a[0]
    (dict(rb=(7, 8, 5)), tvf.TV_ERR_ALIAS),
])
def test_solve_rejects(kw, code):
    st, where, done = solve(**kw)
    assert st == code
    assert where == 0 and done == 0


def step_h(b=0, p=(1, 2, 3), ri=(4, 5, 6), ro=(7, 8, 9), lam=0.01, m=0.0, dims=(NX, NY, NZ),
           pp=None):
    return L.tv_fgp_step_h(None if b is None else addr(b), pp or field(*p), field(*ri),
                           field(*ro), lam, m, *dims, None)


@pytest.mark.parametrize("kw,code", [
    (dict(b=None), tvf.TV_ERR_NULL),
    (dict(p=(1, None, 3)), tvf.TV_ERR_NULL),
    (dict(dims=(0, NY, NZ)), tvf.TV_ERR_DIMS),
    (dict(lam=0.0), tvf.TV_ERR_PARAM),
    (dict(m=float("nan")), tvf.TV_ERR_PARAM),
    (dict(ro=(7, 8, 5)), tvf.TV_ERR_ALIAS),
    (dict(p=(1, 2, 0)), tvf.TV_ERR_ALIAS),
])
def test_step_h_rejects(kw, code):
    assert step_h(**kw) == code


def test_step_h_half_sized_buffers():
    # binary16 volumes are half as long: a p component that starts inside the
    # second half of a float-sized slot overlaps nothing
    vol_h = NX * NY * NZ * 2
    pp = P3(addr(1), addr(1) + vol_h, addr(2))
    ro = P3(addr(7), addr(8), addr(7) + vol_h)
    assert L.tv_fgp_run_h(addr(0), pp, field(4, 5, 6), ro, 0.01, 0, 10, NX, NY, NZ, None,
                          None) == tvf.TV_OK
    pp_bad = P3(addr(1), addr(1) + vol_h - 2, addr(2))  # one element of overlap
    assert L.tv_fgp_run_h(addr(0), pp_bad, field(4, 5, 6), field(7, 8, 9), 0.01, 0, 10,
                          NX, NY, NZ, None, None) == tvf.TV_ERR_ALIAS
    pp_odd = P3(addr(1) + 1, addr(2), addr(3))
    assert L.tv_fgp_run_h(addr(0), pp_odd, field(4, 5, 6), field(7, 8, 9), 0.01, 0, 10,
                          NX, NY, NZ, None, None) == tvf.TV_ERR_ALIGN


def test_primal_h_rejects():
    assert L.tv_primal_h(addr(0), field(1, 2, 3), addr(1), 0.01, NX, NY, NZ, None) \
        == tvf.TV_ERR_ALIAS
    assert L.tv_primal_h(addr(0), field(1, 2, 3), None, 0.01, NX, NY, NZ, None) \
        == tvf.TV_ERR_NULL


@pytest.mark.parametrize("variant", [tvf.TB2, tvf.TB3], ids=["tb2", "tb3"])
def test_run_multistep_accepts_three_volume_workspace(variant):
    # nothing is enqueued with n_outer = 0, so the checks alone decide
    st, where = run(variant=variant, ws=10, n_outer=0)
    assert st == tvf.TV_OK and where == 0
    st, _ = run(variant=variant, ws=None, n_outer=0)
    assert st == tvf.TV_ERR_WORKSPACE


@pytest.mark.parametrize("variant", [tvf.TB2, tvf.TB3], ids=["tb2", "tb3"])
def test_run_multistep_workspace_spans_three_volumes(variant):
    # b placed inside the third volume of the workspace overlaps it; just past it, not
    ws = addr(10)
    for b_addr, code in ((ws + 2 * VOL + 4, tvf.TV_ERR_ALIAS), (ws + 3 * VOL, tvf.TV_OK)):
        where = ctypes.c_int(-7)
        st = L.tv_fgp_run(b_addr, field(1, 2, 3), field(4, 5, 6), field(7, 8, 9), 0.01, 0, 3,
                          NX, NY, NZ, variant, ws, None, ctypes.byref(where))
        assert st == code


def step2(b=0, pi=(1, 2, 3), po=(10, 11, 12), ri=(4, 5, 6), ro=(7, 8, 9), lam=0.01, m1=0.0,
          m2=0.3, dims=(NX, NY, NZ)):
    return L.tv_fgp_step2(None if b is None else addr(b), field(*pi), field(*po), field(*ri),
                          field(*ro), lam, m1, m2, *dims, None)


@pytest.mark.parametrize("kw,code", [
    (dict(b=None), tvf.TV_ERR_NULL),
    (dict(po=(10, None, 12)), tvf.TV_ERR_NULL),
    (dict(dims=(NX, 0, NZ)), tvf.TV_ERR_DIMS),
    (dict(lam=-1.0), tvf.TV_ERR_PARAM),
    (dict(m1=float("nan")), tvf.TV_ERR_PARAM),
    (dict(m2=float("inf")), tvf.TV_ERR_PARAM),
    (dict(po=(1, 11, 12)), tvf.TV_ERR_ALIAS),   # p_out on p_in: the pass needs both
    (dict(po=(10, 11, 4)), tvf.TV_ERR_ALIAS),   # p_out on r_in
    (dict(ro=(7, 8, 0)), tvf.TV_ERR_ALIAS),     # r_out on b
    (dict(ro=(7, 8, 12)), tvf.TV_ERR_ALIAS),    # r_out on p_out
])
def test_step2_rejects(kw, code):
    assert step2(**kw) == code


def step3(b=0, pi=(1, 2, 3), po=(10, 11, 12), ri=(4, 5, 6), ro=(7, 8, 9), lam=0.01, m1=0.0,
          m2=0.3, m3=0.4, dims=(NX, NY, NZ)):
    return L.tv_fgp_step3(None if b is None else addr(b), field(*pi), field(*po), field(*ri),
                          field(*ro), lam, m1, m2, m3, *dims, None)


@pytest.mark.parametrize("kw,code", [
    (dict(b=None), tvf.TV_ERR_NULL),
    (dict(pi=(1, None, 3)), tvf.TV_ERR_NULL),
    (dict(dims=(NX, NY, 0)), tvf.TV_ERR_DIMS),
    (dict(lam=float("nan")), tvf.TV_ERR_PARAM),
    (dict(m1=float("inf")), tvf.TV_ERR_PARAM),
    (dict(m2=float("nan")), tvf.TV_ERR_PARAM),
    (dict(m3=float("-inf")), tvf.TV_ERR_PARAM),
    (dict(po=(1, 11, 12)), tvf.TV_ERR_ALIAS),   # p_out on p_in
    (dict(po=(10, 5, 12)), tvf.TV_ERR_ALIAS),   # p_out on r_in
    (dict(ro=(0, 8, 9)), tvf.TV_ERR_ALIAS),     # r_out on b
    (dict(ro=(7, 11, 9)), tvf.TV_ERR_ALIAS),    # r_out on p_out
])
def test_step3_rejects(kw, code):
    assert step3(**kw) == code


def step2_h(b=0, pi=(1, 2, 3), po=(10, 11, 12), ri=(4, 5, 6), ro=(7, 8, 9), lam=0.01, m1=0.0,
            m2=0.3, dims=(NX, NY, NZ)):
    return L.tv_fgp_step2_h(None if b is None else addr(b), field(*pi), field(*po), field(*ri),
                            field(*ro), lam, m1, m2, *dims, None)


@pytest.mark.parametrize("kw,code", [
    (dict(b=None), tvf.TV_ERR_NULL),
    (dict(dims=(0, NY, NZ)), tvf.TV_ERR_DIMS),
    (dict(m2=float("nan")), tvf.TV_ERR_PARAM),
    (dict(po=(1, 11, 12)), tvf.TV_ERR_ALIAS),
    (dict(ro=(7, 8, 0)), tvf.TV_ERR_ALIAS),
])
def test_step2_h_rejects(kw, code):
    assert step2_h(**kw) == code


def run2_h(ws, n_outer=0, b=0):
    where = ctypes.c_int(-7)
    st = L.tv_fgp_run2_h(addr(b), field(1, 2, 3), ws, field(4, 5, 6), field(7, 8, 9), 0.01,
                         n_outer, 3, NX, NY, NZ, None, ctypes.byref(where))
    return st, where.value


def test_run2_h_workspace():
    # three binary16 volumes: 3 * VOL / 2 bytes from ws; nothing enqueued with n_outer = 0
    assert run2_h(None)[0] == tvf.TV_ERR_NULL
    assert run2_h(addr(10)) == (tvf.TV_OK, 0)
    ws = addr(10)
    assert run2_h(ws, b=0)[0] == tvf.TV_OK
    assert L.tv_fgp_run2_h(ws + 3 * VOL // 2 - 4, field(1, 2, 3), ws, field(4, 5, 6),
                           field(7, 8, 9), 0.01, 0, 3, NX, NY, NZ, None, None) == tvf.TV_ERR_ALIAS
    assert run2_h(addr(9))[0] == tvf.TV_ERR_ALIAS   # first volume is r_b[2]
    assert run2_h(addr(10) + 1)[0] == tvf.TV_ERR_ALIGN


def probe(src=tuple(range(7)), dst=tuple(range(7, 13)), n=200):
    """tv_fgp_stream_probe on fake volumes (k < 1000: the k-th fake volume,
    else a raw address); only calls that fail validation are made."""
    def arr(ks, count):
        if ks is None:
            return None
        return (ctypes.c_void_p * count)(*[None if k is None else addr(k) if k < 1000 else k
                                            for k in ks])
    return L.tv_fgp_stream_probe(arr(src, 7), arr(dst, 6), n, None)


@pytest.mark.parametrize("kw,code", [
    (dict(src=None), tvf.TV_ERR_NULL),
    (dict(dst=None), tvf.TV_ERR_NULL),
    (dict(src=(0, 1, 2, None, 4, 5, 6)), tvf.TV_ERR_NULL),
    (dict(n=0), tvf.TV_ERR_DIMS),
    (dict(n=-5), tvf.TV_ERR_DIMS),
    (dict(n=1 << 62), tvf.TV_ERR_DIMS),
    (dict(src=(0, 1, 2, 3, 4, 5, addr(6) + 4)), tvf.TV_ERR_ALIGN),
    (dict(dst=(7, 8, 9, 10, 11, addr(12) + 8)), tvf.TV_ERR_ALIGN),
    (dict(dst=(7, 8, 9, 10, 11, 3)), tvf.TV_ERR_ALIAS),   # a dst is a src
    (dict(dst=(7, 8, 9, 10, 10, 12)), tvf.TV_ERR_ALIAS),  # two dst alias
])
def test_stream_probe_rejects(kw, code):
    assert probe(**kw) == code


def probe_ex(src=tuple(range(7)), n_src=7, dst=tuple(range(7, 13)), n_dst=6, n=200):
    """tv_fgp_stream_probe_ex on fake volumes, as probe(); only calls that
    fail validation are made."""
    def arr(ks):
        if ks is None:
            return None
        return (ctypes.c_void_p * max(1, len(ks)))(*[None if k is None else addr(k) if k < 1000
                                                      else k for k in ks])
    return L.tv_fgp_stream_probe_ex(arr(src), n_src, arr(dst), n_dst, n, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n_src=2, n_dst=2), tvf.TV_ERR_PARAM),
    (dict(n_src=7, n_dst=5), tvf.TV_ERR_PARAM),
    (dict(n_src=-1, n_dst=6), tvf.TV_ERR_PARAM),
    (dict(src=None), tvf.TV_ERR_NULL),
    (dict(dst=None), tvf.TV_ERR_NULL),
    (dict(src=None, n_src=0, dst=None, n_dst=6), tvf.TV_ERR_NULL),
    (dict(n_dst=0, dst=None, n=0), tvf.TV_ERR_DIMS),
    (dict(n_src=1, n_dst=1, src=(0,), dst=(1,), n=-3), tvf.TV_ERR_DIMS),
    (dict(n_src=1, n_dst=1, src=(addr(0) + 4,), dst=(1,)), tvf.TV_ERR_ALIGN),
    (dict(n_src=0, src=None, dst=(7, 8, 9, 10, 11, addr(12) + 8)), tvf.TV_ERR_ALIGN),
    (dict(n_src=1, n_dst=1, src=(0,), dst=(0,)), tvf.TV_ERR_ALIAS),
    (dict(dst=(7, 8, 9, 10, 10, 12)), tvf.TV_ERR_ALIAS),
    (dict(n_src=0, src=None, dst=(7, 8, 9, 10, 11, 7)), tvf.TV_ERR_ALIAS),
])
def test_stream_probe_ex_rejects(kw, code):
    assert probe_ex(**kw) == code


def run_pp(b=0, p=(1, 2, 3), ra=(4, 5, 6), rb=(7, 8, 9), lam=0.01, n_outer=2, n_inner=3,
           dims=(NX, NY, NZ), variant=0, ws=None, want_p=True):
    where = ctypes.c_int(-7)
    pwhere = ctypes.c_int(-7)
    st = L.tv_fgp_run_pp(None if b is None else addr(b), field(*p), field(*ra), field(*rb),
                         lam, n_outer, n_inner, *dims, variant,
                         None if ws is None else addr(ws), None, ctypes.byref(where),
                         ctypes.byref(pwhere) if want_p else None)
    return st, where.value, pwhere.value


@pytest.mark.parametrize("kw,code", [
    (dict(want_p=False), tvf.TV_ERR_NULL),         # p_final is required
    (dict(b=None), tvf.TV_ERR_NULL),
    (dict(n_outer=-1), tvf.TV_ERR_PARAM),
    (dict(lam=float("inf")), tvf.TV_ERR_PARAM),
    (dict(rb=(7, 8, 4)), tvf.TV_ERR_ALIAS),
    (dict(variant=12), tvf.TV_ERR_WORKSPACE),      # three steps per pass without p workspace
    (dict(variant=12, ws=9), tvf.TV_ERR_ALIAS),
    (dict(variant=99), tvf.TV_ERR_VARIANT),
])
def test_run_pp_rejects(kw, code):
    st, where, pwhere = run_pp(**kw)
    assert st == code
    assert where == 0
    if kw.get("want_p", True):
        assert pwhere == 0


def test_run_pp_with_no_steps_enqueues_nothing():
    for variant, ws in ((0, None), (12, 20)):
        st, where, pwhere = run_pp(n_outer=0, n_inner=10, variant=variant, ws=ws)
        assert (st, where, pwhere) == (tvf.TV_OK, 0, 0)
