"""The correctly rounded square root and quotients of the dual update
(tv_fgp_device.hpp: sqrt_above_one, recip_refined, div_by_refined) on the
GPU, against the host's IEEE float32 sqrt and division (numpy), which the
projection p' = q / max(1, |q|) of the page "TV solver: the FGP step on the
GPU" (section "What one step does") is defined with; and the duality gap's
double square root (tv_fgp_gap_kernel.hpp: sqrt_sum_of_squares) against the
compiler's and numpy's.

The kernels come from tests/device_math/libdevmath.so (built by
__graft_entry__.build()).  Checked: every float above 1 for the square root;
every divisor in (1, 2^26) for the refined reciprocal, which must be the
rounded 1/d (with it the two residual corrections give the rounded
quotient, which tests/device_math/seq.cpp checks on the CPU); quotients over
the range the dual update sends to div_by_refined, with divisors whose
significand is all ones (where one Newton step from the lower reciprocal
estimate falls short) and quotients next to rounding midpoints.
"""
import ctypes
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "device_math", "libdevmath.so")
CHUNK = 1 << 26


@pytest.fixture(scope="module")
def dm():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    if not os.path.exists(LIB):
        raise RuntimeError("%s is missing: run __graft_entry__.build() first" % LIB)
    lib = ctypes.CDLL(LIB)
    for name in ("devmath_sqrt", "devmath_recip"):
        getattr(lib, name).argtypes = [ctypes.c_uint32, ctypes.c_int64, ctypes.c_void_p]
        getattr(lib, name).restype = ctypes.c_int
    lib.devmath_div.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.devmath_div.restype = ctypes.c_int
    lib.devmath_sqrt64.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                   ctypes.c_void_p]
    lib.devmath_sqrt64.restype = ctypes.c_int
    return lib


def bits_of(x):
    return int(np.array([x], dtype=np.float32).view(np.uint32)[0])


def run_range(fn, lo, hi, ref):
    """Mismatches of fn over the float bit patterns lo..hi (inclusive)
    against ref(x) on the host; returns (count, first few)."""
    import torch
    assert 0 <= lo <= hi <= 0xFFFFFFFF
    out = torch.empty(CHUNK, dtype=torch.float32, device="cuda")
    bad, shown = 0, []
    start = lo
    while start <= hi:
        n = min(CHUNK, hi - start + 1)
        assert n <= out.numel() and start + n - 1 <= 0xFFFFFFFF
        assert fn(start, n, out.data_ptr()) == 0
        got = out[:n].cpu().numpy().view(np.uint32)
        x = np.arange(start, start + n, dtype=np.uint64).astype(np.uint32).view(np.float32)
        want = ref(x).astype(np.float32).view(np.uint32)
        miss = np.nonzero(got != want)[0]
        bad += len(miss)
        for i in miss[:4]:
            shown.append((float(x[i]), hex(int(got[i])), hex(int(want[i]))))
        start += n
    return bad, shown


def test_sqrt_above_one_every_float(dm):
    """sqrt_above_one(x) == IEEE sqrtf(x) for every float x from 1 + 2^-22
    (the least float the projection's branch passes on) to +inf."""
    with np.errstate(all="ignore"):
        bad, shown = run_range(dm.devmath_sqrt, bits_of(1.0) + 2, bits_of(np.inf), np.sqrt)
    assert bad == 0, (bad, shown)


def test_refined_reciprocal_every_divisor(dm):
    """recip_refined(d) == IEEE 1/d for every float d in (1, 2^26), the
    divisors the dual update hands to div_by_refined."""
    one = np.float32(1.0)
    bad, shown = run_range(dm.devmath_recip, bits_of(1.0) + 1, bits_of(2.0 ** 26) - 1,
                           lambda x: one / x)
    assert bad == 0, (bad, shown)


def quotient_cases(seed=7, n=1 << 22):
    rng = np.random.default_rng(seed)
    ed = rng.integers(0, 26, n)
    d = np.ldexp(1.0 + rng.integers(0, 1 << 23, n) / 2.0 ** 23, ed)
    d = np.maximum(d, 1.0 + 2.0 ** -23).astype(np.float32)
    en = rng.integers(0, 127, n)
    num = np.ldexp(1.0 + rng.integers(0, 1 << 23, n) / 2.0 ** 23, ed - en)
    num = np.clip(num, 2.0 ** -100, None)
    num = np.minimum(num, d.astype(np.float64)) * rng.choice([-1.0, 1.0], n)
    cases_n, cases_d = [num.astype(np.float32)], [d]
    # all-ones significands against powers of two and neighbours of them
    ones = np.array([np.ldexp(np.float32(2.0 - 2.0 ** -23), k) for k in range(26)], np.float32)
    for k, dv in enumerate(ones):
        for j in range(-100, k + 1):
            for t in (1.0, 1.0 + 2.0 ** -23, 1.0 - 2.0 ** -24, 1.5):
                v = np.float32(np.ldexp(t, j))
                if 2.0 ** -100 <= abs(float(v)) <= float(dv):
                    cases_n += [np.array([v, -v], np.float32)]
                    cases_d += [np.array([dv, dv], np.float32)]
    # quotients within 2^-49 of a rounding midpoint, zeros, n = +-d
    y = (0.5 + rng.integers(0, 1 << 23, n) / 2.0 ** 24)
    mid = y + 2.0 ** -25 + rng.integers(-2, 3, n) * 2.0 ** -49
    nm = (d.astype(np.float64) * mid).astype(np.float32)
    keep = (np.abs(nm) <= d) & (nm != 0)
    cases_n += [nm[keep], np.zeros(4, np.float32), -np.zeros(4, np.float32), d[:4], -d[:4]]
    cases_d += [d[keep], d[:4], d[:4], d[:4], d[:4]]
    return np.concatenate(cases_n), np.concatenate(cases_d)


def test_quotients_match_ieee_division(dm):
    """div_by_refined(n, d, recip_refined(d)) == IEEE n / d, signed zeros
    included, over the range the dual update uses it in: d in (1, 2^26),
    n zero or 2^-100 <= |n| <= d."""
    import torch
    num, den = quotient_cases()
    assert np.all(den > 1) and np.all(den < 2.0 ** 26)
    assert np.all((num == 0) | ((np.abs(num) >= 2.0 ** -100) & (np.abs(num) <= den)))
    tn = torch.from_numpy(num).cuda()
    td = torch.from_numpy(den).cuda()
    out = torch.empty_like(tn)
    assert tn.numel() == td.numel() == out.numel()
    assert dm.devmath_div(tn.data_ptr(), td.data_ptr(), tn.numel(), out.data_ptr()) == 0
    got = out.cpu().numpy().view(np.uint32)
    want = (num / den).astype(np.float32).view(np.uint32)
    miss = np.nonzero(got != want)[0]
    assert len(miss) == 0, (len(miss), [(float(num[i]), float(den[i]), hex(int(got[i])),
                                         hex(int(want[i]))) for i in miss[:6]])


def sums_of_squares(seed=11, n=1 << 22):
    """Sums (x*x + y*y) + z*z of float triples, in fp64, as the gap forms
    them: random magnitudes over the whole float range, zeros, single
    nonzero components (exact squares), the smallest subnormal."""
    rng = np.random.default_rng(seed)
    def floats(k):
        f = np.ldexp(1.0 + rng.integers(0, 1 << 23, k) / 2.0 ** 23,
                     rng.integers(-149, 128, k)).astype(np.float32)
        return np.where(rng.random(k) < 0.1, np.float32(0), f).astype(np.float64)
    x, y, z = floats(n), floats(n), floats(n)
    with np.errstate(over="ignore"):
        s = (x * x + y * y) + z * z
    s = s[np.isfinite(s)]
    tiny = np.float64(np.float32(2.0 ** -149)) ** 2
    extra = np.array([0.0, tiny, 2 * tiny, 1.0, 2.0, 4.0, 0.25, 3.0, 1e-30, 1e30, 1e77], np.float64)
    return np.concatenate([s, extra, x * x])


def test_gap_sqrt_matches_ieee(dm):
    """sqrt_sum_of_squares(s) == sqrt(s) bit for bit, against the compiler's
    double square root and numpy's IEEE one, over sums of squares of
    floats (+0 or at least 2^-298)."""
    import torch
    s = sums_of_squares()
    assert np.all((s == 0) | ((s >= 2.0 ** -298) & np.isfinite(s)))
    ts = torch.from_numpy(s).cuda()
    out = torch.empty_like(ts)
    ref = torch.empty_like(ts)
    assert ts.numel() == out.numel() == ref.numel()
    assert dm.devmath_sqrt64(ts.data_ptr(), ts.numel(), out.data_ptr(), ref.data_ptr()) == 0
    got = out.cpu().numpy().view(np.uint64)
    comp = ref.cpu().numpy().view(np.uint64)
    want = np.sqrt(s).view(np.uint64)
    assert np.array_equal(got, comp), int(np.count_nonzero(got != comp))
    miss = np.nonzero(got != want)[0]
    assert len(miss) == 0, (len(miss), [float(s[i]) for i in miss[:6]])
