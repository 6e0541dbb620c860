"""Property test of the C ABI's overlap rule (no GPU, nothing launched).

Every call that writes device buffers must refuse (TV_ERR_ALIAS) exactly when
a written buffer shares a byte with any other buffer of the call, and accept
otherwise.  Here the buffers of tv_fgp_run are placed at random offsets in a
fake address range, so that they touch, overlap by a few bytes or stay apart,
and the library's answer is compared with a byte-range model.  The runs have
zero inner steps, so a call that passes validation enqueues nothing and no
address is dereferenced.
"""
import ctypes

import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

tvf = pytest.importorskip("stencil_dual_update_amd", reason="libtvfgp.so not built")
L = tvf.lib

NX, NY, NZ = 4, 3, 2
VOL = NX * NY * NZ * 4          # bytes per volume
BASE = 1 << 40                  # fake, never dereferenced
P3 = ctypes.c_void_p * 3

# offsets in 4-byte units over a window a few volumes wide, so that random
# placements overlap often but not always
offsets = st.integers(min_value=0, max_value=6 * VOL // 4).map(lambda k: BASE + 4 * k)


def overlaps(a, b, n):
    return a < b + n and b < a + n


def model_alias(bufs):
    """bufs: (address, bytes, written); True if a written buffer overlaps
    another buffer."""
    for i, (a, na, wa) in enumerate(bufs):
        for c, nc, wc in bufs[i + 1:]:
            if (wa or wc) and a < c + nc and c < a + na:
                return True
    return False


@settings(max_examples=400, deadline=None)
@given(b=offsets, p=st.lists(offsets, min_size=3, max_size=3),
       ra=st.lists(offsets, min_size=3, max_size=3), rb=st.lists(offsets, min_size=3, max_size=3))
def test_run_refuses_exactly_the_overlapping_layouts(b, p, ra, rb):
    bufs = [(b, VOL, False)] + [(x, VOL, True) for x in p + ra + rb]
    where = ctypes.c_int(-1)
    st_ = L.tv_fgp_run(b, P3(*p), P3(*ra), P3(*rb), 0.01, 1, 0, NX, NY, NZ, 0, None, None,
                       ctypes.byref(where))
    assert st_ == (tvf.TV_ERR_ALIAS if model_alias(bufs) else tvf.TV_OK)


@settings(max_examples=300, deadline=None)
@given(b=offsets, p=st.lists(offsets, min_size=3, max_size=3),
       ra=st.lists(offsets, min_size=3, max_size=3), rb=st.lists(offsets, min_size=3, max_size=3),
       ws=offsets)
def test_run_with_workspace_refuses_exactly_the_overlapping_layouts(b, p, ra, rb, ws):
    # the three-step run's workspace is a second p: three volumes
    bufs = ([(b, VOL, False)] + [(x, VOL, True) for x in p + ra + rb]
            + [(ws, 3 * VOL, True)])
    where = ctypes.c_int(-1)
    st_ = L.tv_fgp_run(b, P3(*p), P3(*ra), P3(*rb), 0.01, 1, 0, NX, NY, NZ, tvf.TB3, ws, None,
                       ctypes.byref(where))
    assert st_ == (tvf.TV_ERR_ALIAS if model_alias(bufs) else tvf.TV_OK)


def test_touching_buffers_do_not_overlap():
    # buffers that end exactly where the next begins share no byte
    addrs = [BASE + k * VOL for k in range(10)]
    where = ctypes.c_int(-1)
    st_ = L.tv_fgp_run(addrs[0], P3(*addrs[1:4]), P3(*addrs[4:7]), P3(*addrs[7:10]), 0.01, 1, 0,
                       NX, NY, NZ, 0, None, None, ctypes.byref(where))
    assert st_ == tvf.TV_OK
    # one byte of overlap is refused (alignment kept: move by 4 bytes)
    st_ = L.tv_fgp_run(addrs[0], P3(*addrs[1:4]), P3(*addrs[4:7]),
                       P3(addrs[7], addrs[8], addrs[9] - 4), 0.01, 1, 0, NX, NY, NZ, 0, None,
                       None, ctypes.byref(where))
    assert st_ == tvf.TV_ERR_ALIAS
