"""GPU checks of the bandwidth probes (tv_fgp_stream_probe and
tv_fgp_stream_probe_ex): what each shape writes, element by element, on a
ragged length (a 16-byte body and a tail), with NaN guard bands around every
volume so that a write outside its volume or a read feeding a result shows."""
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

GUARD = 16  # floats of NaN on each side of every volume (keeps 16-byte alignment)


@pytest.fixture(scope="module")
def tvf():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import stencil_dual_update_amd as m
    return m


def guarded(n, fill, gen):
    """A device volume of n floats inside a NaN band: (view, whole)."""
    whole = torch.full((n + 2 * GUARD,), float("nan"), device="cuda")
    view = whole[GUARD:GUARD + n]
    if fill == "rand":
        view.copy_(torch.rand(n, generator=gen, device="cpu").to("cuda"))
    elif fill is not None:
        view.fill_(fill)
    return view, whole


def bands_intact(whole, n):
    return bool(torch.isnan(whole[:GUARD]).all() and torch.isnan(whole[GUARD + n:]).all())


@pytest.mark.parametrize("n", [1, 3, 4, 1000, 1_000_003])
def test_stream_shapes(tvf, n):
    print("stream probe shapes, n =", n, flush=True)
    gen = torch.Generator().manual_seed(n)
    src = [guarded(n, "rand", gen) for _ in range(7)]
    src0 = [s.clone() for s, _ in src]
    # (7, 6) through both entry points
    for call in (lambda s, d: tvf.tv_fgp_stream_probe(s, d),
                 lambda s, d: tvf.tv_fgp_stream_probe_ex(s, d)):
        dst = [guarded(n, None, gen) for _ in range(6)]
        call([s for s, _ in src], [d for d, _ in dst])
        torch.cuda.synchronize()
        for k in range(6):
            want = src0[k] + src0[6]
            assert torch.equal(dst[k][0].view(torch.int32), want.view(torch.int32))
            assert bands_intact(dst[k][1], n)
    # (1, 1): a copy
    dst = guarded(n, None, gen)
    tvf.tv_fgp_stream_probe_ex([src[3][0]], [dst[0]])
    torch.cuda.synchronize()
    assert torch.equal(dst[0].view(torch.int32), src0[3].view(torch.int32))
    assert bands_intact(dst[1], n)
    # (0, 6): dst[k] = k
    dst = [guarded(n, None, gen) for _ in range(6)]
    tvf.tv_fgp_stream_probe_ex([], [d for d, _ in dst])
    torch.cuda.synchronize()
    for k in range(6):
        assert bool((dst[k][0] == float(k)).all())
        assert bands_intact(dst[k][1], n)
    # (7, 0): reads only
    tvf.tv_fgp_stream_probe_ex([s for s, _ in src], [])
    torch.cuda.synchronize()
    # no source was written
    for (s, whole), s0 in zip(src, src0):
        assert torch.equal(s.view(torch.int32), s0.view(torch.int32))
        assert bands_intact(whole, n)


def test_stream_probe_ex_rejects_in_binding(tvf):
    a = torch.zeros(64, device="cuda")
    with pytest.raises(ValueError):
        tvf.tv_fgp_stream_probe_ex([a, a], [a, a])
    with pytest.raises(ValueError):
        tvf.tv_fgp_stream_probe_ex([a], [torch.zeros(32, device="cuda")])
    with pytest.raises(tvf.TvFgpError):
        tvf.tv_fgp_stream_probe_ex([a], [a])   # the copy's destination is its source
