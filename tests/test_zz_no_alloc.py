"""mhc_site_pre_static, the pre call for callers that cannot allocate device
memory: its kernel scratch is the library's fixed 16 MiB device array.  Through
the C ABI it must give what mhc_site_pre gives, within the oracle tolerances,
on calls in a row whose sizes shrink (the array keeps the previous call's
contents), and refuse a shape whose scratch does not fit before enqueuing
anything."""
import numpy as np
import pytest

from mhc_inputs import CONFIGS, make_random_shape, make_site
from parity import assert_gates_close, assert_streams_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
STATIC_BYTES = 16 << 20


@pytest.fixture(scope="module")
def mhc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mhc_hyper_connection_token_amd as m
    m.load_library()
    return m


def _dev(d):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda") for k, v in d.items()}


def _pair(mhc, d, iters, eps, label):
    """The static-scratch call, then the plain call, on the same inputs."""
    T, S, H = d["x"].shape
    print(f"[case] static scratch {label} T={T} S={S} H={H}", flush=True)
    assert mhc.site_pre_scratch_bytes(T, S, H) - 256 <= STATIC_BYTES
    got = mhc.site_pre(d["x"], d["fn_w"], d["scale"], d["base"], iters, eps,
                       static_scratch=True)
    torch.cuda.synchronize()
    got = [o.cpu().numpy() for o in got]
    ref = mhc.site_pre(d["x"], d["fn_w"], d["scale"], d["base"], iters, eps)
    torch.cuda.synchronize()
    ref = [o.cpu().numpy().astype(np.float64) for o in ref]
    for name, a, b in zip(("pre", "post", "comb"), got[:3], ref[:3]):
        assert_gates_close(a, b, f"{label} {name}")
    assert_streams_close(got[3], ref[3], f"{label} y")


def test_static_scratch_calls_in_a_row_match_the_plain_call(mhc):
    # the prefill chunk (token-tiled kernel: the packed weight in the array),
    # then a smaller verify batch (split path: partial sums over the previous
    # call's packed weight), then the wide site (the largest partials), then the
    # decode site
    for name in ("prefill", "verify8", "wide", "decode"):
        c = CONFIGS[name]
        _pair(mhc, _dev(make_site(c)), c.iters, c.eps, name)


def test_static_scratch_ragged_shapes(mhc):
    for T, S, H in ((1025, 4, 1024), (257, 3, 1028), (3, 2, 65536), (70, 6, 52)):
        _pair(mhc, _dev(make_random_shape(T, S, H, seed=T + S)), 20, 1e-6, "ragged")


def test_static_scratch_refuses_what_does_not_fit(mhc):
    T, S, H = 65536, 8, 4  # one K-range: 65536 tokens x 81 floats = 21 MB of partials
    assert mhc.site_pre_scratch_bytes(T, S, H) - 256 > STATIC_BYTES
    print("[case] static scratch too small: refused on the host", flush=True)
    x = torch.zeros((T, S, H), device="cuda")
    R = (2 + S) * S
    w = torch.zeros((R, S * H), device="cuda")
    with pytest.raises(mhc.MhcError) as ei:
        mhc.site_pre(x, w, torch.ones(3, device="cuda"), torch.zeros(R, device="cuda"), 20,
                     1e-6, static_scratch=True)
    assert ei.value.status == 3  # MHC_EUNSUPPORTED
    torch.cuda.synchronize()


def test_static_scratch_inside_a_graph(mhc):
    """The call allocates nothing, so it can be captured even at a size no earlier
    call has used; every replay equals the eager result."""
    T, S, H = 300, 4, 2048
    print("[case] static scratch captured", flush=True)
    d = _dev(make_random_shape(T, S, H, seed=9))
    e = lambda *s: torch.empty(s, device="cuda")  # noqa: E731
    out = (e(T, S), e(T, S), e(T, S, S), e(T, H))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mhc.site_pre(d["x"], d["fn_w"], d["scale"], d["base"], 20, 1e-6, out=out,
                     static_scratch=True)
    torch.cuda.synchronize()
    ref = [t.clone() for t in out]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        mhc.site_pre(d["x"], d["fn_w"], d["scale"], d["base"], 20, 1e-6, out=out,
                     static_scratch=True)
    torch.cuda.synchronize()
    other = _dev(make_random_shape(8, S, H, seed=10))
    for rep in range(3):
        for t in out:
            t.fill_(float("nan"))
        # eager work through the same array between replays
        mhc.site_pre(other["x"], other["fn_w"], other["scale"], other["base"], 20, 1e-6,
                     static_scratch=True)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("pre", "post", "comb", "y"), out, ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs"
