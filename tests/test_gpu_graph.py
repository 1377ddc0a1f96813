"""HIP graph capture of whole sites: every replay equals the eager result bit for bit.

Covers the pre schedules (split partials + finish, the one-token finish with
the branch-input epilogue, packed-weight fused tiles, and at the prefill chunk
the persistent tiles that request half of each next slab into LDS) and the post
kernel.  Every replay is also compared
with the fp64 oracle on every token.  Between replays the program
runs its own eager work (a different site through the same library scratch)
and synchronises, so a replay that depended on state left by the capture, or
on memory cleared only once, would differ.
"""
import numpy as np
import pytest

import oracle
from mhc_inputs import make_random_shape
from parity import assert_streams_close, check_site_with_oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def mhc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mhc_hyper_connection_token_amd as m
    m.load_library()
    return m


def _site(mhc, d, iters, eps, out_pre, out_x):
    mhc.site_pre(d["x"], d["fn_w"], d["scale"], d["base"], iters, eps, out=out_pre)
    mhc.site_post(d["x"], d["f"], out_pre[1], out_pre[2], out=out_x)


def _alloc(T, S, H):
    e = lambda *s: torch.empty(s, device="cuda", dtype=torch.float32)  # noqa: E731
    return (e(T, S), e(T, S), e(T, S, S), e(T, H)), e(T, S, H)


@pytest.mark.parametrize("T,S,H", [(1, 4, 4096), (2, 8, 512), (8, 4, 4096), (130, 4, 1024),
                                   (258, 4, 1024),
                                   # the prefill chunk and the wide site, as the benchmark
                                   # replays them (their eager outputs are parity-tested)
                                   (4096, 4, 4096), (1024, 8, 7168)])
def test_graph_replays_match_eager(mhc, T, S, H):
    print(f"[case] graph T={T} S={S} H={H}", flush=True)
    iters, eps = 20, 1e-6
    d = {k: torch.from_numpy(v).cuda() for k, v in make_random_shape(T, S, H, 5 + T).items()}
    other = {k: torch.from_numpy(v).cuda()
             for k, v in make_random_shape(T, S, H, 99 + T).items()}
    out_pre, out_x = _alloc(T, S, H)
    o_pre, o_x = _alloc(T, S, H)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _site(mhc, d, iters, eps, out_pre, out_x)  # eager reference (also sizes the scratch)
    torch.cuda.synchronize()
    ref = [t.clone() for t in out_pre] + [out_x.clone()]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _site(mhc, d, iters, eps, out_pre, out_x)
    torch.cuda.synchronize()

    host = {k: v.cpu().numpy() for k, v in d.items()}
    o_ref = oracle.site_pre(host["x"], host["fn_w"], host["scale"], host["base"], iters,
                            float(np.float32(eps)))
    for rep in range(3):
        for t in list(out_pre) + [out_x]:
            t.fill_(float("nan"))
        with torch.cuda.stream(s):
            _site(mhc, other, iters, eps, o_pre, o_x)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = list(out_pre) + [out_x]
        for name, a, b in zip(("pre", "post", "comb", "y", "x_out"), got, ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager result"
        # the replay's outputs against the fp64 oracle, every token
        check_site_with_oracle(host["x"], host, [t.cpu().numpy() for t in out_pre], iters, eps,
                               f"graph T{T} S{S} H{H} replay {rep}",
                               x_out=out_x.cpu().numpy(), oracle_pre=o_ref)


def test_graph_replays_match_eager_with_the_epilogue(mhc):
    """One decode token with the branch-input epilogue (partials, then the
    two-block finish) captured in a graph: every replay equals the eager call bit
    for bit, and its pre outputs and z match the fp64 oracle."""
    from mhc_inputs import make_norm_weight
    iters, eps, norm_eps = 20, 1e-6, 1e-5
    T, S, H = 1, 4, 4096
    print("[case] graph T=1 with the epilogue", flush=True)
    d = {k: torch.from_numpy(v).cuda() for k, v in make_random_shape(T, S, H, 21).items()}
    other = {k: torch.from_numpy(v).cuda() for k, v in make_random_shape(T, S, H, 22).items()}
    nw = torch.from_numpy(make_norm_weight(H)).cuda()
    out = mhc.site_pre_zq8(d["x"], d["fn_w"], d["scale"], d["base"], nw, iters, eps, norm_eps)
    o2 = mhc.site_pre_zq8(other["x"], other["fn_w"], other["scale"], other["base"], nw, iters,
                          eps, norm_eps)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mhc.site_pre_zq8(d["x"], d["fn_w"], d["scale"], d["base"], nw, iters, eps, norm_eps,
                         out=out)
    torch.cuda.synchronize()
    ref = [t.clone() for t in out]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        mhc.site_pre_zq8(d["x"], d["fn_w"], d["scale"], d["base"], nw, iters, eps, norm_eps,
                         out=out)
    torch.cuda.synchronize()
    host = {k: v.cpu().numpy() for k, v in d.items()}
    for rep in range(3):
        for t in out:
            t.fill_(0)
        with torch.cuda.stream(s):
            mhc.site_pre_zq8(other["x"], other["fn_w"], other["scale"], other["base"], nw, iters,
                             eps, norm_eps, out=o2)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("pre", "post", "comb", "y", "z", "q", "d"), out, ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager result"
        got = [t.cpu().numpy() for t in out]
        check_site_with_oracle(host["x"], host, got[:4], iters, eps,
                               f"graph epilogue replay {rep}")
        assert_streams_close(got[4], oracle.rmsnorm(got[3], nw.cpu().numpy(), norm_eps),
                             f"graph epilogue replay {rep} z")


def test_graph_survives_scratch_growth_and_capture_refuses_growth(mhc):
    """A graph captured while the library scratch was small stays valid after an
    eager call grows the scratch (the old area is never freed), and a call that
    would have to grow the scratch while its stream is being captured is refused
    with MHC_ECAPTURE before anything is enqueued."""
    iters, eps = 20, 1e-6
    T, S, H = 1, 4, 4096
    print("[case] graph across scratch growth", flush=True)
    d = {k: torch.from_numpy(v).cuda() for k, v in make_random_shape(T, S, H, 11).items()}
    out_pre, out_x = _alloc(T, S, H)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _site(mhc, d, iters, eps, out_pre, out_x)
    torch.cuda.synchronize()
    ref = [t.clone() for t in out_pre] + [out_x.clone()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        _site(mhc, d, iters, eps, out_pre, out_x)
    torch.cuda.synchronize()

    # an eager call whose scratch exceeds anything this suite uses before it (the
    # largest, the decode-exact prefill call, needs 52 MB): the decode-exact path
    # at 4096 tokens, 8 streams, 64 K-ranges x 4096 tokens x 81 floats = 85 MB
    TB, SB, HB = 4096, 8, 1024
    need = 64 * TB * 81 * 4
    assert need > 80 << 20
    big = {k: torch.from_numpy(v).cuda() for k, v in make_random_shape(TB, SB, HB, 12).items()}
    bpre, _ = _alloc(TB, SB, HB)
    mhc.site_pre(big["x"], big["fn_w"], big["scale"], big["base"], iters, eps, out=bpre,
                 exact=True)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in list(out_pre) + [out_x]:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = list(out_pre) + [out_x]
        for name, a, b in zip(("pre", "post", "comb", "y", "x_out"), got, ref):
            assert torch.equal(a, b), f"replay {rep} after growth: {name} differs"

    # growth under capture: refused, nothing enqueued
    TC = 8192  # twice the tokens: more scratch than the current area holds
    assert 64 * TC * 81 * 4 > need + need // 4 + 256
    xc = torch.zeros((TC, SB, HB), device="cuda")
    cpre, _ = _alloc(TC, SB, HB)
    g2 = torch.cuda.CUDAGraph()
    with pytest.raises(mhc.MhcError) as ei:
        with torch.cuda.graph(g2, stream=s):
            mhc.site_pre(xc, big["fn_w"], big["scale"], big["base"], iters, eps, out=cpre,
                         exact=True)
    assert ei.value.status == 6  # MHC_ECAPTURE
    torch.cuda.synchronize()
    # the library still works eagerly afterwards
    with torch.cuda.stream(s):
        _site(mhc, d, iters, eps, out_pre, out_x)
    torch.cuda.synchronize()
    for a, b in zip(list(out_pre) + [out_x], ref):
        assert torch.equal(a, b)
