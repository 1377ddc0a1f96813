"""The persistent site workspace (mhc_workspace_init, mhc_ws_*): a walk over
several sites through caller-owned memory with a ping-pong stream state must be
byte-identical to the allocating entry points (the hyper.rs page, doc comment of
HyperDecodeWs: reuse changes no value), and a HIP graph of that walk, replayed
several times with eager work in between, must reproduce the eager walk on
every replay.  Every site of every walk, and every replay's outputs, are also
compared with the fp64 oracle on every token."""
import numpy as np
import pytest

import oracle
from mhc_inputs import make_norm_weight, make_random_shape
from parity import assert_streams_close, check_site_with_oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
ITERS, EPS, NORM_EPS = 20, 1e-6, 1e-5


@pytest.fixture(scope="module")
def mhc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mhc_hyper_connection_token_amd as m
    m.load_library()
    return m


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _sites(T, S, H, L, seed):
    """L sites: their weights and a branch output f per site (synthetic, fixed)."""
    out = []
    for i in range(L):
        d = make_random_shape(T, S, H, seed=seed + 17 * i)
        out.append({k: _dev(d[k]) for k in ("fn_w", "scale", "base", "f")})
    x0 = _dev(make_random_shape(T, S, H, seed=seed + 1000)["x"])
    return x0, out


def _walk_alloc(mhc, x0, sites, nw=None):
    """The allocating entry points: fresh outputs at every site."""
    x, ys, zq = x0, [], []
    for s in sites:
        if nw is None:
            pre, post, comb, y = mhc.site_pre(x, s["fn_w"], s["scale"], s["base"], ITERS, EPS)
        else:
            pre, post, comb, y, z, q, d = mhc.site_pre_zq8(x, s["fn_w"], s["scale"], s["base"],
                                                           nw, ITERS, EPS, NORM_EPS)
            zq.append((z.clone(), q.clone(), d.clone()))
        ys.append(y.clone())
        x = mhc.site_post(x, s["f"], post, comb)
    torch.cuda.synchronize()
    return x, ys, zq


def _walk_ws(mhc, ws, T, sites, nw=None, record=True, trace=None):
    """The walk through the workspace.  With `trace` (a list), every site appends
    (input state, (pre, post, comb, y), output state), copied out of the
    workspace, for the oracle checks."""
    ys, zq = [], []
    for s in sites:
        x_in = ws.state[:T].clone() if trace is not None else None
        if nw is None:
            ws.site_pre(s["fn_w"], s["scale"], s["base"], ITERS, EPS, T=T)
        else:
            ws.site_pre_zq8(s["fn_w"], s["scale"], s["base"], nw, ITERS, EPS, NORM_EPS, T=T)
            if record:
                zq.append((ws.z[:T].clone(), ws.q[:T].clone(), ws.d[:T].clone()))
        if record:
            ys.append(ws.y[:T].clone())
        outs = ([ws.pre[:T].clone(), ws.post[:T].clone(), ws.comb[:T].clone(),
                 ws.y[:T].clone()] if trace is not None else None)
        ws.site_post(s["f"], T=T)
        if trace is not None:
            trace.append((x_in, outs, ws.state[:T].clone()))
    return ys, zq


def _oracle_check(trace, sites, label):
    """Every site of a traced walk against the fp64 oracle, every token: the pre
    outputs from the site's input state, and its post mix into the next state."""
    for k, (x_in, outs, x_out) in enumerate(trace):
        site = {key: sites[k][key].cpu().numpy() for key in ("fn_w", "scale", "base", "f")}
        check_site_with_oracle(x_in.cpu().numpy(), site, [o.cpu().numpy() for o in outs],
                               ITERS, EPS, f"{label} site {k}", x_out=x_out.cpu().numpy())


@pytest.mark.parametrize("T,S,H,maxT", [(1, 4, 4096, 1), (2, 4, 4096, 4), (7, 3, 1024, 16),
                                        (1, 8, 1024, 2), (130, 4, 4096, 130),
                                        (256, 4, 4096, 260)])
def test_ws_walk_equals_allocating_walk(mhc, T, S, H, maxT):
    print(f"[case] workspace walk T{T} S{S} H{H} max_tokens {maxT}", flush=True)
    x0, sites = _sites(T, S, H, 4, seed=T + S)
    xa, ya, _ = _walk_alloc(mhc, x0, sites)
    ws = mhc.Workspace(maxT, S, H)
    ws.state[:T].copy_(x0)
    trace = []
    yw, _ = _walk_ws(mhc, ws, T, sites, trace=trace)
    torch.cuda.synchronize()
    assert ws.cur == 0  # four posts: back in the first slot
    for i, (u, v) in enumerate(zip(yw, ya)):
        assert torch.equal(u, v), f"site {i}: y differs"
    assert torch.equal(ws.state[:T], xa)
    _oracle_check(trace, sites, f"workspace T{T} S{S} H{H}")


def test_ws_zq8_walk_equals_allocating_walk(mhc):
    T, S, H = 1, 4, 4096
    print("[case] workspace zq8 walk", flush=True)
    x0, sites = _sites(T, S, H, 2, seed=5)
    nw = _dev(make_norm_weight(H))
    xa, ya, za = _walk_alloc(mhc, x0, sites, nw)
    ws = mhc.Workspace(T, S, H)
    ws.state[:T].copy_(x0)
    trace = []
    yw, zw = _walk_ws(mhc, ws, T, sites, nw, trace=trace)
    torch.cuda.synchronize()
    for (u, v) in zip(yw, ya):
        assert torch.equal(u, v)
    for (a, b) in zip(zw, za):
        for u, v in zip(a, b):
            assert torch.equal(u, v)
    assert torch.equal(ws.state[:T], xa)
    _oracle_check(trace, sites, "workspace zq8")
    # the epilogue of every site: the oracle's norm and quantiser on the GPU's y / z
    nwh = nw.cpu().numpy()
    for k, ((z, q, d), y) in enumerate(zip(zw, yw)):
        zh = z.cpu().numpy()
        assert_streams_close(zh, oracle.rmsnorm(y.cpu().numpy(), nwh, NORM_EPS), f"site {k} z")
        qo, do = oracle.q8(zh)
        assert np.array_equal(q.cpu().numpy(), qo) and np.array_equal(d.cpu().numpy(), do)


@pytest.mark.parametrize("T,S,H,use_zq8", [(1, 4, 4096, False), (1, 4, 4096, True),
                                           (4, 4, 4096, False)])
def test_ws_graph_replays_equal_eager_walk(mhc, T, S, H, use_zq8):
    print(f"[case] workspace graph T{T} S{S} H{H} zq8={use_zq8}", flush=True)
    L = 6  # three layers of two sites: an even number of posts
    x0, sites = _sites(T, S, H, L, seed=40 + T)
    nw = _dev(make_norm_weight(H)) if use_zq8 else None
    xa, ya, za = _walk_alloc(mhc, x0, sites, nw)

    ws = mhc.Workspace(T, S, H)
    ws.state[:T].copy_(x0)
    trace = []
    _walk_ws(mhc, ws, T, sites, nw, record=False, trace=trace)  # eager once, traced
    torch.cuda.synchronize()
    _oracle_check(trace, sites, f"workspace graph T{T}")
    # the last site's input state: the replays' last outputs are checked from it
    x_last = trace[-1][0].cpu().numpy()
    last = {key: sites[-1][key].cpu().numpy() for key in ("fn_w", "scale", "base", "f")}
    o_last = oracle.site_pre(x_last, last["fn_w"], last["scale"], last["base"], ITERS,
                             float(np.float32(EPS)))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        _walk_ws(mhc, ws, T, sites, nw, record=False)
    torch.cuda.synchronize()
    assert ws.cur == 0
    other = _dev(make_random_shape(3, S, H, seed=99)["x"])
    for rep in range(3):
        ws.state[:T].copy_(x0)  # eager, outside the graph
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ws.state[:T], xa), f"replay {rep}: final state differs"
        assert torch.equal(ws.y[:T], ya[-1]), f"replay {rep}: last y differs"
        # the replay's own outputs against the oracle: the last site's gates and
        # y, and the final state as its post mix
        check_site_with_oracle(x_last, last, [ws.pre[:T].cpu().numpy(),
                                              ws.post[:T].cpu().numpy(),
                                              ws.comb[:T].cpu().numpy(), ws.y[:T].cpu().numpy()],
                               ITERS, EPS, f"replay {rep}", x_out=ws.state[:T].cpu().numpy(),
                               oracle_pre=o_last)
        if use_zq8:
            for u, v in zip((ws.z[:T], ws.q[:T], ws.d[:T]), za[-1]):
                assert torch.equal(u, v), f"replay {rep}: epilogue differs"
        # eager work of the program's own between replays (library scratch path)
        mhc.site_pre(other, sites[0]["fn_w"], sites[0]["scale"], sites[0]["base"], ITERS, EPS)
        torch.cuda.synchronize()


def test_two_workspaces_on_two_streams(mhc):
    """Each workspace has its own scratch, so two walks may run on two streams at
    once."""
    T, S, H = 1, 4, 4096
    print("[case] two workspaces, two streams", flush=True)
    xa0, sa = _sites(T, S, H, 4, seed=71)
    xb0, sb = _sites(T, S, H, 4, seed=72)
    ra, _, _ = _walk_alloc(mhc, xa0, sa)
    rb, _, _ = _walk_alloc(mhc, xb0, sb)
    wa, wb = mhc.Workspace(T, S, H), mhc.Workspace(T, S, H)
    wa.state[:T].copy_(xa0)
    wb.state[:T].copy_(xb0)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for sa_i, sb_i in zip(sa, sb):
        wa.site_pre(sa_i["fn_w"], sa_i["scale"], sa_i["base"], ITERS, EPS, T=T, stream=s1)
        wb.site_pre(sb_i["fn_w"], sb_i["scale"], sb_i["base"], ITERS, EPS, T=T, stream=s2)
        wa.site_post(sa_i["f"], T=T, stream=s1)
        wb.site_post(sb_i["f"], T=T, stream=s2)
    torch.cuda.synchronize()
    assert torch.equal(wa.state[:T], ra)
    assert torch.equal(wb.state[:T], rb)
    # and both final states against the oracle's walk (the oracle's own gates fed
    # back site after site, so no GPU value enters it)
    for x0, ss, got in ((xa0, sa, wa), (xb0, sb, wb)):
        x = x0.cpu().numpy()
        for s in ss:
            h = {key: s[key].cpu().numpy() for key in ("fn_w", "scale", "base", "f")}
            o = oracle.site_pre(x, h["fn_w"], h["scale"], h["base"], ITERS,
                                float(np.float32(EPS)))
            x = oracle.site_post(x, h["f"], o["post"].astype(np.float32),
                                 o["comb"].astype(np.float32)).astype(np.float32)
        assert_streams_close(got.state[:T].cpu().numpy(), x, "two streams: final state")
