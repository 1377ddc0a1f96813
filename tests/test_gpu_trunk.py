"""GPU parity of the trunk's entry and exit (mhc_expand, mhc_mean, mhc_head)
against the fp64 oracle (O10-O12), plus the exact relations the readings fix."""
import numpy as np
import pytest

import oracle
from mhc_inputs import CONFIGS, make_random_shape, make_site
from parity import assert_gates_close, assert_streams_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def mhc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mhc_hyper_connection_token_amd as m
    m.load_library()
    return m


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _head_weights(S, H, seed):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((S, S * H)) / np.sqrt(S * H)).astype(np.float32)
    scale = rng.uniform(0.5, 1.5, 1).astype(np.float32)
    base = (rng.standard_normal(S) * np.sqrt(0.1)).astype(np.float32)
    return w, scale, base


@pytest.mark.parametrize("T,S,H", [(1, 4, 4096), (3, 1, 4), (17, 3, 132), (300, 8, 256),
                                   (4096, 4, 4096)])
def test_expand_equals_oracle_bit_exact(mhc, T, S, H):
    print(f"[case] expand T{T} S{S} H{H}", flush=True)
    e = np.random.default_rng(T + S).uniform(-1, 1, (T, H)).astype(np.float32)
    x = mhc.expand(_dev(e), S)
    torch.cuda.synchronize()
    assert np.array_equal(x.cpu().numpy(), oracle.expand(e, S))


@pytest.mark.parametrize("T,S,H", [(1, 4, 4096), (3, 1, 4), (17, 3, 132), (300, 8, 256),
                                   (129, 5, 1028)])
def test_mean_matches_oracle(mhc, T, S, H):
    print(f"[case] mean T{T} S{S} H{H}", flush=True)
    x = np.random.default_rng(T * S).uniform(-1, 1, (T, S, H)).astype(np.float32)
    y = mhc.mean(_dev(x))
    torch.cuda.synchronize()
    assert_streams_close(y.cpu().numpy(), oracle.mean(x), f"mean T{T}S{S}H{H}")


@pytest.mark.parametrize("S", [1, 2, 3, 4, 8])
def test_mean_inverts_expand(mhc, S):
    # with one or two streams the fp32 sum of equal copies and the division are
    # exact; from three on the running sum rounds (3e need not be a float), so
    # the mean returns e within the stream tolerance
    print(f"[case] mean(expand) S{S}", flush=True)
    e = np.random.default_rng(S).standard_normal((33, 256)).astype(np.float32)
    y = mhc.mean(mhc.expand(_dev(e), S)).cpu().numpy()
    if S <= 2:
        assert np.array_equal(y, e)
    else:
        assert_streams_close(y, e.astype(np.float64), f"mean(expand) S{S}")


@pytest.mark.parametrize("T,S,H", [(1, 4, 4096), (2, 1, 64), (5, 2, 1024), (17, 3, 132),
                                   (64, 8, 512), (300, 4, 1056), (3, 4, 16384), (9000, 1, 32),
                                   # the fused token tiles (from 256 tokens, S <= 4): ragged
                                   # last tiles, a slab width past the last full column block
                                   (255, 4, 4096), (256, 2, 2052), (259, 3, 1028),
                                   (1001, 4, 4096), (300, 8, 256)])
def test_head_matches_oracle(mhc, T, S, H):
    print(f"[case] head T{T} S{S} H{H}", flush=True)
    x = make_random_shape(T, S, H, seed=T + 11 * S)["x"]
    w, scale, base = _head_weights(S, H, seed=T + S)
    g, y = mhc.head(_dev(x), _dev(w), _dev(scale), _dev(base), 1e-6)
    torch.cuda.synchronize()
    rows = np.unique(np.array([0, 1 % T, T // 2, T - 1, max(0, T - 2)]))
    o = oracle.head(x[rows], w, scale, base, 1e-6)
    assert_gates_close(g.cpu().numpy()[rows], o["gates"], f"head gates T{T}")
    assert_streams_close(y.cpu().numpy()[rows], o["y"], f"head y T{T}")


def test_head_prefill_size_sampled(mhc):
    c = CONFIGS["prefill"]
    d = make_site(c)
    w, scale, base = _head_weights(c.S, c.H, seed=1)
    print("[case] head prefill", flush=True)
    g, y = mhc.head(_dev(d["x"]), _dev(w), _dev(scale), _dev(base), c.eps)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 127, 128, 2047, 4094, 4095])
    o = oracle.head(d["x"][rows], w, scale, base, c.eps)
    assert_gates_close(g.cpu().numpy()[rows], o["gates"], "head prefill gates")
    assert_streams_close(y.cpu().numpy()[rows], o["y"], "head prefill y")


def test_head_with_site_pre_rows_matches_the_site(mhc):
    # the head fed a site's pre rows, first scale and pre biases computes that
    # site's pre gates and branch input (up to fp32 summation order)
    c = CONFIGS["verify8"]
    d = make_site(c)
    S = c.S
    print("[case] head vs site pre", flush=True)
    g, y = mhc.head(_dev(d["x"]), _dev(d["fn_w"][:S]), _dev(d["scale"][:1]),
                    _dev(d["base"][:S]), c.eps)
    pre, post, comb, ys = mhc.site_pre(_dev(d["x"]), _dev(d["fn_w"]), _dev(d["scale"]),
                                       _dev(d["base"]), c.iters, c.eps)
    torch.cuda.synchronize()
    assert_gates_close(g.cpu().numpy(), pre.cpu().numpy().astype(np.float64), "head vs site")
    assert_streams_close(y.cpu().numpy(), ys.cpu().numpy().astype(np.float64), "head y vs site")


def test_head_graph_replays_match_eager(mhc):
    # the fused head packs its weight into the library scratch on every call
    T, S, H = 260, 4, 2048
    print(f"[case] head graph T{T} S{S} H{H}", flush=True)
    x = _dev(make_random_shape(T, S, H, seed=41)["x"])
    x2 = _dev(make_random_shape(T, S, H, seed=42)["x"])
    w, scale, base = (_dev(a) for a in _head_weights(S, H, seed=43))
    w2, scale2, base2 = (_dev(a) for a in _head_weights(S, H, seed=44))
    out = (torch.empty((T, S), device="cuda"), torch.empty((T, H), device="cuda"))
    oth = (torch.empty((T, S), device="cuda"), torch.empty((T, H), device="cuda"))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        mhc.head(x, w, scale, base, 1e-6, out=out)
    torch.cuda.synchronize()
    ref = [t.clone() for t in out]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        mhc.head(x, w, scale, base, 1e-6, out=out)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in out:
            t.fill_(float("nan"))
        with torch.cuda.stream(s):
            mhc.head(x2, w2, scale2, base2, 1e-6, out=oth)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("gates", "y"), out, ref):
            assert torch.equal(a, b), f"replay {rep}: head {name} differs from the eager result"


def test_trunk_zero_tokens(mhc):
    print("[case] trunk T=0", flush=True)
    e = torch.empty((0, 64), device="cuda")
    assert mhc.expand(e, 4).shape == (0, 4, 64)
    assert mhc.mean(torch.empty((0, 4, 64), device="cuda")).shape == (0, 64)
