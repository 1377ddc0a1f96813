"""A walk over sites with mhc_site_post_pre (the post half of a site fused with
the pre half of the next) must be bit-identical to the same walk with separate
mhc_site_pre / mhc_site_post calls, and every site (every token, pre outputs and
post mix) within the oracle's tolerances, with and without the branch-input
epilogue."""
import numpy as np
import pytest

from mhc_inputs import make_norm_weight, make_random_shape
from parity import check_site_with_oracle

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
    host = [make_random_shape(T, S, H, seed=seed + 31 * i) for i in range(L)]
    return host[0]["x"], host


def _walk_separate(mhc, x0, sites, nw):
    x, outs = _dev(x0), []
    for s in sites:
        d = {k: _dev(s[k]) for k in ("fn_w", "scale", "base", "f")}
        if nw is None:
            o = mhc.site_pre(x, d["fn_w"], d["scale"], d["base"], ITERS, EPS)
        else:
            o = mhc.site_pre_zq8(x, d["fn_w"], d["scale"], d["base"], nw, ITERS, EPS, NORM_EPS)
        outs.append((x, o))
        x = mhc.site_post(x, d["f"], o[1], o[2])
    torch.cuda.synchronize()
    return x, outs


def _walk_fused(mhc, x0, sites, nw):
    d0 = {k: _dev(sites[0][k]) for k in ("fn_w", "scale", "base", "f")}
    x = _dev(x0)
    if nw is None:
        o = mhc.site_pre(x, d0["fn_w"], d0["scale"], d0["base"], ITERS, EPS)
    else:
        o = mhc.site_pre_zq8(x, d0["fn_w"], d0["scale"], d0["base"], nw, ITERS, EPS, NORM_EPS)
    outs, f = [(x, o)], d0["f"]
    for s in sites[1:]:
        d = {k: _dev(s[k]) for k in ("fn_w", "scale", "base", "f")}
        r = mhc.site_post_pre(x, f, o[1], o[2], d["fn_w"], d["scale"], d["base"], ITERS, EPS,
                              nw=nw, norm_eps=NORM_EPS)
        x, o = r[0], r[1:]
        outs.append((x, o))
        f = d["f"]
    x = mhc.site_post(x, f, o[1], o[2])
    torch.cuda.synchronize()
    return x, outs


# T >= 256, S <= 4: the fused pre kernel with the post prologue; every other
# shape: the post kernel, then the pre chain (small-batch split, the one-token
# finish with the epilogue, MFMA split for S > 4).
@pytest.mark.parametrize("T,S,H,zq", [(256, 4, 4096, False), (300, 4, 1024, False),
                                      (260, 2, 1056, True), (256, 4, 4096, True),
                                      (1, 4, 4096, False), (2, 4, 4096, True),
                                      (5, 2, 1056, False), (17, 3, 512, True),
                                      (64, 4, 1024, False), (200, 4, 4096, False),
                                      (3, 4, 16384, False), (2, 2, 65536, False),
                                      (3, 8, 512, False), (1, 4, 4096, True),
                                      (257, 1, 8192, False),
                                      # the prefill chunk and a ragged tile count
                                      (4096, 4, 4096, False), (1001, 3, 2048, True)])
def test_fused_walk_equals_separate_calls(mhc, T, S, H, zq):
    print(f"[case] walk T{T} S{S} H{H} zq8={zq}", flush=True)
    L = 4
    x0, sites = _sites(T, S, H, L, seed=T + S)
    nw = _dev(make_norm_weight(H)) if zq else None
    xa, oa = _walk_separate(mhc, x0, sites, nw)
    xb, ob = _walk_fused(mhc, x0, sites, nw)
    assert torch.equal(xa, xb), "final state differs"
    for k, ((x1, o1), (x2, o2)) in enumerate(zip(oa, ob)):
        assert torch.equal(x1, x2), f"site {k}: input state differs"
        for u, v in zip(o1, o2):
            assert torch.equal(u, v), f"site {k}: outputs differ"
    # every site of the walk against the oracle, every token: its pre outputs
    # from its input state, and its post mix into the next site's input state
    nxt = [xs for xs, _ in ob[1:]] + [xb]
    for k, ((xs, o), xn) in enumerate(zip(ob, nxt)):
        check_site_with_oracle(xs.cpu().numpy(), sites[k], [v.cpu().numpy() for v in o[:4]],
                               ITERS, EPS, f"walk site {k}", x_out=xn.cpu().numpy())
