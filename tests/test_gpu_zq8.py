"""GPU parity of the branch-input epilogue (mhc_site_pre_zq8): the RMS norm of y
with a norm weight and its q8 codes, against the fp64 oracle.

z is compared with the oracle's norm of the GPU's own y (isolating the
epilogue) and with the oracle's norm of the oracle's y (end to end).  The int8
codes and block scales are decided in fp32, so they must equal, bit for bit,
the oracle's fp32 quantiser applied to the z the GPU wrote; against the
oracle's quantiser on the oracle's own z they agree within the stream
tolerance (scales) and one step (codes)."""
import numpy as np
import pytest

import oracle
from mhc_inputs import CONFIGS, make_norm_weight, make_random_shape, make_site
from parity import assert_streams_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
NORM_EPS = 1e-5


@pytest.fixture(scope="module")
def mhc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mhc_hyper_connection_token_amd as m
    m.load_library()
    return m


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _check(mhc, d, iters, eps, label, tokens=None):
    H = d["x"].shape[2]
    nw = make_norm_weight(H)
    print(f"[case] zq8 {label}", flush=True)
    out = mhc.site_pre_zq8(_dev(d["x"]), _dev(d["fn_w"]), _dev(d["scale"]), _dev(d["base"]),
                           _dev(nw), iters, eps, NORM_EPS)
    plain = mhc.site_pre(_dev(d["x"]), _dev(d["fn_w"]), _dev(d["scale"]), _dev(d["base"]),
                         iters, eps)
    torch.cuda.synchronize()
    pre, post, comb, y, z, q, dd = [o.cpu().numpy() for o in out]
    # the pre outputs are those of mhc_site_pre
    for a, b in zip((pre, post, comb, y), plain):
        assert np.array_equal(a, b.cpu().numpy())
    idx = np.arange(y.shape[0]) if tokens is None else np.asarray(tokens)
    # epilogue alone: the oracle's norm of the GPU's y
    assert_streams_close(z[idx], oracle.rmsnorm(y[idx], nw, NORM_EPS), f"{label} z (given y)")
    # end to end: the oracle's norm of the oracle's y
    o = oracle.site_pre(d["x"][idx], d["fn_w"], d["scale"], d["base"], iters, float(np.float32(eps)))
    zo = oracle.rmsnorm(o["y"].astype(np.float32), nw, NORM_EPS)
    assert_streams_close(z[idx], zo, f"{label} z (end to end)")
    # codes and scales: the fp32 quantiser on the GPU's z, bit for bit
    qo, do = oracle.q8(z[idx])
    assert np.array_equal(dd[idx], do), f"{label}: block scales differ"
    assert np.array_equal(q[idx], qo), f"{label}: q8 codes differ"
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    # end to end: the oracle's quantiser on the oracle's own z (rounded to fp32,
    # the precision the codes are decided in).  z differs by at most the stream
    # tolerance, so each scale is within it (relative to the token's largest
    # scale) and a code moves by at most one step where z sits near a rounding
    # boundary.
    qe, de = oracle.q8(zo.astype(np.float32))
    assert_streams_close(dd[idx], de, f"{label} block scales (end to end)")
    dq = np.abs(q[idx].astype(np.int32) - qe.astype(np.int32))
    assert dq.max(initial=0) <= 1, f"{label}: a code differs by {dq.max()} end to end"


@pytest.mark.parametrize("name", ["tiny", "decode", "verify4", "verify8"])
def test_zq8_configs(mhc, name):
    c = CONFIGS[name]
    _check(mhc, make_site(c), c.iters, c.eps, name)


def test_zq8_prefill_every_token(mhc):
    c = CONFIGS["prefill"]
    _check(mhc, make_site(c), c.iters, c.eps, "prefill")


# Paths: one token with S <= 4 runs the epilogue in its two-block finish,
# T >= 256 with an on-chip slab in the fused kernel's tail, everything else as
# a launch of its own after the split path.
@pytest.mark.parametrize("T,S,H", [(1, 1, 32), (1, 2, 64), (1, 3, 4608), (1, 4, 8192), (2, 4, 4096), (2, 3, 4608),
                                   (2, 4, 8192), (2, 8, 7168), (3, 2, 64), (17, 4, 1024),
                                   (128, 2, 1056), (130, 4, 4096), (131, 1, 8192),
                                   (256, 2, 1056), (258, 4, 4096), (259, 1, 8192),
                                   (129, 3, 8192)])
def test_zq8_shapes(mhc, T, S, H):
    d = make_random_shape(T, S, H, seed=T + 5 * S)
    _check(mhc, d, 20, 1e-6, f"T{T}S{S}H{H}")


def test_zq8_zero_input_gives_zero_codes(mhc):
    c = CONFIGS["tiny"]
    d = make_site(c)
    d = dict(d, x=np.zeros_like(d["x"]))
    nw = make_norm_weight(c.H)
    print("[case] zq8 zero slab", flush=True)
    out = mhc.site_pre_zq8(_dev(d["x"]), _dev(d["fn_w"]), _dev(d["scale"]), _dev(d["base"]),
                           _dev(nw), c.iters, c.eps, NORM_EPS)
    torch.cuda.synchronize()
    y, z, q, dd = [o.cpu().numpy() for o in out[3:]]
    assert np.all(y == 0) and np.all(z == 0) and np.all(q == 0) and np.all(dd == 0)


def test_zq8_decode_token_matches_its_row_in_a_batch(mhc):
    """One decode token (its own two-block finish with the epilogue) against the
    same token as row 0 of a two-token batch (the split path, then the
    standalone epilogue launch): the same partials and the same sums, so every
    output is equal bit for bit."""
    c = CONFIGS["decode"]
    d = make_site(c)
    d2 = make_random_shape(2, c.S, c.H, seed=77)
    x2 = np.concatenate([d["x"], d2["x"][1:]], axis=0)
    nw = make_norm_weight(c.H)
    print("[case] zq8 decode token vs batched row", flush=True)
    one = mhc.site_pre_zq8(_dev(d["x"]), _dev(d["fn_w"]), _dev(d["scale"]), _dev(d["base"]),
                           _dev(nw), c.iters, c.eps, NORM_EPS)
    two = mhc.site_pre_zq8(_dev(x2), _dev(d["fn_w"]), _dev(d["scale"]), _dev(d["base"]),
                           _dev(nw), c.iters, c.eps, NORM_EPS)
    torch.cuda.synchronize()
    for name, a, b in zip(("pre", "post", "comb", "y", "z", "q", "d"), one, two):
        assert np.array_equal(a.cpu().numpy()[0], b.cpu().numpy()[0]), name
