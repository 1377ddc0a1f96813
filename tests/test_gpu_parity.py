"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Every case prints what it runs before touching the GPU, so a failing run names
its case.  Tolerances are in tests/parity.py.
"""
import numpy as np
import pytest

import oracle
from mhc_inputs import CONFIGS, make_random_shape, make_site
from parity import (assert_gates_close, assert_streams_close, check_site_with_oracle,
                    gate_violation, relative, STREAM_REL)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.fixture(scope="module")
def mhc():
    _need_gpu()
    import mhc_hyper_connection_token_amd as m
    m.load_library()
    return m


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _run_pre(mhc, d, iters, eps):
    out = mhc.site_pre(_dev(d["x"]), _dev(d["fn_w"]), _dev(d["scale"]), _dev(d["base"]),
                       iters, eps)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in out]


def _run_post(mhc, x, f, post, comb):
    out = mhc.site_post(_dev(x), _dev(f), _dev(post), _dev(comb))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _check_site(mhc, d, iters, eps, tokens=None, label=""):
    """Full pre + post parity.  `tokens` limits the oracle to a sample of token rows."""
    pre, post, comb, y = _run_pre(mhc, d, iters, eps)
    xo = _run_post(mhc, d["x"], d["f"], post, comb)
    idx = np.arange(d["x"].shape[0]) if tokens is None else np.asarray(tokens)
    eps32 = float(np.float32(eps))
    o = oracle.site_pre(d["x"][idx], d["fn_w"], d["scale"], d["base"], iters, eps32)
    assert_gates_close(pre[idx], o["pre"], f"{label} pre")
    assert_gates_close(post[idx], o["post"], f"{label} post")
    assert_gates_close(comb[idx], o["comb"], f"{label} comb")
    assert_streams_close(y[idx], o["y"], f"{label} y")
    # post parity on the GPU's own gates (post and comb taken as given)
    op = oracle.site_post(d["x"][idx], d["f"][idx], post[idx], comb[idx])
    assert_streams_close(xo[idx], op, f"{label} x_out")
    return pre, post, comb, y, xo


# ------------------------------------------------------------------ the five workloads
@pytest.mark.parametrize("name", ["tiny", "decode", "verify4", "verify8"])
def test_config_parity_full(mhc, name):
    c = CONFIGS[name]
    _say(f"config {name} T={c.T} S={c.S} H={c.H}")
    d = make_site(c)
    _check_site(mhc, d, c.iters, c.eps, label=name)


@pytest.mark.parametrize("name", ["prefill", "wide"])
def test_config_parity_full_size_every_token(mhc, name):
    """The prefill chunk (1,024 token tiles of the fused kernel) and the wide site
    (16 64-token tiles of the MFMA partials), every token against the oracle."""
    c = CONFIGS[name]
    _say(f"config {name} T={c.T} S={c.S} H={c.H} (every token)")
    d = make_site(c)
    _check_site(mhc, d, c.iters, c.eps, label=name)


# ------------------------------------------------------------------ ragged and edge shapes
@pytest.mark.parametrize("T,S,H,iters", [
    (1, 1, 4, 1), (2, 2, 8, 3), (3, 3, 12, 20), (5, 4, 132, 20), (16, 4, 4096, 20),
    (17, 4, 260, 7), (33, 5, 36, 20), (70, 6, 52, 20), (19, 7, 1028, 20),
    (9, 8, 7168, 20), (130, 8, 40, 20), (257, 2, 1000, 20), (40, 1, 8196, 50),
    # mid-size batches on the solo K-split (S <= 4, T < 256)
    (127, 4, 4096, 20), (128, 4, 4096, 20), (131, 3, 1028, 20), (129, 4, 68, 20),
    (200, 1, 8192, 20), (255, 2, 4, 5),
    # one token (one-token partial groups): row counts per thread 1, 2, 2, 4 and
    # column quads per lane 1, 2 and 4
    (1, 1, 260, 20), (1, 2, 36, 20), (1, 3, 1028, 20), (1, 4, 8192, 20), (1, 4, 16000, 20),
    # batches large enough for the token-tiled fused kernel (S <= 4, T >= 256)
    (256, 4, 4096, 20), (259, 3, 1028, 20), (300, 2, 4, 5), (261, 4, 2052, 1),
    (257, 4, 68, 20), (320, 1, 8192, 20),
    # S > 4 from 512 tokens: 64-token MFMA blocks with a partly empty last block
    (513, 8, 1024, 20), (700, 6, 516, 20), (1000, 5, 260, 3), (577, 7, 128, 20),
    # the fused tiles at S = 4 with a ragged last tile, and large batches of
    # every stream count (a tile count the grid does not divide, 200 Sinkhorn
    # rounds, the largest token count of the ragged set)
    (1025, 4, 1024, 20), (2047, 4, 2048, 1), (512, 4, 4096, 20), (513, 3, 1536, 20),
    (1040, 2, 512, 20), (4097, 4, 4096, 20), (5000, 1, 3072, 7), (700, 4, 2048, 200),
    (2100, 3, 4096, 20), (8192, 2, 1024, 20),
    # large batches whose slab does not fit the fused tiles (split path)
    (600, 4, 4100, 20), (1030, 2, 2560, 20),
])
def test_ragged_shapes(mhc, T, S, H, iters):
    _say(f"ragged T={T} S={S} H={H} iters={iters}")
    d = make_random_shape(T, S, H, seed=T * 7 + S)
    _check_site(mhc, d, iters, 1e-6, label=f"T{T}S{S}H{H}")


def test_zero_tokens_is_a_no_op(mhc):
    _say("T=0")
    x = torch.empty((0, 4, 64), device="cuda")
    w = torch.zeros((24, 256), device="cuda")
    out = mhc.site_pre(x, w, torch.ones(3, device="cuda"), torch.zeros(24, device="cuda"), 20, 1e-6)
    assert out[3].shape == (0, 64)
    xo = mhc.site_post(x, torch.empty((0, 64), device="cuda"), out[1], out[2])
    torch.cuda.synchronize()
    assert xo.shape == (0, 4, 64)


def test_many_iterations_and_larger_eps(mhc):
    c = CONFIGS["tiny"]
    d = make_site(c)
    for iters, eps in ((1, 1e-6), (200, 1e-6), (20, 1e-3)):
        _say(f"tiny iters={iters} eps={eps}")
        _check_site(mhc, d, iters, eps, label=f"iters{iters}")


# ------------------------------------------------------------------ exact special cases
def test_one_hot_pre_returns_the_stream_bit_exact(mhc):
    c = CONFIGS["verify4"]
    d = make_site(c)
    S = c.S
    for chosen in range(S):
        _say(f"one-hot pre stream {chosen}")
        w = d["fn_w"].copy()
        w[:S] = 0.0
        base = d["base"].copy()
        base[:S] = -1000.0
        base[chosen] = 1000.0
        pre, post, comb, y = _run_pre(mhc, dict(d, fn_w=w, base=base), c.iters, c.eps)
        assert np.array_equal(pre, np.eye(S, dtype=np.float32)[chosen][None].repeat(c.T, 0))
        assert np.array_equal(y, d["x"][:, chosen, :])


def test_identity_post_is_bit_exact(mhc):
    c = CONFIGS["verify8"]
    d = make_site(c)
    _say("post = 0, comb = I")
    post = np.zeros((c.T, c.S), np.float32)
    comb = np.broadcast_to(np.eye(c.S, dtype=np.float32), (c.T, c.S, c.S)).copy()
    xo = _run_post(mhc, d["x"], d["f"], post, comb)
    assert np.array_equal(xo, d["x"])


def test_permutation_post_routes_source_to_target(mhc):
    S, H, T = 8, 512, 3
    d = make_random_shape(T, S, H, 77)
    _say("post permutation")
    comb = np.zeros((T, S, S), np.float32)
    for j in range(S):
        comb[:, j, (j + 3) % S] = 1.0
    xo = _run_post(mhc, d["x"], d["f"], np.zeros((T, S), np.float32), comb)
    for k in range(S):
        assert np.array_equal(xo[:, k], d["x"][:, (k - 3) % S])


def test_uniform_comb_block_entries_are_identical(mhc):
    c = CONFIGS["decode"]
    d = make_site(c)
    S, eps, iters = c.S, 0.05, 7
    _say("uniform comb logits")
    w = d["fn_w"].copy()
    w[2 * S:] = 0.0
    base = d["base"].copy()
    base[2 * S:] = 0.3
    pre, post, comb, y = _run_pre(mhc, dict(d, fn_w=w, base=base), iters, eps)
    assert np.all(comb == comb.reshape(-1)[0])
    a = np.exp(np.float64(0.3))
    for _ in range(2 * iters):
        a = a / (S * a + np.float32(eps))
    assert abs(comb.reshape(-1)[0] - a) <= 1e-6 + 1e-5 * a


# ------------------------------------------------------------------ determinism, invariance
def test_run_twice_is_bit_identical(mhc):
    c = CONFIGS["verify8"]
    d = make_site(c)
    _say("determinism")
    a = _run_pre(mhc, d, c.iters, c.eps)
    b = _run_pre(mhc, d, c.iters, c.eps)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_small_batch_rows_equal_solo_decode_bit_exact(mhc):
    c = CONFIGS["verify8"]
    d = make_site(c)
    _say("T-invariance within the small-batch plan")
    batch = _run_pre(mhc, d, c.iters, c.eps)
    for t in (0, 3, 7):
        solo = _run_pre(mhc, dict(d, x=d["x"][t:t + 1]), c.iters, c.eps)
        for u, v in zip(batch, solo):
            assert np.array_equal(u[t], v[0])


def test_end_to_end_post_from_oracle_gates(mhc):
    c = CONFIGS["verify4"]
    d = make_site(c)
    _say("post from oracle gates")
    o = oracle.site_pre(d["x"], d["fn_w"], d["scale"], d["base"], c.iters, float(np.float32(c.eps)))
    post32 = o["post"].astype(np.float32)
    comb32 = o["comb"].astype(np.float32)
    xo = _run_post(mhc, d["x"], d["f"], post32, comb32)
    assert_streams_close(xo, oracle.site_post(d["x"], d["f"], post32, comb32), "x_out")


def test_red_arm_one_iteration_off_is_detected(mhc):
    """Non-vacuity: an oracle run with one Sinkhorn round fewer must NOT pass."""
    c = CONFIGS["tiny"]
    d = make_site(c)
    _say("red arm")
    pre, post, comb, y = _run_pre(mhc, d, 3, c.eps)
    o = oracle.site_pre(d["x"], d["fn_w"], d["scale"], d["base"], 2, float(np.float32(c.eps)))
    assert gate_violation(comb, o["comb"]) > 0


def test_native_library_is_loaded(mhc):
    maps = open("/proc/self/maps").read()
    assert mhc.LIB_PATH in maps


def test_large_batch_shapes_alternate(mhc):
    """Large batches of different shapes (1 to 4 streams, fused tiles and the
    split path) share the library scratch; calls that alternate between them
    must each match the oracle on every token."""
    seq = [(700, 4, 4096), (513, 3, 1536), (600, 2, 2048), (1040, 1, 512), (700, 4, 4096),
           (513, 3, 1536), (530, 4, 512), (600, 2, 2048)]
    for i, (T, S, H) in enumerate(seq):
        _say(f"alternating group shapes: call {i} T={T} S={S} H={H}")
        d = make_random_shape(T, S, H, seed=400 + i)
        _check_site(mhc, d, 20, 1e-6, label=f"call{i} T{T}S{S}H{H}")


# ------------------------------------------------------------------ the largest batch accepted
@pytest.mark.parametrize("S,H", [(4, 4096), (8, 7168)])
def test_largest_accepted_batch(mhc, S, H):
    """T*S*H one short of 2^31, the largest batch the calls accept (the fused
    token tiles at S = 4, the split path at S = 8): byte offsets into x and x'
    pass 2^31 and 2^32.  x and f are drawn on the device (U[-1, 1), like the
    configs, from a seeded generator); the outputs of a sample of tokens (the
    first and last, both sides of each byte-offset power of two, and random
    ones) are compared with the oracle run on those tokens alone, which is
    exact because a token's outputs depend only on its own slab."""
    n = S * H
    T = (2 ** 31 - 1) // n
    _say(f"largest batch T={T} S={S} H={H}")
    small = make_random_shape(1, S, H, seed=4242 + S)
    g = torch.Generator(device="cuda").manual_seed(1000 + S)
    x = torch.empty((T, S, H), device="cuda").uniform_(-1.0, 1.0, generator=g)
    f = torch.empty((T, H), device="cuda").uniform_(-1.0, 1.0, generator=g)
    fn_w, scale, base = _dev(small["fn_w"]), _dev(small["scale"]), _dev(small["base"])
    pre, post, comb, y = mhc.site_pre(x, fn_w, scale, base, 20, 1e-6)
    xo = mhc.site_post(x, f, post, comb)
    torch.cuda.synchronize()
    pick = {0, 1, T - 2, T - 1}
    for k in (31, 32, 33):
        t = (2 ** k + 4 * n - 1) // (4 * n)  # first token whose slab starts at or past 2^k bytes
        pick.update(u for u in (t - 1, t) if 0 <= u < T)
    pick.update(np.random.default_rng(7 + S).choice(T, 24, replace=False).tolist())
    idx = torch.tensor(sorted(pick), device="cuda")
    site = {"fn_w": small["fn_w"], "scale": small["scale"], "base": small["base"],
            "f": f[idx].cpu().numpy()}
    outs = [o[idx].cpu().numpy() for o in (pre, post, comb, y)]
    xs, xos = x[idx].cpu().numpy(), xo[idx].cpu().numpy()
    del x, f, pre, post, comb, y, xo
    torch.cuda.empty_cache()
    check_site_with_oracle(xs, site, outs, 20, 1e-6, f"largest T{T}S{S}H{H}", x_out=xos)


# ------------------------------------------------------------------ persistent tiles
@pytest.mark.parametrize("S,H", [(4, 4096), (2, 8192), (3, 2048), (4, 4000), (1, 1100)])
def test_persistent_tiles_match_the_fused_tiles_bit_for_bit(mhc, S, H):
    """From two 4-token tiles per compute unit the pre chain runs on a
    persistent grid that requests half of each next slab into LDS; smaller
    batches (from 256 tokens) run one block per tile.  Both compute a tile the
    same way, so the rows of one large batch equal, bit for bit, those of the
    same tokens run in batches below the threshold (every batch a multiple of
    four tokens, so the tiles line up, and at least 256 tokens, so none takes
    the split path).  The batch ends on a ragged tile; H = 4000 and 1100 leave
    the last chunks of some waves past the hidden size.  The whole batch is
    also checked against the oracle, every token."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    step = 4 * cus                 # one tile per compute unit
    T = 4 * step + 261             # over four tiles per unit, ragged end
    _say(f"persistent tiles T={T} S={S} H={H} ({cus} compute units)")
    d = make_random_shape(T, S, H, seed=7000 + S)
    whole = _run_pre(mhc, d, 20, 1e-6)
    cuts = list(range(0, 4 * step + 1, step)) + [T]
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        sub = {k: d[k][a:b] if k in ("x", "f") else d[k] for k in d}
        parts.append(_run_pre(mhc, sub, 20, 1e-6))
    for i, name in enumerate(("pre", "post", "comb", "y")):
        joined = np.concatenate([p[i] for p in parts])
        assert np.array_equal(whole[i], joined), f"{name} differs between the two schedules"
    check_site_with_oracle(d["x"], d, list(whole), 20, 1e-6, f"persistent T{T}S{S}H{H}")
