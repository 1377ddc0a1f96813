"""Decode-exact batching (mhc_site_pre_exact): every row of a batched call must be
bit-identical to a solo T=1 call of mhc_site_pre on that token (the hyper.rs
page, doc comment of pre_exact), and within the oracle's tolerances.

Shapes cover the solo decode kernels (T <= 2), the small-batch split (T <= 16),
the sizes where mhc_site_pre switches to its large-batch schedules (the fused
kernel from 256 tokens at S <= 4, wider MFMA tiles above 64 at S > 4), and more
tokens than one pass of the exact path holds (8192).  The K-range per block runs
from 128 floats (one column quad per lane) to 2048 (the long-range kernel)."""
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


def _pre(mhc, d, iters, eps, exact):
    out = mhc.site_pre(_dev(d["x"]), _dev(d["fn_w"]), _dev(d["scale"]), _dev(d["base"]),
                       iters, eps, exact=exact)
    torch.cuda.synchronize()
    return [o.cpu().numpy() for o in out]


def _check(mhc, d, iters, eps, rows, label):
    print(f"[case] exact {label}", flush=True)
    batch = _pre(mhc, d, iters, eps, True)
    for t in rows:
        solo = _pre(mhc, dict(d, x=d["x"][t:t + 1]), iters, eps, False)
        for name, u, v in zip(("pre", "post", "comb", "y"), batch, solo):
            assert np.array_equal(u[t], v[0]), f"{label}: row {t} {name} differs from solo"
    idx = np.asarray(rows)
    o = oracle.site_pre(d["x"][idx], d["fn_w"], d["scale"], d["base"], iters,
                        float(np.float32(eps)))
    pre, post, comb, y = batch
    assert_gates_close(pre[idx], o["pre"], f"{label} pre")
    assert_gates_close(post[idx], o["post"], f"{label} post")
    assert_gates_close(comb[idx], o["comb"], f"{label} comb")
    assert_streams_close(y[idx], o["y"], f"{label} y")
    return batch


@pytest.mark.parametrize("T,S,H", [(1, 4, 4096), (2, 4, 4096), (2, 8, 1024), (3, 4, 4096),
                                   (16, 3, 512), (17, 4, 4096), (40, 8, 1024),
                                   (130, 4, 4096), (129, 6, 512), (300, 2, 1056),
                                   (256, 4, 4096), (65, 8, 1024),
                                   (257, 1, 64), (5, 4, 16384), (3, 2, 65536),
                                   (40, 1, 65536)])
def test_exact_rows_equal_solo(mhc, T, S, H):
    d = make_random_shape(T, S, H, seed=3 * T + S)
    rows = sorted({0, 1 % T, T // 2, T - 1})
    _check(mhc, d, 20, 1e-6, rows, f"T{T}S{S}H{H}")


def test_exact_prefill_rows_equal_solo(mhc):
    c = CONFIGS["prefill"]
    _check(mhc, make_site(c), c.iters, c.eps, [0, 5, 127, 128, 2049, 4095], "prefill")


def test_exact_more_tokens_than_one_pass(mhc):
    d = make_random_shape(8200, 1, 32, seed=11)
    _check(mhc, d, 20, 1e-6, [0, 8191, 8192, 8199], "T8200S1H32")


@pytest.mark.parametrize("T,S,H", [(8, 4, 4096), (255, 4, 4096), (200, 2, 1024), (64, 8, 1024),
                                   (33, 6, 512)])
def test_exact_matches_plain_call_below_the_large_batch_schedules(mhc, T, S, H):
    # below 256 tokens (S <= 4) or up to 64 (S > 4) both entry points run the
    # same kernels with the solo K-split
    d = make_random_shape(T, S, H, seed=7 * T + S)
    print(f"[case] exact vs plain T{T}S{S}H{H}", flush=True)
    for u, v in zip(_pre(mhc, d, 20, 1e-6, True), _pre(mhc, d, 20, 1e-6, False)):
        assert np.array_equal(u, v)


def test_exact_zero_tokens_is_a_no_op(mhc):
    x = torch.empty((0, 4, 128), device="cuda")
    w = torch.zeros((24, 512), device="cuda")
    s = torch.ones(3, device="cuda")
    b = torch.zeros(24, device="cuda")
    print("[case] exact T=0", flush=True)
    pre, post, comb, y = mhc.site_pre(x, w, s, b, 20, 1e-6, exact=True)
    torch.cuda.synchronize()
    assert pre.shape == (0, 4) and y.shape == (0, 128)
