"""GPU check of the pre-packed weight (mhc_pack_weight, mhc_site_pre_packed):
the packed call gives bit-identical outputs to mhc_site_pre on every schedule
(the large-batch kernel reads the packed weight, the small-batch path fn_w),
and matches the fp64 oracle."""
import numpy as np
import pytest

import oracle
from mhc_inputs import make_random_shape
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


@pytest.mark.parametrize("T,S,H", [(1, 4, 4096), (300, 4, 4096), (4096, 4, 4096),
                                   (261, 3, 1028), (257, 1, 8192), (300, 2, 4),
                                   # a hidden size with a partly padded last column block
                                   (300, 4, 1056), (513, 4, 3000)])
def test_packed_equals_plain(mhc, T, S, H):
    print(f"[case] packed T={T} S={S} H={H}", flush=True)
    d = {k: torch.from_numpy(v).cuda() for k, v in make_random_shape(T, S, H, seed=T + S).items()}
    packed = mhc.pack_weight(d["fn_w"], S, H)
    a = mhc.site_pre(d["x"], d["fn_w"], d["scale"], d["base"], 20, 1e-6)
    b = mhc.site_pre(d["x"], d["fn_w"], d["scale"], d["base"], 20, 1e-6, packed=packed)
    torch.cuda.synchronize()
    for name, u, v in zip(("pre", "post", "comb", "y"), a, b):
        assert torch.equal(u, v), f"{name} differs between the packed and the plain call"
    # and against the oracle on a few rows
    rows = np.unique(np.array([0, T // 2, T - 1]))
    h = {k: v.cpu().numpy() for k, v in d.items()}
    o = oracle.site_pre(h["x"][rows], h["fn_w"], h["scale"], h["base"], 20,
                        float(np.float32(1e-6)))
    got = [t.cpu().numpy()[rows] for t in b]
    assert_gates_close(got[0], o["pre"], "packed pre")
    assert_gates_close(got[1], o["post"], "packed post")
    assert_gates_close(got[2], o["comb"], "packed comb")
    assert_streams_close(got[3], o["y"], "packed y")


def test_no_packed_form_for_wide_sites(mhc):
    T, S, H = 300, 8, 256
    print(f"[case] packed wide T={T} S={S} H={H}", flush=True)
    assert mhc.packed_weight_bytes(S, H) == 0
    d = {k: torch.from_numpy(v).cuda() for k, v in make_random_shape(T, S, H, seed=9).items()}
    with pytest.raises(mhc.MhcError):
        mhc.pack_weight(d["fn_w"], S, H)


@pytest.mark.parametrize("T,S,H", [(2, 4, 4096), (300, 4, 4096), (4096, 4, 4096), (259, 3, 1028)])
def test_packed_walk_equals_plain_walk(mhc, T, S, H):
    print(f"[case] packed walk T={T} S={S} H={H}", flush=True)
    a = {k: torch.from_numpy(v).cuda() for k, v in make_random_shape(T, S, H, seed=1).items()}
    b = {k: torch.from_numpy(v).cuda() for k, v in make_random_shape(T, S, H, seed=2).items()}
    p0, q0, c0, _ = mhc.site_pre(a["x"], a["fn_w"], a["scale"], a["base"], 20, 1e-6)
    packed = mhc.pack_weight(b["fn_w"], S, H)
    plain = mhc.site_post_pre(a["x"], a["f"], q0, c0, b["fn_w"], b["scale"], b["base"], 20, 1e-6)
    pk = mhc.site_post_pre(a["x"], a["f"], q0, c0, b["fn_w"], b["scale"], b["base"], 20, 1e-6,
                           packed=packed)
    torch.cuda.synchronize()
    for name, u, v in zip(("x_out", "pre", "post", "comb", "y"), plain, pk):
        assert torch.equal(u, v), f"{name} differs between the packed and the plain walk"


def test_packed_calls_with_zero_tokens(mhc):
    S, H = 4, 4096
    print("[case] packed T=0", flush=True)
    w = torch.zeros(((2 + S) * S, S * H), device="cuda")
    packed = mhc.pack_weight(w, S, H)
    x = torch.empty((0, S, H), device="cuda")
    out = mhc.site_pre(x, w, torch.ones(3, device="cuda"), torch.zeros(24, device="cuda"), 20,
                       1e-6, packed=packed)
    torch.cuda.synchronize()
    assert out[3].shape == (0, H)
