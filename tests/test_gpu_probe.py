"""GPU check of the bandwidth probe (mhc_bandwidth_probe): the copy moves every
byte, and the read folds every element into its block sums."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def mhc():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mhc_hyper_connection_token_amd as m
    m.load_library()
    return m


@pytest.mark.parametrize("n", [4, 1024, 1000004, 3 << 20])
def test_probe_copy_and_read(mhc, n):
    print(f"[case] bandwidth probe n={n}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(n)
    src = torch.rand(n, device="cuda", generator=g)
    dst = torch.full_like(src, float("nan"))
    mhc.bandwidth_probe(src, dst, True)
    sink = torch.empty(int(mhc.load_library().mhc_probe_sink_floats(n * 4)), device="cuda")
    mhc.bandwidth_probe(src, sink, False)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    want = float(src.double().sum())
    got = float(sink.double().sum())
    assert abs(got - want) <= 1e-5 * abs(want) + 1e-6
