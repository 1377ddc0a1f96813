"""Comparison rules shared by the GPU parity tests.

Gates (pre, post, comb): element-wise |gpu - oracle| <= 1e-6 + 1e-5 * |oracle|.
Streams (y, x'): max|gpu - oracle| / max(max|oracle|, 1e-6) <= 2e-5, evaluated
per token row: the largest error divided by the largest magnitude of the
expected row, floored at 1e-6 (the measure of the `relative` helper on the
docs.rs page "memra-engine 0.125.0 src/bin/glm5_prime_v2_gate.rs").  Every
output must be finite.
"""
import numpy as np

GATE_RTOL = 1e-5
GATE_ATOL = 1e-6
STREAM_REL = 2e-5


def gate_violation(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    if not np.all(np.isfinite(got)):
        return np.inf
    excess = np.abs(got - want) - (GATE_ATOL + GATE_RTOL * np.abs(want))
    return float(np.max(excess)) if excess.size else -np.inf


def assert_gates_close(got, want, name):
    v = gate_violation(got, want)
    if v > 0:
        got = np.asarray(got, np.float64)
        d = np.abs(got - want)
        i = np.unravel_index(np.argmax(d - GATE_RTOL * np.abs(want)), d.shape)
        raise AssertionError(f"{name}: tolerance exceeded by {v:.3e} at {i}: "
                             f"gpu={got[i]!r} oracle={want[i]!r}")


def relative(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    worst = np.max(np.abs(got - want)) if got.size else 0.0
    scale = max(np.max(np.abs(want)) if want.size else 0.0, 1e-6)
    return float(worst / scale)


def row_profile(got, want):
    """Worst row and per-eighth worst relative error, for failure messages."""
    got = np.asarray(got, np.float64).reshape(want.shape[0], -1)
    want = np.asarray(want, np.float64).reshape(want.shape[0], -1)
    rows = want.shape[0]
    rels = np.array([relative(got[r], want[r]) for r in range(rows)])
    buckets = [float(np.max(rels[b * rows // 8:max((b + 1) * rows // 8, b * rows // 8 + 1)]))
               for b in range(8) if b * rows // 8 < rows]
    r = int(np.argmax(rels))
    return f"rows={rows} worst row {r} rel {rels[r]:.3e}; per-eighth worst {buckets}"


def row_relative(got, want):
    """relative() of every token row: got/want are [T, ...]; returns [T]."""
    got = np.asarray(got, np.float64).reshape(want.shape[0], -1)
    want = np.asarray(want, np.float64).reshape(want.shape[0], -1)
    if got.shape[1] == 0:
        return np.zeros(got.shape[0])
    worst = np.max(np.abs(got - want), axis=1)
    scale = np.maximum(np.max(np.abs(want), axis=1), 1e-6)
    return worst / scale


def assert_streams_close(got, want, name):
    """Per token row relative() <= 2e-5; got/want are [T, ...]."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    if want.shape[0] == 0:
        return
    rels = row_relative(got, want)
    t = int(np.argmax(rels))
    if rels[t] > STREAM_REL:
        raise AssertionError(f"{name}: relative {rels[t]:.3e} > {STREAM_REL} at token {t}; "
                             + row_profile(got, want))


def check_site_with_oracle(x_in, site, outs, iters, eps, label, x_out=None, oracle_pre=None):
    """One site against the fp64 oracle, every token: the pre outputs (pre, post,
    comb, y) from the site's input state x_in, and, with x_out, the post mix of
    the site's f with the GPU's own post and comb gates.  site holds fn_w, scale,
    base (and f); outs = (pre, post, comb, y) as numpy arrays.  Returns the
    oracle's pre outputs."""
    import oracle
    x_in = np.asarray(x_in, np.float32)
    pre, post, comb, y = (np.asarray(o) for o in outs[:4])
    o = oracle_pre or oracle.site_pre(x_in, site["fn_w"], site["scale"], site["base"], iters,
                                      float(np.float32(eps)))
    assert_gates_close(pre, o["pre"], f"{label} pre")
    assert_gates_close(post, o["post"], f"{label} post")
    assert_gates_close(comb, o["comb"], f"{label} comb")
    assert_streams_close(y, o["y"], f"{label} y")
    if x_out is not None:
        want = oracle.site_post(x_in, site["f"], post, comb)
        assert_streams_close(x_out, want, f"{label} x_out")
    return o
