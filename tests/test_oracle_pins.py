"""Pins for the fp64 oracle: checks against facts fixed by the pages or by
mathematics, not against the oracle's own formulas.

Each test names the part of the method it pins and the mistake it would catch.
The method is the per-token mHC site program of the docs.rs page
"memra_engine 0.125.0 src/memra_engine/hyper.rs" (module documentation,
arithmetic contract; HyperTopology::rows; doc comment of ``post``).
"""
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
from mhc_inputs import CONFIGS, make_random_shape, make_site

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


def _site(T, S, H, seed=7):
    return make_random_shape(T, S, H, seed)


# ---------------------------------------------------------------- page constants
def test_configs_use_the_pages_constants():
    g = json.load(open(GOLDEN))
    prod = g["production_site"]
    for name in ("decode", "verify4", "verify8", "prefill"):
        c = CONFIGS[name]
        assert (c.S, c.H, c.iters) == (prod["streams"], prod["hidden"], prod["sinkhorn_iterations"])
        assert c.eps == prod["eps"]
    mini = g["mini_fixture"]
    c = CONFIGS["tiny"]
    assert (c.S, c.H, c.iters, c.eps) == (mini["hc_mult"], mini["hidden_size"],
                                          mini["hc_sinkhorn_iters"], mini["hc_eps"])
    assert CONFIGS["decode"].R == g["rows_for_four_streams"]["rows"]
    w = g["mixes_weight_shape_production"]
    assert (CONFIGS["decode"].R, CONFIGS["decode"].n) == (w["rows"], w["cols"])


def test_oracle_output_shapes_follow_rows_rule():
    d = make_site(CONFIGS["tiny"])
    o = oracle.site_pre(d["x"], d["fn_w"], d["scale"], d["base"], 20, np.float32(1e-6))
    assert o["mixes"].shape == (4, 24)
    assert o["pre"].shape == (4, 4) and o["post"].shape == (4, 4)
    assert o["comb"].shape == (4, 4, 4) and o["y"].shape == (4, 128)
    with pytest.raises(ValueError):  # three scales, exactly
        oracle.site_pre(d["x"], d["fn_w"], np.ones(2, np.float32), d["base"], 20, 1e-6)


# ---------------------------------------------------------------- O1/O2: RMS rescale
@pytest.mark.parametrize("a", [1e-3, 0.5, 1.0, 3.0])
def test_rms_closed_form_constant_slab(a):
    """x = a everywhere, every fn_w row one-hot: m_r = a / sqrt(a^2 + eps).
    Catches eps outside the root, a missing eps, or a wrong power."""
    S, H, eps = 3, 8, 1e-6
    n, R = S * H, (2 + S) * S
    x = np.full((1, S, H), a, np.float32)
    w = np.zeros((R, n), np.float32)
    for r in range(R):
        w[r, (5 * r) % n] = 1.0
    o = oracle.site_pre(x, w, np.ones(3, np.float32), np.zeros(R, np.float32), 3, eps)
    af = float(np.float32(a))
    want = af / math.sqrt(af * af + eps)
    np.testing.assert_allclose(o["mixes"][0], want, rtol=1e-14, atol=0)


def test_rms_mean_is_over_the_whole_slab():
    """Only stream 0 non-zero: mean(x^2) over S*H is 1/S, so m = 1/sqrt(1/S + eps).
    Catches a mean over hidden only (would give 1/sqrt(1 + eps))."""
    S, H, eps = 4, 8, 1e-6
    n, R = S * H, (2 + S) * S
    x = np.zeros((1, S, H), np.float32)
    x[0, 0, :] = 1.0
    w = np.zeros((R, n), np.float32)
    w[:, 0] = 1.0
    o = oracle.site_pre(x, w, np.ones(3, np.float32), np.zeros(R, np.float32), 2, eps)
    np.testing.assert_allclose(o["mixes"][0], 1.0 / math.sqrt(1.0 / S + eps), rtol=1e-14)


def test_mixes_match_a_library_matvec():
    """GEMV + RMS against numpy's fp64 matmul (a library routine)."""
    d = _site(3, 4, 64, seed=3)
    T, S, H = d["x"].shape
    eps = 1e-6
    o = oracle.site_pre(d["x"], d["fn_w"], d["scale"], d["base"], 5, eps)
    xs = d["x"].reshape(T, S * H).astype(np.float64)
    raw = xs @ d["fn_w"].astype(np.float64).T
    rinv = 1.0 / np.sqrt(np.mean(xs * xs, axis=1) + eps)
    np.testing.assert_allclose(o["mixes"], raw * rinv[:, None], rtol=1e-11, atol=1e-13)


def test_mixes_scale_invariance():
    """m(c*x) ~= m(x) for c*c*mean(x^2) >> eps: the difference is bounded by
    eps/mean(x^2) relatively, and vanishes between two large c."""
    d = _site(2, 4, 32, seed=11)
    x = d["x"]
    args = (d["fn_w"], d["scale"], d["base"], 3, 1e-6)
    m1 = oracle.site_pre(x, *args)["mixes"]
    m2 = oracle.site_pre(x * np.float32(2 ** 10), *args)["mixes"]
    m3 = oracle.site_pre(x * np.float32(2 ** 11), *args)["mixes"]
    ms = np.mean(x.astype(np.float64).reshape(x.shape[0], -1) ** 2, axis=1)  # per token
    assert np.all(np.abs(m2 - m1) <= (2e-6 / ms * np.max(np.abs(m1), axis=1))[:, None] + 1e-12)
    np.testing.assert_allclose(m3, m2, rtol=1e-11, atol=1e-13)
    # and the small-scale side: with c^2*mean ~ eps the mixes shrink as the closed form says
    c = np.float32(2 ** -10)
    m4 = oracle.site_pre(x * c, *args)["mixes"]
    ratio = np.sqrt((ms + 1e-6) / (ms + 1e-6 / float(c) ** 2))
    np.testing.assert_allclose(m4, m1 * ratio[:, None], rtol=1e-9, atol=1e-13)


# ---------------------------------------------------------------- O3/O4: split and gates
def test_gate_rows_order_and_saturation():
    """fn_w = 0 makes z = base.  Saturated bases give exact 0/1 (pre) and 0/2 (post).
    Catches swapped pre/post row blocks, a wrong post factor, or a sigmoid that is
    not 1/(1+exp(-z))."""
    S, H = 4, 8
    R = (2 + S) * S
    x = make_random_shape(1, S, H, 5)["x"]
    base = np.zeros(R, np.float32)
    base[:S] = -1000.0
    base[2] = 1000.0             # pre one-hot at stream 2
    base[S:2 * S] = -1000.0
    base[S + 1] = 1000.0         # post 2.0 at stream 1
    o = oracle.site_pre(x, np.zeros((R, S * H), np.float32), np.ones(3, np.float32), base, 4, 1e-6)
    assert o["pre"][0].tolist() == [0.0, 0.0, 1.0, 0.0]
    assert o["post"][0].tolist() == [0.0, 2.0, 0.0, 0.0]
    base[:] = 0.0
    o = oracle.site_pre(x, np.zeros((R, S * H), np.float32), np.ones(3, np.float32), base, 4, 1e-6)
    assert np.all(o["pre"] == 0.5) and np.all(o["post"] == 1.0)


def test_scale_groups_map_to_row_blocks():
    """Constant slab of ones, one-hot fn_w rows: every m_r = 1/sqrt(1+eps).
    With scale = (0.5, 2, 3) and base = 0: pre = sigma(0.5 m), post = 2 sigma(2 m).
    Catches a row block multiplied by another block's scale."""
    S, H, eps = 4, 4, 1e-6
    n, R = S * H, (2 + S) * S
    x = np.ones((1, S, H), np.float32)
    w = np.zeros((R, n), np.float32)
    for r in range(R):
        w[r, r % n] = 1.0
    scale = np.array([0.5, 2.0, 3.0], np.float32)
    o = oracle.site_pre(x, w, scale, np.zeros(R, np.float32), 7, eps)
    m = 1.0 / math.sqrt(1.0 + eps)
    np.testing.assert_allclose(o["pre"][0], 1.0 / (1.0 + math.exp(-0.5 * m)), rtol=1e-15)
    np.testing.assert_allclose(o["post"][0], 2.0 / (1.0 + math.exp(-2.0 * m)), rtol=1e-15)
    # comb logits all equal 3m: the uniform-block recursion applies (see below)
    a = math.exp(3.0 * m)
    for _ in range(2 * 7):
        a = a / (S * a + eps)
    np.testing.assert_allclose(o["comb"][0], a, rtol=1e-13)


def test_base_is_not_rms_scaled():
    """Doubling x leaves z's base term alone: with fn_w = 0 the gates do not move
    at all when x is scaled.  Catches base folded in before the RMS rescale."""
    S, H = 2, 8
    R = (2 + S) * S
    d = make_random_shape(1, S, H, 9)
    w = np.zeros((R, S * H), np.float32)
    o1 = oracle.site_pre(d["x"], w, d["scale"], d["base"], 3, 1e-6)
    o2 = oracle.site_pre(d["x"] * np.float32(0.001), w, d["scale"], d["base"], 3, 1e-6)
    for k in ("pre", "post", "comb"):
        assert np.array_equal(o1[k], o2[k])


# ---------------------------------------------------------------- O5: Sinkhorn structure
@pytest.mark.parametrize("iters", [1, 2, 3, 7, 20])
@pytest.mark.parametrize("S", [1, 2, 3, 4, 8])
def test_sinkhorn_uniform_block_scalar_recursion(iters, S):
    """Equal logits b: every pass divides each entry a by (S*a + eps), so after
    `iters` row+column rounds every entry is the 2*iters-th term of that scalar
    recursion.  A large eps makes each pass visible: catches a wrong pass count,
    a missing pass, or eps left out of one pass."""
    eps = 0.05
    b = 0.3
    comb = oracle.sinkhorn(np.full((S, S), b), iters, eps)
    a = math.exp(b)
    for _ in range(2 * iters):
        a = a / (S * a + eps)
    np.testing.assert_allclose(comb, a, rtol=1e-14)


@pytest.mark.parametrize("iters", [1, 2, 5, 20, 50])
def test_sinkhorn_cross_ratio_is_invariant(iters):
    """Every pass is a positive diagonal scaling, so comb = D1 exp(Z) D2 and the
    cross ratios of exp(Z) survive at any iteration count and eps.  Catches a
    transposed block, a wrong logit index, or a non-diagonal update."""
    rng = np.random.default_rng(iters)
    for S in (2, 3, 4, 8):
        z = rng.normal(0, 1.0, (S, S))
        comb = oracle.sinkhorn(z, iters, 1e-6)
        for j in range(S):
            for k in range(S):
                cr = comb[j, k] * comb[0, 0] / (comb[j, 0] * comb[0, k])
                assert cr == pytest.approx(math.exp(z[j, k] + z[0, 0] - z[j, 0] - z[0, k]),
                                           rel=1e-12)


def test_site_comb_logits_are_row_major_source_by_target():
    """Site level: with fn_w = 0 the comb logits are base[2S + j*S + k]; the site's
    comb must carry the cross ratios of exactly that (row-major, j = source) block.
    Catches a transposed or mis-offset comb block in the split."""
    S, H = 4, 8
    R = (2 + S) * S
    x = make_random_shape(1, S, H, 6)["x"]
    rng = np.random.default_rng(5)
    base = rng.normal(0, 1.0, R).astype(np.float32)
    o = oracle.site_pre(x, np.zeros((R, S * H), np.float32), np.ones(3, np.float32), base, 20, 1e-6)
    z = base[2 * S:].astype(np.float64).reshape(S, S)
    comb = o["comb"][0]
    for j in range(S):
        for k in range(S):
            cr = comb[j, k] * comb[0, 0] / (comb[j, 0] * comb[0, k])
            assert cr == pytest.approx(math.exp(z[j, k] + z[0, 0] - z[j, 0] - z[0, k]), rel=1e-12)


def test_sinkhorn_ends_on_a_column_pass_and_rows_converge():
    """After the final column pass every column sums to s/(s+eps) (just below 1);
    row sums approach 1 as iterations grow.  One round leaves the rows visibly
    unbalanced (non-vacuity).  Catches row/column order swapped."""
    rng = np.random.default_rng(2)
    eps = 1e-6
    z = rng.normal(0, 1.5, (4, 4))
    prev = None
    for iters in (1, 2, 5, 10, 20, 50, 200):
        c = oracle.sinkhorn(z, iters, eps)
        col = c.sum(axis=0)
        assert np.all(col < 1.0) and np.all(1.0 - col < 4 * eps)
        row_err = np.max(np.abs(c.sum(axis=1) - 1.0))
        if iters == 1:
            assert row_err > 1e-3
        if prev is not None:
            assert row_err <= prev + 1e-12
        prev = row_err
    assert prev < 1e-5


def test_sinkhorn_two_stream_limit_closed_form():
    """S=2, eps -> 0: the doubly stochastic limit is [[p,1-p],[1-p,p]] with
    p = sqrt(C00 C11) / (sqrt(C00 C11) + sqrt(C01 C10))."""
    z = np.array([[0.7, -0.4], [0.2, 1.1]])
    c0 = np.exp(z)
    g = math.sqrt(c0[0, 0] * c0[1, 1])
    h = math.sqrt(c0[0, 1] * c0[1, 0])
    p = g / (g + h)
    comb = oracle.sinkhorn(z, 500, 1e-300)
    np.testing.assert_allclose(comb, [[p, 1 - p], [1 - p, p]], rtol=1e-12)


def test_sinkhorn_rank_one_logits_balance_in_one_round():
    """z_jk = alpha_j + beta_k (rank-one exp(Z)) with eps -> 0: one round gives 1/S."""
    S = 4
    al = np.array([0.3, -1.0, 2.0, 0.1])
    be = np.array([-0.5, 0.4, 1.2, 0.0])
    comb = oracle.sinkhorn(al[:, None] + be[None, :], 1, 1e-300)
    np.testing.assert_allclose(comb, 1.0 / S, rtol=1e-14)


def test_single_stream_site():
    """S=1: three rows; comb is the scalar recursion a <- a/(a+eps) applied 2*iters
    times from exp(z); y = sigma(z0) * x."""
    H, eps, iters = 16, 1e-3, 5
    d = make_random_shape(2, 1, H, 4)
    o = oracle.site_pre(d["x"], d["fn_w"], d["scale"], d["base"], iters, eps)
    for t in range(2):
        m = o["mixes"][t]
        z = [float(d["scale"][g]) * m[g] + float(d["base"][g]) for g in range(3)]
        a = math.exp(z[2])
        for _ in range(2 * iters):
            a = a / (a + eps)
        assert o["comb"][t, 0, 0] == pytest.approx(a, rel=1e-14)
        pre = 1.0 / (1.0 + math.exp(-z[0]))
        np.testing.assert_allclose(o["y"][t], pre * d["x"][t, 0].astype(np.float64), rtol=1e-14)


# ---------------------------------------------------------------- O6: collapse
@pytest.mark.parametrize("c", [0, 1, 3])
def test_collapse_one_hot_returns_that_stream_exactly(c):
    S, H = 4, 64
    R = (2 + S) * S
    d = make_random_shape(3, S, H, 21)
    w = d["fn_w"].copy()
    w[:S] = 0.0
    base = d["base"].copy()
    base[:S] = -1000.0
    base[c] = 1000.0
    o = oracle.site_pre(d["x"], w, d["scale"], base, 20, 1e-6)
    assert np.array_equal(o["y"], d["x"][:, c, :].astype(np.float64))


def test_collapse_half_gates_give_half_the_stream_sum():
    S, H = 4, 32
    R = (2 + S) * S
    d = make_random_shape(2, S, H, 22)
    w = d["fn_w"].copy()
    w[:S] = 0.0
    base = d["base"].copy()
    base[:S] = 0.0
    o = oracle.site_pre(d["x"], w, d["scale"], base, 20, 1e-6)
    want = 0.5 * d["x"].astype(np.float64).sum(axis=1)
    np.testing.assert_allclose(o["y"], want, rtol=1e-15, atol=1e-15)


# ---------------------------------------------------------------- O7: post
def test_post_identity_is_exact():
    """post = 0, comb = I: x' == x bit for bit."""
    S, H = 4, 40
    d = make_random_shape(3, S, H, 31)
    post = np.zeros((3, S), np.float32)
    comb = np.broadcast_to(np.eye(S, dtype=np.float32), (3, S, S)).copy()
    out = oracle.site_post(d["x"], d["f"], post, comb)
    assert np.array_equal(out, d["x"].astype(np.float64))


def test_post_permutation_moves_source_to_target():
    """comb[j,k] = 1 iff k = (j+1) mod S routes source stream j into target k:
    x'[k] = x[k-1].  Catches a transposed comb in the post mix."""
    S, H = 4, 16
    d = make_random_shape(2, S, H, 32)
    comb = np.zeros((2, S, S), np.float32)
    for j in range(S):
        comb[:, j, (j + 1) % S] = 1.0
    out = oracle.site_post(d["x"], d["f"], np.zeros((2, S), np.float32), comb)
    for k in range(S):
        assert np.array_equal(out[:, k], d["x"][:, (k - 1) % S].astype(np.float64))


def test_post_branch_term_scales_f_per_target_stream():
    S, H = 3, 12
    d = make_random_shape(2, S, H, 33)
    post = np.array([[0.5, 2.0, -1.0], [1.0, 0.0, 3.0]], np.float32)
    out = oracle.site_post(d["x"], d["f"], post, np.zeros((2, S, S), np.float32))
    want = post[:, :, None].astype(np.float64) * d["f"][:, None, :].astype(np.float64)
    assert np.array_equal(out, want)


# ---------------------------------------------------------------- whole-site checks
def test_token_independence_is_bit_exact():
    d = make_site(CONFIGS["tiny"])
    a = (d["fn_w"], d["scale"], d["base"], 20, 1e-6)
    full = oracle.site_pre(d["x"], *a, nthreads=3)
    for t in range(d["x"].shape[0]):
        one = oracle.site_pre(d["x"][t:t + 1], *a, nthreads=1)
        for k in ("mixes", "pre", "post", "comb", "y"):
            assert np.array_equal(full[k][t], one[k][0])
    pf = oracle.site_post(d["x"], d["f"], full["post"].astype(np.float32),
                          full["comb"].astype(np.float32), nthreads=2)
    for t in range(d["x"].shape[0]):
        p1 = oracle.site_post(d["x"][t:t + 1], d["f"][t:t + 1],
                              full["post"][t:t + 1].astype(np.float32),
                              full["comb"][t:t + 1].astype(np.float32), nthreads=1)
        assert np.array_equal(pf[t], p1[0])


def _decimal_site(x, w, scale, base, iters, eps):
    """Brute force at 40 significant digits with Python's decimal module, for tiny
    inputs: an independent evaluation of the same steps in another arithmetic."""
    getcontext().prec = 40
    T, S, H = x.shape
    n, R = S * H, (2 + S) * S
    D = Decimal
    e = D(float(eps))
    outs = []
    for t in range(T):
        xs = [D(float(v)) for v in x[t].reshape(-1)]
        ss = sum((v * v for v in xs), D(0))
        rinv = 1 / (ss / n + e).sqrt()
        m = [rinv * sum((D(float(w[r, i])) * xs[i] for i in range(n)), D(0)) for r in range(R)]
        g = [0] * S + [1] * S + [2] * (S * S)
        z = [D(float(scale[g[r]])) * m[r] + D(float(base[r])) for r in range(R)]
        pre = [1 / (1 + (-z[c]).exp()) for c in range(S)]
        post = [2 / (1 + (-z[S + k]).exp()) for k in range(S)]
        C = [[z[2 * S + j * S + k].exp() for k in range(S)] for j in range(S)]
        for _ in range(iters):
            for j in range(S):
                s = sum(C[j], D(0)) + e
                C[j] = [v / s for v in C[j]]
            for k in range(S):
                s = sum((C[j][k] for j in range(S)), D(0)) + e
                for j in range(S):
                    C[j][k] = C[j][k] / s
        y = [sum((pre[c] * xs[c * H + i] for c in range(S)), D(0)) for i in range(H)]
        outs.append((m, pre, post, C, y))
    return outs


@pytest.mark.parametrize("S,H,iters", [(1, 3, 1), (2, 1, 3), (3, 8, 20), (4, 8, 3), (8, 3, 2)])
def test_oracle_matches_high_precision_brute_force(S, H, iters):
    d = make_random_shape(2, S, H, 40 + S)
    eps = float(np.float32(1e-6))
    o = oracle.site_pre(d["x"], d["fn_w"], d["scale"], d["base"], iters, eps)
    ref = _decimal_site(d["x"], d["fn_w"], d["scale"], d["base"], iters, eps)
    for t, (m, pre, post, C, y) in enumerate(ref):
        np.testing.assert_allclose(o["mixes"][t], [float(v) for v in m], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(o["pre"][t], [float(v) for v in pre], rtol=1e-13)
        np.testing.assert_allclose(o["post"][t], [float(v) for v in post], rtol=1e-13)
        np.testing.assert_allclose(o["comb"][t], [[float(v) for v in r] for r in C], rtol=1e-12)
        np.testing.assert_allclose(o["y"][t], [float(v) for v in y], rtol=1e-12, atol=1e-14)


def test_oracle_rejects_what_the_pages_refuse():
    """Zero iterations, non-positive eps, zero streams (HyperTopology::from_plan)."""
    d = make_random_shape(1, 2, 4, 1)
    with pytest.raises(ValueError):
        oracle.site_pre(d["x"], d["fn_w"], d["scale"], d["base"], 0, 1e-6)
    with pytest.raises(ValueError):
        oracle.site_pre(d["x"], d["fn_w"], d["scale"], d["base"], 3, 0.0)
    with pytest.raises(ValueError):
        oracle.sinkhorn(np.zeros((2, 2)), 0, 1e-6)


# ------------------------------------------------------------------ branch-input epilogue
# O8 (RMS norm of y with weight nw) and O9 (q8 codes), hc_fused_gate.rs page, v4z
# timing block.  The page fixes the buffers (z, int8 q[H], fp32 d[H/32]) and the
# norm epsilon 1e-5, not the formulas; the pins below fix what the readings mean.
NORM_EPS = 1e-5


@pytest.mark.parametrize("a", [0.25, 3.0])
def test_rmsnorm_constant_row_closed_form(a):
    H = 64
    y = np.full((1, H), a, dtype=np.float32)
    nw = np.linspace(0.5, 1.5, H).astype(np.float32)
    z = oracle.rmsnorm(y, nw, NORM_EPS)
    want = np.float64(a) / np.sqrt(np.float64(a) ** 2 + NORM_EPS) * nw.astype(np.float64)
    np.testing.assert_allclose(z[0], want, rtol=1e-14, atol=0)


def test_rmsnorm_output_has_unit_weighted_rms_and_scale_invariance():
    rng = np.random.default_rng(11)
    y = rng.standard_normal((3, 256)).astype(np.float32)
    nw = rng.uniform(0.5, 2.0, 256).astype(np.float32)
    z = oracle.rmsnorm(y, nw, NORM_EPS)
    ms = (y.astype(np.float64) ** 2).mean(axis=1)
    # mean((z / nw)^2) = ms / (ms + eps)
    np.testing.assert_allclose(((z / nw) ** 2).mean(axis=1), ms / (ms + NORM_EPS), rtol=1e-12)
    c = 2.0 ** 8
    z2 = oracle.rmsnorm(y * np.float32(c), nw, NORM_EPS)
    # scaling y by c changes z only through eps: z2 / z = sqrt(ms + eps) / sqrt(ms + eps / c^2)
    ratio = np.sqrt(ms + NORM_EPS) / np.sqrt(ms + NORM_EPS / c ** 2)
    np.testing.assert_allclose(z2, z * ratio[:, None], rtol=1e-12)
    # the mean is over the row (hidden), one scale per token
    assert not np.allclose(z[0] / z[0].max(), z[1] / z[1].max())


def test_rmsnorm_matches_high_precision_brute_force():
    rng = np.random.default_rng(5)
    y = rng.standard_normal((2, 40)).astype(np.float32)
    nw = rng.uniform(0.5, 1.5, 40).astype(np.float32)
    z = oracle.rmsnorm(y, nw, NORM_EPS)
    getcontext().prec = 40
    for t in range(2):
        ys = [Decimal(float(v)) for v in y[t]]
        ss = sum((v * v for v in ys), Decimal(0))
        r = 1 / (ss / len(ys) + Decimal(NORM_EPS)).sqrt()
        want = [float(v * r * Decimal(float(w))) for v, w in zip(ys, nw)]
        np.testing.assert_allclose(z[t], want, rtol=1e-14)


def test_q8_scale_is_block_max_over_127_and_the_max_maps_to_127():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((2, 96)).astype(np.float32)
    q, d = oracle.q8(z)
    for t in range(2):
        for b in range(3):
            blk = z[t, 32 * b:32 * b + 32]
            amax = np.max(np.abs(blk))
            assert d[t, b] == np.float32(amax) / np.float32(127.0)
            i = int(np.argmax(np.abs(blk)))
            assert q[t, 32 * b + i] == (127 if blk[i] > 0 else -127)
    assert np.all(np.abs(q.astype(np.int32)) <= 127)
    # reconstruction within half a step
    rec = q.astype(np.float64) * np.repeat(d.astype(np.float64), 32, axis=1)
    step = np.repeat(d.astype(np.float64), 32, axis=1)
    assert np.all(np.abs(rec - z) <= 0.5 * step * (1 + 1e-6) + 1e-12)


def test_q8_ties_round_away_from_zero_and_zero_blocks():
    z = np.zeros((1, 64), dtype=np.float32)
    z[0, 0] = 127.0             # amax 127 -> d = 1, id = 1: codes equal the values
    z[0, 1] = 2.5
    z[0, 2] = -2.5
    z[0, 3] = 0.5
    z[0, 4] = -0.49
    q, d = oracle.q8(z)
    assert d[0, 0] == 1.0 and d[0, 1] == 0.0
    assert list(q[0, :5]) == [127, 3, -3, 1, 0]
    assert np.all(q[0, 32:] == 0)   # an all-zero block: d = 0 and all codes 0


# ------------------------------------------------------------------ trunk entry and exit
# O10 (expand), O11 (mean), O12 (gated head): hyper.rs page, doc comments of
# `expand`, `contract_mean` and `collapse`, and the HyperHead loader (weight
# [S][S*H], bias [S], one scale).  The page names the kernels and shapes only;
# the pins fix what the readings mean.
@pytest.mark.parametrize("S", [1, 3, 4, 8])
def test_expand_copies_the_embedding_into_every_stream(S):
    rng = np.random.default_rng(S)
    e = rng.standard_normal((5, 24)).astype(np.float32)
    x = oracle.expand(e, S)
    assert x.shape == (5, S, 24)
    for k in range(S):
        assert np.array_equal(x[:, k, :], e)


@pytest.mark.parametrize("S", [1, 2, 3, 5, 8])
def test_mean_inverts_expand_exactly(S):
    # the page calls the mean kernel the inverse of the entry; S equal copies
    # summed in double are exact, and so is the division by S
    rng = np.random.default_rng(10 + S)
    e = rng.standard_normal((3, 40)).astype(np.float32)
    assert np.array_equal(oracle.mean(oracle.expand(e, S)), e.astype(np.float64))


def test_mean_known_values_and_brute_force():
    S, H = 4, 6
    x = np.zeros((1, S, H), dtype=np.float32)
    for k in range(S):
        x[0, k, :] = k
    assert np.all(oracle.mean(x) == 1.5)  # (0 + 1 + 2 + 3) / 4
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 3, 10)).astype(np.float32)
    y = oracle.mean(x)
    getcontext().prec = 40
    for t in range(2):
        for i in range(10):
            want = sum((Decimal(float(x[t, k, i])) for k in range(3)), Decimal(0)) / 3
            assert abs(y[t, i] - float(want)) <= 1e-15 * max(1.0, abs(float(want)))


def _head_case(T, S, H, seed):
    rng = np.random.default_rng(seed)
    x = rng.uniform(-1, 1, (T, S, H)).astype(np.float32)
    w = (rng.standard_normal((S, S * H)) / np.sqrt(S * H)).astype(np.float32)
    return x, w


def test_head_with_a_sites_pre_rows_gives_that_sites_pre_gates_and_branch_input():
    # the head is the pre half of a site with its own S rows, one scale and S
    # biases: fed a site's pre rows, scale and biases it must reproduce that
    # site's pre gates and collapse (the site oracle is pinned on its own above)
    d = _site(3, 4, 64, seed=21)
    S = 4
    o = oracle.site_pre(d["x"], d["fn_w"], d["scale"], d["base"], 20, 1e-6)
    h = oracle.head(d["x"], d["fn_w"][:S], d["scale"][:1], d["base"][:S], 1e-6)
    np.testing.assert_allclose(h["gates"], o["pre"], rtol=1e-13, atol=0)
    np.testing.assert_allclose(h["y"], o["y"], rtol=1e-12, atol=1e-15)


def test_head_closed_forms_zero_weight_and_saturation():
    T, S, H = 2, 3, 16
    x, _ = _head_case(T, S, H, 4)
    w = np.zeros((S, S * H), dtype=np.float32)
    base = np.array([0.3, -1.2, 2.0], dtype=np.float32)
    h = oracle.head(x, w, np.array([0.7], np.float32), base, 1e-6)
    g = 1.0 / (1.0 + np.exp(-base.astype(np.float64)))  # the scale multiplies m = 0 only
    np.testing.assert_allclose(h["gates"], np.tile(g, (T, 1)), rtol=1e-15)
    want = np.einsum("c,tci->ti", g, x.astype(np.float64))
    np.testing.assert_allclose(h["y"], want, rtol=1e-13, atol=1e-15)
    # saturated biases pick one stream exactly
    h = oracle.head(x, w, np.array([1.0], np.float32),
                    np.array([-800.0, 800.0, -800.0], np.float32), 1e-6)
    assert np.array_equal(h["gates"], np.tile([0.0, 1.0, 0.0], (T, 1)))
    assert np.array_equal(h["y"], x[:, 1, :].astype(np.float64))


def test_head_matches_high_precision_brute_force():
    T, S, H = 2, 2, 5
    x, w = _head_case(T, S, H, 9)
    scale, base, eps = np.float32(1.3), np.array([0.2, -0.4], np.float32), 1e-6
    h = oracle.head(x, w, np.array([scale]), base, eps)
    getcontext().prec = 40
    n = S * H
    for t in range(T):
        xs = [Decimal(float(v)) for v in x[t].reshape(-1)]
        ss = sum((v * v for v in xs), Decimal(0))
        rinv = 1 / (ss / n + Decimal(eps)).sqrt()
        gates = []
        for c in range(S):
            dot = sum((Decimal(float(a)) * b for a, b in zip(w[c], xs)), Decimal(0))
            z = Decimal(float(scale)) * rinv * dot + Decimal(float(base[c]))
            gates.append(1 / (1 + (-z).exp()))
        np.testing.assert_allclose(h["gates"][t], [float(g) for g in gates], rtol=1e-14)
        for i in range(H):
            want = sum((gates[c] * xs[c * H + i] for c in range(S)), Decimal(0))
            assert abs(h["y"][t, i] - float(want)) <= 1e-14 * max(1.0, abs(float(want)))
