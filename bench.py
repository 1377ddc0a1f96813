#!/usr/bin/env python3
"""Benchmark of the mHC site program (pre + post) on one MI355X.

A step is one whole site over one batch of synthetic input already resident in
HBM: mhc_site_pre (mixes, RMS rescale, gates, Sinkhorn, collapse) followed by
mhc_site_post (post mix).  The timed workload is the prefill chunk (T=4096
tokens, 4 streams, hidden 4096, 20 Sinkhorn iterations, eps 1e-6): `value` is
its token throughput, timed as one replay of the K sites captured in a HIP
graph (the eager per-call figures ride along).  The same JSON line carries the decode site (T=1) in
microseconds per site, the HBM roofline of the dominant kernel, and the CPU
oracle's throughput on the host as a baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
       python bench.py --kernels-only N      # a few launches for rocprofv3 runs
       python bench.py --write-traffic FETCH_DB WRITE_DB   # counters -> profiles/
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "mHC site tokens/s + HBM GB/s (% peak), streams=4 d=4096; µs/site at T=1"
PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_prefill.json")


def kernel_source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "mhc_hyper_connection_token_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# kernel -> the source files whose change invalidates its measured traffic
KERNEL_SOURCES = {
    "post_kernel": ["mhc_post.hip", "mhc_device.h"],
    "pre_kernel": ["mhc_fused.hip", "mhc_device.h"],
    "pre_call": ["mhc_fused.hip", "mhc_device.h"],
    "walk_call": ["mhc_fused.hip", "mhc_device.h"],
    "wide_pre_call": ["mhc_partials.hip", "mhc_split.h", "mhc_finish.hip", "mhc_device.h"],
    "wide_post_kernel": ["mhc_post.hip", "mhc_device.h"],
}


def algorithmic_bytes(T, S, H):
    R = (2 + S) * S
    pre = 4 * (T * (S * H + H + 2 * S + S * S) + R * S * H + 3 + R)
    post = 4 * T * (2 * S * H + H + S + S * S)
    return pre, post


def to_dev(d, torch):
    return {k: torch.from_numpy(v).to("cuda") for k, v in d.items()}


def alloc_out(T, S, H, torch):
    e = lambda *s: torch.empty(s, device="cuda", dtype=torch.float32)  # noqa: E731
    return (e(T, S), e(T, S), e(T, S, S), e(T, H)), e(T, S, H)


def run_kernels_only(n, mhc, torch, CONFIGS, make_site, workloads=("prefill", "decode")):
    """A handful of launches of each workload kernel plus a plain 256 MiB device
    copy (the reference for scaling rocprof's byte counters).  With the prefill
    workload it also runs n walk steps (a site's post fused with the next pre)."""
    for name in workloads:
        c = CONFIGS[name]
        t = to_dev(make_site(c), torch)
        (pre_o, xo) = alloc_out(c.T, c.S, c.H, torch)
        for _ in range(n):
            mhc.site_pre(t["x"], t["fn_w"], t["scale"], t["base"], c.iters, c.eps, out=pre_o)
            mhc.site_post(t["x"], t["f"], pre_o[1], pre_o[2], out=xo)
        torch.cuda.synchronize()
        print(f"[kernels-only] {name}: {n} sites", flush=True)
        if name == "prefill":
            nxt, _ = alloc_out(c.T, c.S, c.H, torch)
            for _ in range(n):
                mhc.site_post_pre(t["x"], t["f"], pre_o[1], pre_o[2], t["fn_w"], t["scale"],
                                  t["base"], c.iters, c.eps, out=(xo,) + tuple(nxt))
            torch.cuda.synchronize()
            print(f"[kernels-only] {name}: {n} walk steps", flush=True)
    src = torch.empty(64 << 20, device="cuda", dtype=torch.float32)
    dst = torch.empty_like(src)
    for _ in range(n):
        dst.copy_(src)
    torch.cuda.synchronize()
    print("[kernels-only] copy 256 MiB done", flush=True)


def time_site(mhc, torch, t, c, out_pre, out_x, steps, warmup):
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        mhc.site_pre(t["x"], t["fn_w"], t["scale"], t["base"], c.iters, c.eps, out=out_pre)
        mhc.site_post(t["x"], t["f"], out_pre[1], out_pre[2], out=out_x)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        ev[i][0].record(stream)
        mhc.site_pre(t["x"], t["fn_w"], t["scale"], t["base"], c.iters, c.eps, out=out_pre)
        ev[i][1].record(stream)
        mhc.site_post(t["x"], t["f"], out_pre[1], out_pre[2], out=out_x)
        ev[i][2].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    eager_ms = start.elapsed_time(end) / steps
    pre_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    post_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps

    # The timed steps: the `steps` sites (pre + post each) captured in one HIP
    # graph, as a trunk captures its sites, and replayed once, so that only
    # device time and the gaps between kernels count.  One untimed replay first
    # (the scratch was sized by the eager calls above).
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for _ in range(steps):
            mhc.site_pre(t["x"], t["fn_w"], t["scale"], t["base"], c.iters, c.eps, out=out_pre)
            mhc.site_post(t["x"], t["f"], out_pre[1], out_pre[2], out=out_x)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(side):
        start.record(side)
        g.replay()
        end.record(side)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end) / steps, pre_ms, post_ms, wall, eager_ms


def time_kernels_alone(mhc, torch, t, c, out_pre, out_x, calls=20, reps=5):
    """Device µs per launch of the token-tiled pre kernel and of the post kernel,
    each from time_graph (HIP graph of `calls` launches, HIP events on its
    stream).  The pre kernel is timed where a site step runs it, right after the
    weight pack: a graph of (pack, packed-weight pre call) pairs less a graph of
    the packs alone.  Back to back with itself it runs slower; that figure is
    returned as well."""
    packed = mhc.pack_weight(t["fn_w"], c.S, c.H)
    torch.cuda.synchronize()

    def pre_packed():
        mhc.site_pre(t["x"], t["fn_w"], t["scale"], t["base"], c.iters, c.eps, out=out_pre,
                     packed=packed)

    def pack():
        mhc.pack_weight(t["fn_w"], c.S, c.H, out=packed)

    def pack_then_pre():
        pack()
        pre_packed()

    back_to_back_us = time_graph(torch, pre_packed, calls=calls, reps=reps)
    pack_us = time_graph(torch, pack, calls=calls, reps=reps)
    pair_us = time_graph(torch, pack_then_pre, calls=calls, reps=reps)
    post_us = time_graph(torch, lambda: mhc.site_post(
        t["x"], t["f"], out_pre[1], out_pre[2], out=out_x), calls=calls, reps=reps)
    del packed
    return {"pre_kernel_us": pair_us - pack_us, "pre_kernel_back_to_back_us": back_to_back_us,
            "pack_kernel_us": pack_us, "post_kernel_us": post_us}


def time_site_packed(mhc, torch, t, c, out_pre, out_x, steps):
    """The timed steps of time_site with the site's weight packed once beforehand
    (mhc_pack_weight, outside the timed region) and read by mhc_site_pre_packed:
    K sites in one HIP graph, replayed once after one untimed replay.  Returns ms
    per step, or None when the shape has no packed form."""
    if mhc.packed_weight_bytes(c.S, c.H) == 0:
        return None
    packed = mhc.pack_weight(t["fn_w"], c.S, c.H)
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for _ in range(3):
            mhc.site_pre(t["x"], t["fn_w"], t["scale"], t["base"], c.iters, c.eps, out=out_pre,
                         packed=packed)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for _ in range(steps):
            mhc.site_pre(t["x"], t["fn_w"], t["scale"], t["base"], c.iters, c.eps, out=out_pre,
                         packed=packed)
            mhc.site_post(t["x"], t["f"], out_pre[1], out_pre[2], out=out_x)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(side):
        g.replay()
        a.record(side)
        g.replay()
        b.record(side)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def time_decode(mhc, torch, t, c, out_pre, out_x, sites, graph_sites=50, zq8=None):
    """Decode sites back to back on one stream: (a) eager calls, no per-call events
    (host launch cost included); (b) a HIP graph of `graph_sites` sites replayed,
    which leaves only device time and the gaps between kernels.  Returns µs/site
    for both.  With zq8=(nw, norm_eps, out7) the pre half is the call with the
    branch-input epilogue."""
    def site():
        if zq8 is None:
            mhc.site_pre(t["x"], t["fn_w"], t["scale"], t["base"], c.iters, c.eps, out=out_pre)
            po, pc = out_pre[1], out_pre[2]
        else:
            nw, neps, o7 = zq8
            mhc.site_pre_zq8(t["x"], t["fn_w"], t["scale"], t["base"], nw, c.iters, c.eps, neps,
                             out=o7)
            po, pc = o7[1], o7[2]
        mhc.site_post(t["x"], t["f"], po, pc, out=out_x)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        for _ in range(50):
            site()
        torch.cuda.synchronize()
        a.record(s)
        for _ in range(sites):
            site()
        b.record(s)
    torch.cuda.synchronize()
    eager_us = a.elapsed_time(b) * 1e3 / sites

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(graph_sites):
            site()
    torch.cuda.synchronize()
    reps = max(2, sites // graph_sites)
    with torch.cuda.stream(s):
        g.replay()
        a.record(s)
        for _ in range(reps):
            g.replay()
        b.record(s)
    torch.cuda.synchronize()
    graph_us = a.elapsed_time(b) * 1e3 / (reps * graph_sites)
    return eager_us, graph_us


def fit_line(xs, ys):
    """Least-squares line through the points (xs, ys): (slope, intercept)."""
    n = len(xs)
    if n < 2 or len(ys) != n:
        raise ValueError("need at least two (x, y) points")
    mx, my = sum(xs) / n, sum(ys) / n
    sxx = sum((a - mx) ** 2 for a in xs)
    if sxx == 0:
        raise ValueError("the x values are all equal")
    slope = sum((a - mx) * (b - my) for a, b in zip(xs, ys)) / sxx
    return slope, my - slope * mx


def time_cold_decode(mhc, torch, c, sets=200, reps=5):
    """Decode sites (T=1) rotating through `sets` distinct weight / state / branch
    sets (1.5 MiB of weight each at 4 x 4096, so 200 sets exceed the 256 MB
    memory-side cache), one HIP graph of `sets` sites, replayed; against the
    same graph over one set.  Returns µs per site for both."""
    from mhc_inputs import make_random_shape
    base_set = make_random_shape(c.T, c.S, c.H, seed=1)
    g = torch.Generator(device="cuda").manual_seed(11)
    R = (2 + c.S) * c.S
    pool = []
    for _ in range(sets):
        pool.append({
            "x": torch.rand((c.T, c.S, c.H), device="cuda", generator=g) * 2 - 1,
            "fn_w": torch.randn((R, c.S * c.H), device="cuda", generator=g) / (c.S * c.H) ** 0.5,
            "scale": torch.rand(3, device="cuda", generator=g) + 0.5,
            "base": torch.randn(R, device="cuda", generator=g) * 0.1 ** 0.5,
            "f": torch.rand((c.T, c.H), device="cuda", generator=g) * 2 - 1})
    warm = to_dev(base_set, torch)
    (o_pre, o_x) = alloc_out(c.T, c.S, c.H, torch)

    def graph_us(seq):
        def run():
            for st in seq:
                mhc.site_pre(st["x"], st["fn_w"], st["scale"], st["base"], c.iters, c.eps,
                             out=o_pre)
                mhc.site_post(st["x"], st["f"], o_pre[1], o_pre[2], out=o_x)
        return time_graph(torch, run, calls=1, reps=reps) / len(seq)
    cold_us = graph_us(pool)
    warm_us = graph_us([warm] * sets)
    del pool
    torch.cuda.empty_cache()
    return {"sets": sets, "cold_us_per_site": round(cold_us, 3),
            "warm_us_per_site": round(warm_us, 3),
            "note": "decode sites (T=1, S=4, H=4096) in one HIP graph: cold rotates through "
                    "distinct weight/state/branch sets (about 1.6 MB each, more than the "
                    "memory-side cache in total); warm repeats one set"}


def run_bandwidth_probe(mhc, torch, gib=1, reps=20):
    """HBM rate of a plain stream on this part: mhc_bandwidth_probe copying and
    reading `gib` GiB (streaming 16-byte loads and stores), HIP events around
    `reps` calls."""
    n = (gib << 30) // 4
    src = torch.empty(n, device="cuda", dtype=torch.float32).uniform_(-1, 1)
    dst = torch.empty_like(src)
    sink = torch.empty(int(mhc.load_library().mhc_probe_sink_floats(n * 4)), device="cuda",
                       dtype=torch.float32)
    copy_us = time_calls(torch, lambda: mhc.bandwidth_probe(src, dst, True), reps, 3)
    read_us = time_calls(torch, lambda: mhc.bandwidth_probe(src, sink, False), reps, 3)
    nbytes = n * 4
    del src, dst, sink
    torch.cuda.empty_cache()
    copy_gbps = 2 * nbytes / (copy_us * 1e-6) / 1e9
    read_gbps = nbytes / (read_us * 1e-6) / 1e9
    return {"bytes": nbytes, "copy_us": round(copy_us, 2), "read_us": round(read_us, 2),
            "copy_GBps": round(copy_gbps, 1), "read_GBps": round(read_gbps, 1),
            "copy_frac_of_peak": round(copy_gbps / PEAK_HBM_GBPS, 4),
            "read_frac_of_peak": round(read_gbps / PEAK_HBM_GBPS, 4),
            "note": "mhc_bandwidth_probe: a plain copy (read + write counted) and a plain "
                    "read of 1 GiB, the rate a pure stream reaches on this part against the "
                    "published 8 TB/s"}


def time_pre_zq8(mhc, torch, t, c, nw, norm_eps, out7, steps, warmup):
    """Mean µs of the pre call with the branch-input epilogue, back to back on the
    current stream (HIP events around each call)."""
    def call():
        mhc.site_pre_zq8(t["x"], t["fn_w"], t["scale"], t["base"], nw, c.iters, c.eps, norm_eps,
                         out=out7)
    return time_calls(torch, call, steps, warmup)


def time_pre_variant(mhc, torch, t, c, out_pre, exact, steps, warmup):
    """Mean µs of one pre call (plain or decode-exact), back to back."""
    def call():
        mhc.site_pre(t["x"], t["fn_w"], t["scale"], t["base"], c.iters, c.eps, out=out_pre,
                     exact=exact)
    return time_calls(torch, call, steps, warmup)


def time_calls(torch, call, steps, warmup):
    """Mean µs of call() over `steps` back-to-back calls on the current stream
    (HIP events around each call)."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record(stream)
        call()
        b.record(stream)
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / steps * 1e3


def zq8_bytes(T, H):
    """Algorithmic HBM bytes of the epilogue on its own: read y and nw; write z,
    the int8 codes and one fp32 scale per 32 columns."""
    return 4 * T * H + 4 * H + 4 * T * H + T * H + 4 * (T * H // 32)


def alloc_zq8(T, S, H, torch):
    e = lambda *s, dt=torch.float32: torch.empty(s, device="cuda", dtype=dt)  # noqa: E731
    return (e(T, S), e(T, S), e(T, S, S), e(T, H), e(T, H), e(T, H, dt=torch.int8),
            e(T, H // 32))


def time_graph(torch, fn, calls=20, reps=5):
    """Device µs per call: `calls` calls captured in a HIP graph on a side
    stream, replayed `reps` times (HIP events around the replays)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(calls):
            fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(s):
        g.replay()
        a.record(s)
        for _ in range(reps):
            g.replay()
        b.record(s)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (calls * reps)


def time_ws_decode(mhc, torch, td, cd, sites=50, reps=20):
    """Decode sites through a persistent workspace: a HIP graph of `sites` sites
    (pre + post, the state ping-ponging between the workspace's two slots),
    replayed; µs per site."""
    ws = mhc.Workspace(cd.T, cd.S, cd.H)
    ws.state[:cd.T].copy_(td["x"])

    def walk():
        for _ in range(sites):
            ws.site_pre(td["fn_w"], td["scale"], td["base"], cd.iters, cd.eps, T=cd.T)
            ws.site_post(td["f"], T=cd.T)
    return time_graph(torch, walk, calls=1, reps=reps) / sites


def time_walk(mhc, torch, c, x0, L, steps, warmup):
    """A walk over L sites of the prefill chunk (each site its own synthetic
    weights and branch output f, drawn on the device): (a) separate pre and post
    calls per site, (b) the post half of each site fused with the next site's pre
    (mhc_site_post_pre).  Returns (separate_us, fused_us) per site."""
    T, S, H = c.T, c.S, c.H
    R = (2 + S) * S
    g = torch.Generator(device="cuda").manual_seed(7)
    sites = []
    for _ in range(L):
        sites.append({
            "fn_w": torch.randn((R, S * H), device="cuda", generator=g) / (S * H) ** 0.5,
            "scale": torch.rand(3, device="cuda", generator=g) + 0.5,
            "base": torch.randn(R, device="cuda", generator=g) * 0.1 ** 0.5,
            "f": torch.rand((T, H), device="cuda", generator=g) * 2 - 1})
    e = lambda *s: torch.empty(s, device="cuda", dtype=torch.float32)  # noqa: E731
    xs = [x0, e(T, S, H), e(T, S, H)]
    gates = [(e(T, S), e(T, S), e(T, S, S), e(T, H)) for _ in range(2)]

    def separate():
        x = xs[0]
        for k, st in enumerate(sites):
            o = gates[k % 2]
            mhc.site_pre(x, st["fn_w"], st["scale"], st["base"], c.iters, c.eps, out=o)
            xn = xs[1 + k % 2]
            mhc.site_post(x, st["f"], o[1], o[2], out=xn)
            x = xn

    def fused():
        o = gates[0]
        mhc.site_pre(xs[0], sites[0]["fn_w"], sites[0]["scale"], sites[0]["base"], c.iters,
                     c.eps, out=o)
        x = xs[0]
        for k in range(1, L):
            st, prev = sites[k], sites[k - 1]
            on = gates[k % 2]
            xn = xs[1 + k % 2]
            mhc.site_post_pre(x, prev["f"], o[1], o[2], st["fn_w"], st["scale"], st["base"],
                              c.iters, c.eps, out=(xn,) + tuple(on))
            x, o = xn, on
        mhc.site_post(x, sites[-1]["f"], o[1], o[2], out=xs[1 + L % 2])

    packs = ([mhc.pack_weight(st["fn_w"], S, H) for st in sites]
             if mhc.packed_weight_bytes(S, H) else None)

    def fused_packed():
        o = gates[0]
        mhc.site_pre(xs[0], sites[0]["fn_w"], sites[0]["scale"], sites[0]["base"], c.iters,
                     c.eps, out=o, packed=packs[0])
        x = xs[0]
        for k in range(1, L):
            st, prev = sites[k], sites[k - 1]
            on = gates[k % 2]
            xn = xs[1 + k % 2]
            mhc.site_post_pre(x, prev["f"], o[1], o[2], st["fn_w"], st["scale"], st["base"],
                              c.iters, c.eps, out=(xn,) + tuple(on), packed=packs[k])
            x, o = xn, on
        mhc.site_post(x, sites[-1]["f"], o[1], o[2], out=xs[1 + L % 2])

    return (time_calls(torch, separate, steps, warmup) / L,
            time_calls(torch, fused, steps, warmup) / L,
            time_graph(torch, separate, calls=4, reps=3) / L,
            time_graph(torch, fused, calls=4, reps=3) / L,
            (time_graph(torch, fused_packed, calls=4, reps=3) / L) if packs else None)


def time_decode_walk(mhc, torch, c, x0, L=50, zq8=False, distinct=4):
    """Decode sites (T=1) chained as a trunk runs them, `distinct` site weights
    in rotation, in one HIP graph: the first pre, then mhc_site_post_pre per
    site, then the last post; with zq8 every pre carries the branch-input
    epilogue.  Returns µs per site (graph replay)."""
    T, S, H = c.T, c.S, c.H
    R = (2 + S) * S
    g = torch.Generator(device="cuda").manual_seed(11)
    sites = [{"fn_w": torch.randn((R, S * H), device="cuda", generator=g) / (S * H) ** 0.5,
              "scale": torch.rand(3, device="cuda", generator=g) + 0.5,
              "base": torch.randn(R, device="cuda", generator=g) * 0.1 ** 0.5,
              "f": torch.rand((T, H), device="cuda", generator=g) * 2 - 1}
             for _ in range(distinct)]
    nw = torch.rand(H, device="cuda", generator=g) + 0.5
    e = lambda *s, dt=torch.float32: torch.empty(s, device="cuda", dtype=dt)  # noqa: E731
    xs = [x0.clone(), e(T, S, H), e(T, S, H)]
    outs = [(e(T, S), e(T, S), e(T, S, S), e(T, H), e(T, H), e(T, H, dt=torch.int8),
             e(T, H // 32)) for _ in range(2)]

    def walk():
        st = sites[0]
        o = outs[0]
        if zq8:
            mhc.site_pre_zq8(xs[0], st["fn_w"], st["scale"], st["base"], nw, c.iters, c.eps,
                             out=o)
        else:
            mhc.site_pre(xs[0], st["fn_w"], st["scale"], st["base"], c.iters, c.eps, out=o[:4])
        x = xs[0]
        for k in range(1, L):
            st, prev = sites[k % distinct], sites[(k - 1) % distinct]
            on = outs[k % 2]
            xn = xs[1 + k % 2]
            mhc.site_post_pre(x, prev["f"], o[1], o[2], st["fn_w"], st["scale"], st["base"],
                              c.iters, c.eps, nw=nw if zq8 else None,
                              out=(xn,) + tuple(on if zq8 else on[:4]))
            x, o = xn, on
        mhc.site_post(x, sites[(L - 1) % distinct]["f"], o[1], o[2], out=xs[1 + L % 2])
    return time_graph(torch, walk, calls=1, reps=20) / L


def run_sweep(mhc, torch):
    """Device time of the pre call, plain and decode-exact, over T (one JSON line
    per shape)."""
    from mhc_inputs import make_random_shape
    for (S, H) in [(4, 4096), (2, 4096), (8, 7168)]:
        for T in (1, 2, 4, 16, 17, 32, 64, 96, 128, 192, 256, 384, 512, 1024, 2048, 4096):
            if S == 8 and T > 1024:
                continue
            t = to_dev(make_random_shape(T, S, H, seed=T), torch)
            out, _ = alloc_out(T, S, H, torch)
            res = {}
            for name, exact in (("plain_us", False), ("exact_us", True)):
                res[name] = round(time_graph(torch, lambda: mhc.site_pre(
                    t["x"], t["fn_w"], t["scale"], t["base"], 20, 1e-6, out=out,
                    exact=exact)), 2)
            print(json.dumps({"sweep": "pre", "T": T, "streams": S, "hidden": H, **res}),
                  flush=True)
            del t, out
            torch.cuda.empty_cache()


def cpu_baseline(c, d, cpu_seconds=15.0, max_wall=30.0):
    """The fp64 oracle (pre + post) on the host cores over a bounded sample of the
    prefill workload: whole passes over its tokens (or a prefix, if one pass would
    exceed the bound), repeated until about `cpu_seconds` of CPU work is done."""
    import numpy as np

    import oracle
    threads = oracle.default_threads()
    eps = float(np.float32(c.eps))

    def one(n):
        o = oracle.site_pre(d["x"][:n], d["fn_w"], d["scale"], d["base"], c.iters, eps,
                            nthreads=threads)
        oracle.site_post(d["x"][:n], d["f"][:n], o["post"].astype(np.float32),
                         o["comb"].astype(np.float32), nthreads=threads)

    probe = min(c.T, 64)
    t0 = time.perf_counter()
    one(probe)
    per_tok = (time.perf_counter() - t0) / probe
    n = int(min(c.T, max(probe, (cpu_seconds / threads) / max(per_tok, 1e-9))))
    passes, tokens, t0 = 0, 0, time.perf_counter()
    while True:
        one(n)
        passes += 1
        tokens += n
        dt = time.perf_counter() - t0
        if dt * threads >= cpu_seconds or dt >= max_wall:
            break
    return {"value": round(tokens / dt, 2), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{passes} pass(es) over the first {n} of {c.T} tokens of the prefill "
                      f"workload, pre + post, {dt:.2f} s wall on {threads} threads"}


def oracle_per_config(cpu_seconds_cap=8.0):
    """The fp64 oracle (pre + post) on every workload config, at all host cores
    and at one thread, median of 3 runs each.  A config whose full run would
    take more than `cpu_seconds_cap` seconds of one core is timed on a prefix of
    its tokens (the oracle is per token, so its rate does not depend on T), and
    the token count is reported."""
    import statistics

    import numpy as np

    import oracle
    from mhc_inputs import CONFIGS, make_site
    cores = oracle.default_threads()
    rows = {}
    for name in ("tiny", "decode", "verify4", "verify8", "prefill", "wide"):
        c = CONFIGS[name]
        d = make_site(c)
        eps = float(np.float32(c.eps))

        def run(n, threads):
            t0 = time.perf_counter()
            o = oracle.site_pre(d["x"][:n], d["fn_w"], d["scale"], d["base"], c.iters, eps,
                                nthreads=threads)
            oracle.site_post(d["x"][:n], d["f"][:n], o["post"].astype(np.float32),
                             o["comb"].astype(np.float32), nthreads=threads)
            return time.perf_counter() - t0

        probe_n = min(c.T, 16)
        per_tok_1 = run(probe_n, 1) / probe_n
        n1 = int(min(c.T, max(1, cpu_seconds_cap / max(per_tok_1, 1e-9))))
        one = statistics.median(run(n1, 1) for _ in range(3))
        alln = statistics.median(run(c.T, cores) for _ in range(3))
        rows[name] = {"T": c.T, "streams": c.S, "hidden": c.H,
                      "all_cores_ms": round(alln * 1e3, 3),
                      "all_cores_tokens_per_s": round(c.T / alln, 1),
                      "one_thread_tokens": n1,
                      "one_thread_ms": round(one * 1e3, 3),
                      "one_thread_tokens_per_s": round(n1 / one, 1)}
    return {"cores": cores, "configs": rows,
            "note": "fp64 oracle, pre + post (post fed the oracle's own gates rounded to "
                    "fp32), wall clock, median of 3; all_cores: every token of the config "
                    "on all host threads; one_thread: one thread on the first "
                    "one_thread_tokens tokens"}


def load_traffic(kernel):
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        rec = json.load(open(TRAFFIC_FILE)).get(kernel)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash(KERNEL_SOURCES[kernel]):
        return None  # kernel changed since the counters were taken
    return rec.get("bytes_per_launch")


# prefill kernels whose counters make up each measured unit
TRAFFIC_UNITS = {
    "pre_kernel": ["fused_pf_kernel<4, 8>"],
    "pre_call": ["pack_weight_kernel<4, 24, 8>", "fused_pf_kernel<4, 8>"],
    "post_kernel": ["post_kernel<4>"],
    "walk_call": ["pack_weight_kernel<4, 24, 8>", "fused_pre_kernel<4, 8, 1, false, true, false>"],
    "wide_pre_call": ["partials_kernel<5, 4, true>", "finish_kernel<8>"],
    "wide_post_kernel": ["post_kernel<8>"],
}


def write_traffic(fetch_db, write_db):
    """Turn two rocprofv3 counter runs of `--kernels-only` (FETCH_SIZE, then
    WRITE_SIZE; KiB per dispatch) into bytes per prefill launch, scaled by what
    the same counters read for the plain 256 MiB device copy of that run."""
    import sqlite3
    import statistics
    from collections import defaultdict

    def per_kernel(db, counter):
        rows = sqlite3.connect(db).execute(
            "select kernel_name, grid_size, counter_name, value from counters_collection"
        ).fetchall()
        groups = defaultdict(list)
        for name, grid, cname, value in rows:
            if cname == counter:
                # the kernel's name with its template arguments, without the
                # return type, namespace and parameter list
                head = name.split("(")[0].strip()
                if head.startswith("void "):
                    head = head[5:]
                base, sep, targs = head.partition("<")
                short = base.split("::")[-1].strip() + sep + targs
                groups[(short, int(grid))].append(float(value))
        return {k: statistics.mean(v) for k, v in groups.items()}

    fetch, write = per_kernel(fetch_db, "FETCH_SIZE"), per_kernel(write_db, "WRITE_SIZE")
    copy_kib = 256 * 1024.0
    copies = [k for k in write if "copy" in k[0].lower() and abs(write[k] - copy_kib) < 1024]
    if not copies or copies[0] not in fetch:
        raise SystemExit("no 256 MiB copy kernel found in the counter runs")
    ck = copies[0]
    f_scale, w_scale = copy_kib / fetch[ck], copy_kib / write[ck]

    def largest(name):  # the prefill launch of a kernel has its largest grid
        keys = [k for k in fetch if k[0] == name and k in write]
        if not keys:
            raise SystemExit(f"kernel {name} missing from the counter runs")
        return max(keys, key=lambda k: k[1])

    out = {"fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "copy_kernel": ck[0], "copy_fetch_kib": fetch[ck], "copy_write_kib": write[ck]}
    for unit, names in TRAFFIC_UNITS.items():
        parts = {}
        total = 0.0
        for nm in names:
            k = largest(nm)
            b = (f_scale * fetch[k] + w_scale * write[k]) * 1024.0
            parts[nm] = {"grid_threads": k[1], "fetch_kib": fetch[k], "write_kib": write[k],
                         "scaled_bytes": round(b)}
            total += b
        out[unit] = {"bytes_per_launch": round(total), "kernels": parts,
                     "source_hash": kernel_source_hash(KERNEL_SOURCES[unit])}
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-sites", type=int, default=2000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernels-only", type=int, default=0)
    ap.add_argument("--workloads", default="prefill,decode",
                    help="configs (mhc_inputs.CONFIGS names) run by --kernels-only")
    ap.add_argument("--sweep", action="store_true",
                    help="print device time of the pre call (plain and decode-exact) over T")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="write the measured traffic file from two rocprofv3 counter runs")
    args = ap.parse_args()
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the mHC site program is token-parallel with "
              "no cross-GPU exchange, and this benchmark runs and reports a single GPU "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mhc_hyper_connection_token_amd as mhc
    from mhc_inputs import CONFIGS, make_site

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mhc.load_library()
    if args.sweep:
        run_sweep(mhc, torch)
        return
    if args.kernels_only:
        run_kernels_only(args.kernels_only, mhc, torch, CONFIGS, make_site,
                         tuple(w for w in args.workloads.split(",") if w))
        return

    # ---- prefill chunk: the timed workload
    c = CONFIGS["prefill"]
    d = make_site(c)
    t = to_dev(d, torch)
    out_pre, out_x = alloc_out(c.T, c.S, c.H, torch)
    ms, pre_ms, post_ms, wall, eager_ms = time_site(mhc, torch, t, c, out_pre, out_x,
                                                    args.steps, args.warmup)
    packed_ms = time_site_packed(mhc, torch, t, c, out_pre, out_x, args.steps)
    pre_b, post_b = algorithmic_bytes(c.T, c.S, c.H)
    site_gbps = (pre_b + post_b) / (ms * 1e-3) / 1e9
    # The dominant kernel: the token-tiled pre kernel (mhc_site_pre_packed with
    # the weight packed beforehand launches only it, timed after the pack as in
    # a site step) against the post kernel, from HIP graphs of K launches, HIP
    # events on the stream the kernels run on.  The pre kernel moves the pre
    # call's algorithmic bytes (x, the weight once, y and the gates).
    kern = time_kernels_alone(mhc, torch, t, c, out_pre, out_x, calls=max(10, args.steps // 2))
    if kern["post_kernel_us"] >= kern["pre_kernel_us"]:
        dom, dom_us, dom_b, bound_name = ("post_kernel", kern["post_kernel_us"], post_b,
                                          "post_kernel<4> (mhc_site_post)")
    else:
        dom, dom_us, dom_b, bound_name = (
            "pre_kernel", kern["pre_kernel_us"], pre_b,
            "fused_pf_kernel<4,8> (mhc_site_pre's token-tiled pre chain on persistent tiles, "
            "half of each next slab requested into LDS; the weight pack is a kernel of its own)")
    achieved = dom_b / (dom_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": bound_name, "achieved": round(achieved, 1),
                "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                "traffic": load_traffic(dom), "algorithmic_bytes_per_launch": dom_b,
                "avg_launch_us": round(dom_us, 2),
                "other_kernel_us": round(kern["post_kernel_us"] if dom == "pre_kernel"
                                         else kern["pre_kernel_us"], 2),
                "pre_call_eager_us": round(pre_ms * 1e3, 2),
                "pre_kernel_back_to_back_us": round(kern["pre_kernel_back_to_back_us"], 2),
                "pack_kernel_us": round(kern["pack_kernel_us"], 2),
                "note": "avg_launch_us: the pre kernel as a site step runs it, right after the "
                        "weight pack: a HIP graph of K (pack, pre kernel) pairs less a graph of K "
                        "packs, HIP events on their stream (pre_kernel_back_to_back_us: K pre "
                        "launches with nothing between them); achieved = algorithmic bytes per "
                        "launch / avg_launch_us; traffic = 2.0 x FETCH_SIZE + WRITE_SIZE of one launch "
                        "(rocprofv3 counters scaled by a plain copy), null if the kernel's "
                        "sources changed since; pre_call_eager_us: pack + pre kernel as one "
                        "eager call"}

    # ---- decode site (T=1): microseconds per site, back to back
    cd = CONFIGS["decode"]
    td = to_dev(make_site(cd), torch)
    dpre, dx = alloc_out(cd.T, cd.S, cd.H, torch)
    n = args.decode_sites
    d_eager_us, d_graph_us = time_decode(mhc, torch, td, cd, dpre, dx, n)
    d_ws_us = time_ws_decode(mhc, torch, td, cd)
    d_walk_us = time_decode_walk(mhc, torch, cd, td["x"])
    d_walk_zq_us = time_decode_walk(mhc, torch, cd, td["x"], zq8=True)
    pre1, post1 = algorithmic_bytes(cd.T, cd.S, cd.H)

    # ---- decode: the Sinkhorn's share (iters sweep, least-squares line over
    # µs per site) and a cold variant (weights rotating through more than the
    # 256 MB memory-side cache)
    sweep_iters = (1, 5, 10, 20, 40)
    it_us = []
    for it in sweep_iters:
        cit = dataclasses.replace(cd, iters=it)
        it_us.append(time_decode(mhc, torch, td, cit, dpre, dx, 500)[1])
    slope, intercept = fit_line(sweep_iters, it_us)
    iters_sweep = {"iters": list(sweep_iters), "us_per_site": [round(v, 3) for v in it_us],
                   "slope_us_per_iter": round(slope, 4),
                   "intercept_us": round(intercept, 3),
                   "note": "decode site (T=1) from a HIP graph of 50 sites at each Sinkhorn "
                           "iteration count; slope = the Sinkhorn's cost per iteration, "
                           "intercept = everything else"}
    cold = time_cold_decode(mhc, torch, cd, sets=200)
    cold["walk_cold_us_per_site"] = round(
        time_decode_walk(mhc, torch, cd, td["x"], L=200, distinct=200), 3)
    cold["note"] += ("; walk_cold: 200 sites chained with mhc_site_post_pre, each with its "
                     "own weight, one graph")

    # ---- pure-stream bandwidth of this part (mhc_bandwidth_probe over 1 GiB)
    probe = run_bandwidth_probe(mhc, torch)

    # ---- small sites (the tiny config, the decode site, the verify batches):
    # pre, post and the whole site, each from a HIP graph of 50 calls (device
    # time plus the gaps between kernels)
    verify = {}
    for vname in ("tiny", "decode", "verify4", "verify8"):
        cv = CONFIGS[vname]
        tv = to_dev(make_site(cv), torch)
        vpre, vx = alloc_out(cv.T, cv.S, cv.H, torch)
        v_pre_us = time_graph(torch, lambda: mhc.site_pre(
            tv["x"], tv["fn_w"], tv["scale"], tv["base"], cv.iters, cv.eps, out=vpre),
            calls=50, reps=10)
        v_post_us = time_graph(torch, lambda: mhc.site_post(
            tv["x"], tv["f"], vpre[1], vpre[2], out=vx), calls=50, reps=10)
        _, v_site_us = time_decode(mhc, torch, tv, cv, vpre, vx, 500)
        verify[f"{vname}_T{cv.T}_H{cv.H}"] = {"pre_us": round(v_pre_us, 3),
                              "post_us": round(v_post_us, 3),
                              "site_us": round(v_site_us, 3),
                              "tokens_per_s": round(cv.T / (v_site_us * 1e-6), 1)}
    # ---- wide site (T = 1024, S = 8, H = 7168): the split path, bound by the
    # fp32 MFMA rate of its partials (33 flop per byte)
    cw = CONFIGS["wide"]
    tw = to_dev(make_site(cw), torch)
    wpre, wx = alloc_out(cw.T, cw.S, cw.H, torch)
    w_pre_us = time_graph(torch, lambda: mhc.site_pre(
        tw["x"], tw["fn_w"], tw["scale"], tw["base"], cw.iters, cw.eps, out=wpre), calls=10, reps=5)
    w_post_us = time_graph(torch, lambda: mhc.site_post(
        tw["x"], tw["f"], wpre[1], wpre[2], out=wx), calls=10, reps=5)

    def wide_site():
        mhc.site_pre(tw["x"], tw["fn_w"], tw["scale"], tw["base"], cw.iters, cw.eps, out=wpre)
        mhc.site_post(tw["x"], tw["f"], wpre[1], wpre[2], out=wx)
    w_site_us = time_graph(torch, wide_site, calls=10, reps=5)
    wpre_b, wpost_b = algorithmic_bytes(cw.T, cw.S, cw.H)
    w_rows = (2 + cw.S) * cw.S
    w_flop = 2.0 * cw.T * w_rows * cw.S * cw.H  # the mixes contraction
    wide = {"T": cw.T, "streams": cw.S, "hidden": cw.H,
            "pre_us": round(w_pre_us, 2), "post_us": round(w_post_us, 2),
            "site_us": round(w_site_us, 2),
            "tokens_per_s": round(cw.T / (w_site_us * 1e-6), 1),
            "algorithmic_GBps": round((wpre_b + wpost_b) / (w_site_us * 1e-6) / 1e9, 1),
            "pre_mixes_TFLOPs": round(w_flop / (w_pre_us * 1e-6) / 1e12, 2),
            "note": "generalised width; pre, post and site each as 10 calls in a HIP graph "
                    "replayed; pre_mixes_TFLOPs is the fp32 mixes contraction (2*T*R*S*H flop) "
                    "over the whole pre call (partials + finish), against 157.3 TFLOP/s"}
    del tw, wpre, wx
    torch.cuda.empty_cache()

    verify["note"] = ("small sites (S=4, 20 iterations): pre alone, post alone and the whole "
                      "site, each as 50 calls in a HIP graph replayed, HIP-event time per call")

    # ---- branch-input epilogue (RMS norm of y with a weight, q8 codes): the pre
    # call with it, against the same call without it
    from mhc_inputs import make_norm_weight
    norm_eps = 1e-5
    nw_p = torch.from_numpy(make_norm_weight(c.H, 1)).cuda()
    o7 = alloc_zq8(c.T, c.S, c.H, torch)
    zq_pre_us = time_pre_zq8(mhc, torch, t, c, nw_p, norm_eps, o7, args.steps, args.warmup)
    nw_d = torch.from_numpy(make_norm_weight(cd.H, 1)).cuda()
    o7d = alloc_zq8(cd.T, cd.S, cd.H, torch)
    zq_d_eager_us, zq_d_graph_us = time_decode(mhc, torch, td, cd, dpre, dx, n,
                                               zq8=(nw_d, norm_eps, o7d))
    epi_b = zq8_bytes(c.T, c.H)
    epi_us = zq_pre_us - pre_ms * 1e3

    # ---- a walk over 8 sites: separate calls against the fused post-then-pre schedule
    walk_sep_us, walk_fused_us, walk_sep_g_us, walk_fused_g_us, walk_packed_g_us = time_walk(
        mhc, torch, c, t["x"], 8, max(3, args.steps // 5), 2)
    walk_traffic = load_traffic("walk_call")
    walk = {"sites": 8,
            "separate_us_per_site": round(walk_sep_us, 2),
            "fused_us_per_site": round(walk_fused_us, 2),
            "separate_graph_us_per_site": round(walk_sep_g_us, 2),
            "fused_graph_us_per_site": round(walk_fused_g_us, 2),
            "fused_packed_weight_graph_us_per_site": (round(walk_packed_g_us, 2)
                                                      if walk_packed_g_us else None),
            "fused_packed_weight_tokens_per_s": (round(c.T / (walk_packed_g_us * 1e-6), 1)
                                                 if walk_packed_g_us else None),
            "fused_tokens_per_s": round(c.T / (walk_fused_g_us * 1e-6), 1),
            "fused_equivalent_GBps": round((pre_b + post_b) / (walk_fused_g_us * 1e-6) / 1e9, 1),
            "fused_call_traffic": walk_traffic,
            "fused_traffic_GBps": (round(walk_traffic / (walk_fused_g_us * 1e-6) / 1e9, 1)
                                   if walk_traffic else None),
            "note": "prefill chunk, 8 sites with their own weights; fused: each site's post "
                    "and the next site's pre in one kernel (mhc_site_post_pre), bit-identical "
                    "to the separate calls.  *_us_per_site: eager walks with HIP events; "
                    "*_graph_us_per_site: 4 walks captured in one HIP graph, replayed; the "
                    "rates use the graph figure; fused_packed_weight: every site weight packed "
                    "once beforehand (mhc_pack_weight), the walk reading the packed copies.  equivalent_GBps counts one pre + post's "
                    "algorithmic bytes (the fused call does not re-read the new state); "
                    "traffic_GBps is the measured HBM bytes of the fused call (pack + kernel) "
                    "per site time"}

    # ---- trunk entry and exit at the prefill size
    emb = torch.empty((c.T, c.H), device="cuda", dtype=torch.float32).uniform_(-1, 1)
    xs = torch.empty((c.T, c.S, c.H), device="cuda", dtype=torch.float32)
    ym = torch.empty((c.T, c.H), device="cuda", dtype=torch.float32)
    hw = t["fn_w"][:c.S].contiguous()
    hs, hb = t["scale"][:1].contiguous(), t["base"][:c.S].contiguous()
    hg = torch.empty((c.T, c.S), device="cuda", dtype=torch.float32)
    exp_us = time_calls(torch, lambda: mhc.expand(emb, c.S, out=xs), args.steps, args.warmup)
    mean_us = time_calls(torch, lambda: mhc.mean(t["x"], out=ym), args.steps, args.warmup)
    head_us = time_calls(torch, lambda: mhc.head(t["x"], hw, hs, hb, c.eps, out=(hg, ym)),
                         args.steps, args.warmup)
    stream_b = 4 * c.T * c.H * (c.S + 1)  # expand and mean: T*H in, T*S*H out (or back)
    head_b = 4 * (c.T * c.S * c.H + c.S * c.S * c.H + 1 + c.S + c.T * c.S + c.T * c.H)
    trunk = {"expand_us": round(exp_us, 2), "mean_us": round(mean_us, 2),
             "head_us": round(head_us, 2),
             "expand_GBps": round(stream_b / (exp_us * 1e-6) / 1e9, 1),
             "mean_GBps": round(stream_b / (mean_us * 1e-6) / 1e9, 1),
             "head_algorithmic_GBps": round(head_b / (head_us * 1e-6) / 1e9, 1),
             "note": "trunk entry (expand), unweighted exit (mean) and gated-head exit at "
                     "T=4096 S=4 H=4096; HIP events per call; bytes count each operand once "
                     "(from 256 tokens the head runs on the fused token tiles and reads x once)"}
    del emb, xs, hg

    # ---- decode-exact batching: a 64-token verify batch and the prefill chunk
    from mhc_inputs import make_random_shape
    d64 = to_dev(make_random_shape(64, c.S, c.H, seed=64), torch)
    p64, _ = alloc_out(64, c.S, c.H, torch)
    ex = {"T64_exact_us": time_pre_variant(mhc, torch, d64, c, p64, True, args.steps, args.warmup),
          "T64_plain_us": time_pre_variant(mhc, torch, d64, c, p64, False, args.steps,
                                           args.warmup),
          "T4096_exact_us": time_pre_variant(mhc, torch, t, c, out_pre, True, args.steps,
                                             args.warmup),
          "T4096_plain_us": round(pre_ms * 1e3, 2)}
    ex = {k: round(v, 2) for k, v in ex.items()}
    del d64, p64

    # ---- CPU oracle baseline (host cores, bounded sample), and the oracle on
    # every config at all cores and at one thread
    cpu = None if args.no_cpu_baseline else cpu_baseline(c, d)
    if cpu is not None:
        cpu["per_config"] = oracle_per_config()

    line = {
        "metric": METRIC,
        "value": round(c.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "prefill chunk: T=4096 tokens, streams=4, hidden=4096, "
                               "20 Sinkhorn iterations, eps=1e-6 (pre + post per step)",
                   "T": c.T, "streams": c.S, "hidden": c.H, "iters": c.iters,
                   "parallelism": "single GPU"},
        "site_hbm": {"algorithmic_GBps": round(site_gbps, 1),
                     "frac_of_peak": round(site_gbps / PEAK_HBM_GBPS, 4),
                     "pre_us": round(pre_ms * 1e3, 2), "post_us": round(post_ms * 1e3, 2),
                     "eager_ms_per_step": round(eager_ms, 4),
                     "packed_weight_ms_per_step": (round(packed_ms, 4) if packed_ms else None),
                     "packed_weight_tokens_per_s": (round(c.T / (packed_ms * 1e-3), 1)
                                                    if packed_ms else None),
                     "packed_weight_GBps": (round((pre_b + post_b) / (packed_ms * 1e-3) / 1e9,
                                                  1) if packed_ms else None),
                     "algorithmic_bytes_per_step": pre_b + post_b,
                     "note": "ms_per_step: the `steps` sites (pre + post each) captured in one "
                             "HIP graph and replayed once after one untimed replay, HIP events "
                             "around the replay; eager_ms_per_step: the same steps as plain "
                             "calls with an event between the calls, whose per-call times give "
                             "pre_us and post_us; packed_weight_*: the same timed steps with "
                             "the site weight packed once beforehand (mhc_pack_weight) and read "
                             "by mhc_site_pre_packed, as a trunk with fixed weights runs them"},
        "small_sites": verify,
        "decode_iters_sweep": iters_sweep,
        "decode_cold": cold,
        "bandwidth_probe": probe,
        "wide_site": wide,
        "decode_t1": {"us_per_site": round(d_graph_us, 3), "eager_us_per_site": round(d_eager_us, 3),
                      "workspace_graph_us_per_site": round(d_ws_us, 3),
                      "walk_graph_us_per_site": round(d_walk_us, 3),
                      "walk_zq8_graph_us_per_site": round(d_walk_zq_us, 3),
                      "sites": n,
                      "note": "us_per_site: a HIP graph of 50 sites (pre + post) replayed on one "
                              "stream, HIP-event time / sites (device time plus the gaps between "
                              "kernels); eager: the same sites as plain calls, host launch "
                              "included; workspace: 50 sites through a persistent workspace "
                              "(ping-pong state), one graph; walk: 50 sites with four "
                              "rotating weights chained with mhc_site_post_pre (at T=1 its "
                              "post and pre run as separate kernels), one graph, without and "
                              "with the epilogue",
                      "algorithmic_bytes_per_site": pre1 + post1},
        "epilogue_zq8": {
            "prefill_pre_zq8_us": round(zq_pre_us, 2),
            "prefill_added_us": round(epi_us, 2),
            "prefill_algorithmic_bytes_alone": epi_b,
            "decode_t1_us_per_site": round(zq_d_graph_us, 3),
            "decode_t1_eager_us_per_site": round(zq_d_eager_us, 3),
            "note": "the pre call with the epilogue (z = RMS-norm(y) * nw, q8 codes and "
                    "scales); added_us = its time minus pre_us; decode sites as in decode_t1 "
                    "with the epilogue in the pre call"},
        "site_walk": walk,
        "trunk_ends": trunk,
        "pre_exact": dict(ex, note="mhc_site_pre_exact (every row bit-identical to a solo "
                                     "T=1 call) against mhc_site_pre, same inputs, S=4 H=4096"),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
