"""Host-side logic of bench.py: the one-GPU guard, the algorithmic byte counts
the roofline divides by, and the scaling of rocprofv3 byte counters into
traffic per launch (on synthetic counter databases)."""
import json
import os
import sqlite3
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_of_the_workloads():
    # the prefill chunk: 941.8 MB per pre + post step; the decode site: 1.80 MB
    pre, post = bench.algorithmic_bytes(4096, 4, 4096)
    assert pre + post == 941_817_964
    assert pre == 4 * (4096 * (16384 + 4096 + 8 + 16) + 24 * 16384 + 3 + 24)
    pre1, post1 = bench.algorithmic_bytes(1, 4, 4096)
    assert pre1 + post1 == 1_802_524
    # the wide site: 282.9 MB pre, 499.4 MB post
    pw, qw = bench.algorithmic_bytes(1024, 8, 7168)
    assert round(pw / 1e6, 1) == 282.9 and round(qw / 1e6, 1) == 499.4


def _counter_db(path, counter, rows):
    c = sqlite3.connect(path)
    c.execute("create table counters_collection (kernel_name text, grid_size int, "
              "counter_name text, value real)")
    for name, grid, value in rows:
        c.execute("insert into counters_collection values (?, ?, ?, ?)",
                  (name, grid, counter, value))
    c.commit()
    c.close()


def test_write_traffic_scales_by_the_copy_kernel(tmp_path, monkeypatch):
    fetch, write = str(tmp_path / "f.db"), str(tmp_path / "w.db")
    copy = "__amd_rocclr_copyBuffer(void*)"
    _counter_db(fetch, "FETCH_SIZE", [
        (copy, 1 << 20, 131072.0),  # half of 256 MiB: the factor becomes 2
        ("void mhc::pack_weight_kernel<4, 24, 8>(float const*)", 98304, 800.0),
        ("void mhc::fused_pf_kernel<4, 8>(...)", 131072, 100000.0),
        ("void mhc::fused_pf_kernel<4, 8>(...)", 512, 5.0),  # decode-size
        ("void mhc::post_kernel<4>(...)", 4194304, 160000.0),
        ("void mhc::fused_pre_kernel<4, 8, 1, false, true, false>(...)", 524288, 150000.0),
        ("void mhc::partials_kernel<5, 4, true>(...)", 131072, 210000.0),
        ("void mhc::finish_kernel<8>(...)", 262144, 120000.0),
        ("void mhc::post_kernel<8>(...)", 1835008, 130000.0)])
    _counter_db(write, "WRITE_SIZE", [
        (copy, 1 << 20, 262144.0),
        ("void mhc::pack_weight_kernel<4, 24, 8>(float const*)", 98304, 1536.0),
        ("void mhc::fused_pf_kernel<4, 8>(...)", 131072, 60000.0),
        ("void mhc::fused_pf_kernel<4, 8>(...)", 512, 1.0),
        ("void mhc::post_kernel<4>(...)", 4194304, 262144.0),
        ("void mhc::fused_pre_kernel<4, 8, 1, false, true, false>(...)", 524288, 330000.0),
        ("void mhc::partials_kernel<5, 4, true>(...)", 131072, 12000.0),
        ("void mhc::finish_kernel<8>(...)", 262144, 29000.0),
        ("void mhc::post_kernel<8>(...)", 1835008, 229376.0)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    bench.write_traffic(fetch, write)
    rec = json.load(open(out))
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    # the largest grid of each kernel is the prefill launch
    assert rec["pre_call"]["bytes_per_launch"] == round((2 * 800 + 1536 + 2 * 100000 + 60000) * 1024)
    assert rec["post_kernel"]["bytes_per_launch"] == round((2 * 160000 + 262144) * 1024)
    # the walk kernel is told apart from the plain one by its template arguments
    assert rec["walk_call"]["bytes_per_launch"] == round((2 * 800 + 1536 + 2 * 150000 + 330000)
                                                         * 1024)
    # the fused kernel alone, and the wide site's calls (S = 8 has kernels of its own)
    assert rec["pre_kernel"]["bytes_per_launch"] == round((2 * 100000 + 60000) * 1024)
    assert rec["wide_pre_call"]["bytes_per_launch"] == round((2 * 210000 + 12000 + 2 * 120000
                                                              + 29000) * 1024)
    assert rec["wide_post_kernel"]["bytes_per_launch"] == round((2 * 130000 + 229376) * 1024)
    # the stored hash is that of the measured kernels' sources
    assert rec["pre_call"]["source_hash"] == bench.kernel_source_hash(bench.KERNEL_SOURCES["pre_call"])


def test_traffic_is_dropped_when_the_kernel_sources_change(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    json.dump({"pre_call": {"bytes_per_launch": 123, "source_hash": "not-the-current-one"}},
              open(out, "w"))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    assert bench.load_traffic("pre_call") is None
    json.dump({"pre_call": {"bytes_per_launch": 123, "source_hash":
                            bench.kernel_source_hash(bench.KERNEL_SOURCES["pre_call"])}},
              open(out, "w"))
    assert bench.load_traffic("pre_call") == 123


def test_fit_line_matches_least_squares():
    import numpy as np
    xs = [1, 5, 10, 20, 40]
    ys = [8.58, 8.71, 8.66, 9.32, 10.48]
    slope, intercept = bench.fit_line(xs, ys)
    want = np.polyfit(np.array(xs, float), np.array(ys, float), 1)
    assert abs(slope - want[0]) < 1e-12 and abs(intercept - want[1]) < 1e-12
    # an exact line is recovered exactly
    assert bench.fit_line([0, 1, 2], [3.0, 5.0, 7.0]) == (2.0, 3.0)
    with pytest.raises(ValueError):
        bench.fit_line([1], [2.0])
    with pytest.raises(ValueError):
        bench.fit_line([2, 2], [1.0, 3.0])


def test_traffic_units_name_kernels_that_exist():
    """Every kernel named in the traffic table is a __global__ template in the
    library sources with that many template arguments, so a renamed or
    re-templated kernel fails here rather than as a missing counter row on the
    GPU machine."""
    import glob
    import re
    src = "".join(open(p).read() for p in
                  glob.glob(os.path.join(ROOT, "mhc_hyper_connection_token_amd", "csrc", "*.hip")))
    kernels = {}
    for m in re.finditer(r"template\s*<([^>]*)>\s*__global__[^;{]*?\bvoid\s+(\w+)\s*\(", src):
        kernels[m.group(2)] = len([a for a in m.group(1).split(",") if a.strip()])
    for unit, names in bench.TRAFFIC_UNITS.items():
        for nm in names:
            base, _, args = nm.partition("<")
            assert base in kernels, f"{unit}: no kernel named {base}"
            nargs = len([a for a in args.rstrip(">").split(",") if a.strip()])
            assert nargs == kernels[base], f"{unit}: {nm} has {nargs} template arguments"
