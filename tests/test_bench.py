"""bench.py's host-side parts, no GPU needed: the one-GPU contract, the work
counts its rates divide by, and the lookup of stored HBM byte counters."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2, r.stderr
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line for a configuration that was not run


@pytest.mark.parametrize("shape,flops", [
    ((2, 16, 4096, 64, 128), 2.062e11),    # prefill_v1
    ((1, 32, 16384, 128, 128), 4.398e12),  # prefill_v2
    ((1, 8, 65536, 64, 128), 1.319e13),    # longctx_v1
])
def test_prefill_work_of_the_workloads(shape, flops):
    assert bench.prefill_flops(*shape) == pytest.approx(flops, rel=1e-3)


@pytest.mark.parametrize("N,window", [(100, 0), (100, 10), (100, 1), (64, 64), (64, 200), (257, 40)])
def test_visible_pair_count_against_brute_force(N, window):
    # the metric counts a causal head as N^2/2 pairs (N(N+1)/2 - N/2) and a
    # window W < N as W^2/2 + (N - W) W (the exact count less W/2)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    vis = j <= i
    if 0 < window < N:
        vis &= j > i - window
    exact = int(vis.sum())
    per_pair = 2.0 * (2 * 64 + 2 * 128)
    short = window / 2.0 if 0 < window < N else N / 2.0
    assert bench.prefill_flops(1, 1, N, 64, 128, window) / per_pair == pytest.approx(exact - short, abs=1e-9)
    assert bench.backward_flops(1, 1, N, 64, 128, window) / (12 * 64 + 4 * 128) == pytest.approx(exact - short,
                                                                                                abs=1e-9)


def test_decode_bytes_scale_with_the_cache_format():
    ctx = np.array([1, 63, 64, 65, 700], np.int32)
    small = dict(B=5, H=8, H_kv=2, ctx_len=ctx, max_pages=16)
    bf, f8 = W.decode_v2(**small), W.decode_v2_fp8(**small)
    v1 = W.decode_v1(**small)
    tokens = int(ctx.sum())
    # the keys and values of every visible token are read once; fp8 halves them
    rest_bf = bench.decode_bytes(bf) - tokens * 2 * (128 + 128) * 2
    rest_f8 = bench.decode_bytes(f8) - tokens * 2 * (128 + 128) * 1
    assert rest_bf == rest_f8 > 0
    # V1 reads two key caches of width 64 and one value cache of width 128
    rest_v1 = bench.decode_bytes(v1) - tokens * 2 * (64 + 64 + 128) * 2
    assert 0 < rest_v1 < 2 * rest_bf


def test_stored_counters_are_used_only_for_matching_sources(monkeypatch):
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        stored = json.load(f)
    names = [k for k in stored if not k.startswith("_")]
    assert {"prefill_v1", "decode_v2"} <= set(names)
    for name in names:
        e = stored[name]
        got = bench.load_traffic(name)
        if e["source_hash"] == bench.kernel_source_hash(name):
            assert got == e["bytes_per_launch"] > 0
        else:
            assert got is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda name: "0" * 16)
    assert all(bench.load_traffic(n) is None for n in names)
    assert bench.load_traffic("no_such_workload") is None
