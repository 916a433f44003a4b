"""bench.py's contract, checked without a GPU: the workloads it times cover
the benchmark configurations (Q2_0 M=1 and N=K=5120 batched rows, W8A16
M in {1, 8, 16}, the FFN shapes at M in {1, 8, 16, 32}), weight rings larger
than the 256 MB on-die cache, exactly K timed steps that each read a cold
copy whatever K is, and one GPU only."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_headline_and_sweep_cover_the_configurations():
    b = _bench()
    name, cls, _, N, K, M = b.HEADLINE
    assert (cls.fmt, N, K, M) == ("q2_0", 5120, 5120, 1)
    shapes = {(e[1].fmt, e[3], e[4], e[5]) for e in b.sweep_list()}
    assert ("q2_0", 256, 1024, 1) in shapes
    for m in (2, 4, 5, 8, 16):
        assert ("q2_0", 5120, 5120, m) in shapes
    for m in (1, 8, 16):
        assert ("w8a16", 5120, 5120, m) in shapes
    for n, k in ((17408, 5120), (5120, 17408)):
        for m in (1, 8, 16, 32):
            assert ("q2_0", n, k, m) in shapes and ("w8a16", n, k, m) in shapes
    assert len({e[0] for e in b.sweep_list()}) == len(b.sweep_list())  # names are unique (--only)


def test_weight_rings_exceed_the_on_die_cache():
    b = _bench()
    for nbytes in (b.q2_0_bytes(5120, 5120), b.q2_0_bytes(17408, 5120), b.fp8_bytes(5120, 5120),
                   b.fp8_bytes(5120, 17408)):
        r = b.ring_size(nbytes)
        assert r >= 8 and r * nbytes > 256 * 1024 * 1024
    assert b.q2_0_bytes(5120, 5120) == 6963200
    assert b.fp8_bytes(5120, 5120) == 26220800


def test_timed_plan_times_exactly_the_requested_steps():
    b = _bench()
    for R in (8, 21, 23, 78):
        L = b.graph_len(R)
        assert L % R == 0 and L >= b.MIN_GRAPH_STEPS and L - R < b.MIN_GRAPH_STEPS
        for steps in (1, 5, 20, 200, 997, 1000, 2000):
            full, rest = b.timed_plan(R, steps)
            assert full * L + rest == steps and 0 <= rest < L


def test_every_timed_read_is_cold_at_the_drivers_step_count():
    """At --steps 20 --warmup 5 (and at the defaults), every timed read of a
    weight copy follows more than 256 MiB of reads of other copies since that
    copy's previous read, for every workload whose configuration asks for
    cold-cycled weights (all but the 70 KB N=256, K=1024 latency case)."""
    b = _bench()
    for steps in (20, 2000, 997, 1):
        for entry in [b.HEADLINE] + b.sweep_list():
            name, cls, wid, N, K, M = entry
            wl = cls(name, wid, N, K, M)
            R = b.ring_size(wl.bytes)
            t = b.timed_traffic(R, wl.bytes, steps)
            assert t["distinct_copies"] == min(steps, R)
            if (N, K) == (256, 1024):
                continue
            assert t["reuse_distance_bytes"] > 256 * 1024 * 1024, (name, steps, t)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
