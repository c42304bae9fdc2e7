"""Host-side logic of bench.py that needs no GPU: the one-GPU guard, the line
and percentile helpers, and the source hash that ties the recorded counter
bytes to the kernels they were measured on."""
import importlib.util
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_lines_bytes_counts_whole_128_byte_lines():
    b = _bench()
    assert b.lines_bytes([0]) == 0.0
    assert b.lines_bytes([1, 128, 129, 488, 896, 1254]) == 128 * (1 + 1 + 2 + 4 + 7 + 10)
    rng = np.random.default_rng(3)
    x = rng.integers(0, 20000, 1000)
    assert b.lines_bytes(x) == float(sum(-(-int(v) // 128) * 128 for v in x))


def test_percentiles_of_launch_times():
    b = _bench()
    ms = [0.2, 0.1, 0.4, 0.3, 0.5]
    p = b.percentiles_us(ms)
    assert p["min"] == 100.0 and p["max"] == 500.0 and p["median"] == 300.0
    assert p["mean"] == 300.0 and p["launches"] == 5


def test_source_hash_ignores_comments_and_spacing_only():
    b = _bench()
    a = "int f(int x) {\n  return x + 1;  // one more\n}\n"
    same = "/* a comment */ int f(int x) { return x + 1; }"
    other = "int f(int x) { return x + 2; }"
    h = lambda t: b.gather_sources_sha256(read=lambda rel: t, sources=("x",))
    assert h(a) == h(same)
    assert h(a) != h(other)


def test_recorded_counters_match_the_current_kernels():
    """The counter bytes in bench.py were taken with the kernels as they are:
    their source hashes must match, or bench.py would report null traffic."""
    b = _bench()
    assert b.gather_sources_sha256() == b.GATHER_SOURCES_SHA256
    assert b.gather_sources_sha256(sources=b.CACHE_SOURCES) == b.CACHE_SOURCES_SHA256
