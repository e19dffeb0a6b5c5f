"""CPU tests of the benchmark's statistics and record handling (no GPU):
the distribution-free median confidence interval, the raw-sample
re-aggregation and the kernel-trace summary."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest
from scipy.stats import binom

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _coverage(n, j):
    """P[x_(j) <= median <= x_(n+1-j)] for a continuous distribution:
    1 - 2 P[Bin(n, 1/2) <= j - 1]."""
    return 1.0 - 2.0 * binom.cdf(j - 1, n, 0.5)


@pytest.mark.parametrize("n", [6, 9, 10, 25, 50, 101, 1000, 5000])
def test_median_ci_is_the_narrowest_95_percent_order_statistic_pair(n):
    rng = np.random.default_rng(n)
    xs = rng.standard_normal(n)
    med, (lo, hi), cover = bench.median_ci95(xs)
    v = np.sort(xs)
    assert med == pytest.approx(np.median(xs), abs=0)
    j = int(np.searchsorted(v, lo)) + 1          # lo = x_(j)
    assert v[j - 1] == lo and v[n - j] == hi
    assert cover == pytest.approx(_coverage(n, j), rel=1e-9, abs=1e-12)
    assert cover >= 0.95
    if j < n // 2:
        assert _coverage(n, j + 1) < 0.95        # one step narrower falls short


def test_median_ci_nine_samples():
    med, (lo, hi), cover = bench.median_ci95([9, 1, 8, 2, 7, 3, 6, 4, 5])
    assert med == 5 and (lo, hi) == (2, 8)
    assert cover == pytest.approx(1 - 2 * 10 / 512)


def test_median_ci_covers_in_simulation():
    # the interval contains the true median in about its stated share of
    # repetitions (exponential samples: a skewed distribution)
    rng = np.random.default_rng(1)
    hits, reps = 0, 4000
    for _ in range(reps):
        xs = rng.exponential(size=15)
        _, (lo, hi), cover = bench.median_ci95(xs)
        hits += lo <= np.log(2) <= hi
    assert abs(hits / reps - cover) < 0.02


def test_reaggregate_rebuilds_summaries(tmp_path):
    p = tmp_path / "s.jsonl"
    sink = bench.SampleSink(str(p))
    xs = [0.5, 0.4, 0.6, 0.45, 0.55, 0.52, 0.48, 0.41, 0.59]
    for i, x in enumerate(xs):
        sink.add("wl", "call", i, 20, x)
    sink.add("wl", "kernel", 0, 20, 0.3)
    sink.f.close()
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--reaggregate", str(p)],
                         capture_output=True, text=True, check=True).stdout
    rows = {json.loads(l)["leg"]: json.loads(l) for l in out.splitlines()}
    assert rows["call"]["median_ms_per_step"] == 0.5
    assert rows["call"]["ci95_ms_per_step"] == [0.41, 0.59]
    assert rows["kernel"]["n"] == 1


def test_summarize_trace(tmp_path):
    f = tmp_path / "k_kernel_trace.csv"
    f.write_text("Kernel_Name,Grid_Size_X,Grid_Size_Y,Grid_Size_Z,Start_Timestamp,End_Timestamp\n"
                 "gemm_a,512,1,1,1000,3000\n"
                 "gemm_a,512,1,1,5000,9000\n"
                 "quant,256,1,1,0,500\n")
    out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-trace",
                          str(tmp_path)], capture_output=True, text=True, check=True).stdout
    line = next(l for l in out.splitlines() if "gemm_a" in l)
    assert "| 2 | 3.00 | 3.00 |" in line
