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


def test_summarize_pmc_records_the_sustained_clock(tmp_path):
    # one dispatch of 1000 us whose GRBM_GUI_ACTIVE sums to 8 x 1.8e6 cycles
    # over the 8 XCDs: 1.8 GHz; MFMA busy 1024 SIMDs x 0.9e6 cycles: 50 %
    name = "void kq::gemm_w8a8_kernel<256, 256, 2, 4, 64, __hip_bfloat16, false>(...)"
    (tmp_path / "s_kernel_trace.csv").write_text(
        "Dispatch_Id,Kernel_Name,Start_Timestamp,End_Timestamp\n"
        f"7,\"{name}\",0,1000000\n")
    (tmp_path / "s_counter_collection.csv").write_text(
        "Dispatch_Id,Kernel_Name,Grid_Size,Counter_Name,Counter_Value\n"
        f"7,\"{name}\",1572864,GRBM_GUI_ACTIVE,{8 * 1.8e6}\n"
        f"7,\"{name}\",1572864,SQ_VALU_MFMA_BUSY_CYCLES,{1024 * 0.9e6}\n")
    out = tmp_path / "clock.json"
    subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--summarize-pmc", str(tmp_path),
                    "--workload", "wl", "--clock-out", str(out)], capture_output=True, text=True,
                   check=True)
    rec = json.load(open(out))["gemm_w8a8_256x256w8@wl"]
    assert rec["clock_ghz"] == pytest.approx(1.8)
    assert rec["mfma_busy_pct"] == pytest.approx(50.0)
    assert rec["cycles"] == pytest.approx(1.8e6)
    assert rec["source_hash"] == bench.kernel_source_hash("gemm_w8a8_256x256w8")


class _FakeGraph:
    def __init__(self, per_call_ms):
        self.per_call_ms = per_call_ms


def test_fast_shapes_get_more_calls_per_sample(monkeypatch):
    per_call = 0.01   # ms per call: 20 calls take 0.2 ms, below the 1 ms floor
    monkeypatch.setattr(bench, "graph_capture", lambda fn, steps: _FakeGraph(per_call))
    monkeypatch.setattr(bench, "warm_replays", lambda g, s: 1)
    monkeypatch.setattr(bench, "graph_replay_time", lambda g, steps: g.per_call_ms)
    got = []

    class Sink:
        def add(self, wl, leg, i, steps, v):
            got.append(steps)

    s = bench.measure(None, 20, 5, 0.1, Sink(), "wl", "call")
    assert s["calls_per_sample"] * per_call >= bench.MIN_SAMPLE_MS
    assert set(got) == {s["calls_per_sample"]}
    s = bench.measure(None, 500, 5, 0.1, Sink(), "wl", "call")   # 5 ms: unchanged
    assert s["calls_per_sample"] == 500
