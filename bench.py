#!/usr/bin/env python3
"""Throughput of the INT8 quantized linear on one MI355X.

A step is one full linear call -- per-token activation quantization, the
INT8 MFMA GEMM and its fused dequant+bias epilogue -- on the largest DiT
workload (W8A8, M=16384 tokens, K=3072, N=12288, bf16 out: a 4K-scale
image's tokens through an MLP-width projection), with the offline weight
quantization done once before timing.  Inputs are seeded synthetic draws
(the pages' models and prompts are not available), resident in HBM before
the timed region; working sets under 512 MB are rotated over enough
independent copies that the 256 MB Infinity Cache cannot hold them.

Timing protocol (mlx-kquant pull request 89 commit list: the DiT shape
harness, discarding the first call of a shape visit, median CIs, raw
samples on disk before the summaries; MLX pull request 4722: median of
nine pairs):
  - W eager warmup steps, then the K timed steps are captured in one HIP
    graph (host launch overhead does not bound microsecond-scale calls);
  - the graph is replayed untimed for at least 0.5 s (the clock and the
    caches settle: the first replays run measurably slower);
  - then each sample is one replay of exactly K steps, bracketed by
    synchronizations and HIP events on the replaying stream; value and
    ms_per_step are the MEDIAN of the samples (at least 9), with a
    distribution-free 95% confidence interval;
  - every raw sample is appended to a JSONL file (--samples-out) as it is
    taken, before any summary; --reaggregate rebuilds the summaries from
    such a file without a GPU.
The GEMM kernel alone is timed the same way through kq_w8a8_gemm on the
same pre-quantized activations: that median gives the roofline figure.
Measured floors beside the published peaks: an MFMA-only loop
(kq_probe_mfma_i8) and a streaming read (kq_probe_read).  The CPU oracle
is timed on the host after the GPU runs, on a bounded sample of each
workload.

--save-hashes PATH / --check-hashes PATH (MLX pull request 4722,
"Exactness": outputs hashed on one build and checked on another) hash every
workload's output at seed 0, so a change of kernels, routes or levers can
be shown bit-identical.

Prints ONE JSON line (rank 0, N=1).  `--gpus N` with N > 1 exits: this
build targets one GPU.
"""
from __future__ import annotations

import argparse
import contextlib
import hashlib
import json
import math
import os
import platform
import statistics
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0   # MI355X dense INT8 MFMA, tera-ops/s
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E, GB/s
PEAK_FP16_TFLOPS = 2500.0  # MI355X dense FP16 MFMA
ROTATE_BYTES = 512 << 20  # working set rotated per timed pass
METRIC = "W8A8/W4A8 GEMM INT8 TOPS + % of INT8 MFMA peak; GEMV GB/s at M≤16"
HEADLINE_WARM_S = 0.5
EXTRA_WARM_S = 0.2


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------ statistics
def median_ci95(xs):
    """Median and a distribution-free 95% confidence interval for it from
    order statistics: the narrowest symmetric pair (x_(j), x_(n+1-j)) whose
    binomial(n, 1/2) coverage 1 - 2 P[Bin(n, 1/2) < j] is at least 95%.
    Returns (median, (lo, hi), coverage)."""
    v = sorted(xs)
    n = len(v)
    if n == 0:
        raise ValueError("no samples")
    med = statistics.median(v)
    if n < 6:
        return med, (v[0], v[-1]), 1.0
    # P[Bin(n,1/2) <= i] accumulated with exact integers
    total = 1 << n
    cdf, term = 0, 1                      # term = C(n, i)
    best = (v[0], v[-1], 1.0)
    for j in range(1, n // 2 + 1):
        cdf += term                       # now P[Bin < j] * 2^n
        term = term * (n - (j - 1)) // j
        cover = 1.0 - 2.0 * (cdf / total)
        if cover < 0.95:
            break
        best = (v[j - 1], v[n - j], cover)
    return med, (best[0], best[1]), best[2]


def summarize(samples, steps):
    med, (lo, hi), cover = median_ci95(samples)
    return {"n": len(samples), "steps_each": steps,
            "ms_per_step": [round(x, 6) for x in samples],
            "median_ms_per_step": round(med, 6),
            "ci95_ms_per_step": [round(lo, 6), round(hi, 6)], "ci_coverage": round(cover, 4)}


class SampleSink:
    """Raw samples, appended and flushed to JSONL as they are taken."""

    def __init__(self, path: str):
        self.path = path
        self.run = f"{time.strftime('%Y%m%dT%H%M%S')}-{os.getpid()}"
        self.f = open(path, "a")

    def add(self, workload, leg, i, steps, ms):
        self.f.write(json.dumps({"run": self.run, "workload": workload, "leg": leg, "sample": i,
                                 "steps": steps, "ms_per_step": ms}) + "\n")
        self.f.flush()


def reaggregate(path: str) -> int:
    """Per (run, workload, leg) medians and CIs rebuilt from a raw-sample
    file; one JSON line each.  Needs no GPU."""
    groups = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line:
                continue
            r = json.loads(line)
            groups.setdefault((r["run"], r["workload"], r["leg"]), []).append(r)
    for (run, wl, leg), rs in groups.items():
        xs = [r["ms_per_step"] for r in rs]
        s = summarize(xs, rs[0]["steps"])
        print(json.dumps({"run": run, "workload": wl, "leg": leg, **s}))
    return 0


# ------------------------------------------------------------ workloads
def algorithmic_bytes(wl, M=None) -> int:
    """Compulsory HBM bytes of one linear call: bf16 x, the weights (int8 +
    fp32 scale, or int4 + fp16 scale and offset per 64-group = 0.5625 B per
    weight), the fp32 bias and y."""
    M = wl.M if M is None else M
    x = 2 * M * wl.K
    if wl.fmt == "w8":
        w = wl.N * wl.K + 4 * wl.N
    else:
        w = wl.N * wl.K // 2 + 4 * wl.N * (wl.K // 64)
    y = (4 if wl.out == "f32" else 2) * M * wl.N
    return x + w + 4 * wl.N + y


def weight_bytes(wl) -> int:
    if wl.fmt == "w8":
        return wl.N * wl.K + 4 * wl.N
    return wl.N * wl.K // 2 + 4 * wl.N * (wl.K // 64)


def dev(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits):
    import numpy as np
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


@contextlib.contextmanager
def env_lever(name: str, value: str):
    """Set an environment lever for the duration (restored afterwards)."""
    prev = os.environ.get(name)
    os.environ[name] = value
    try:
        yield
    finally:
        if prev is None:
            del os.environ[name]
        else:
            os.environ[name] = prev


class Prepared:
    """Device-resident inputs of one workload, in R rotation copies."""

    def __init__(self, wl, seed=0, x_override=None, max_copies=16):
        import torch
        import synth
        import w8a8_gemm_dit_amd as kq

        self.wl = wl
        self.kq = kq
        self.out_dtype = torch.float32 if wl.out == "f32" else torch.bfloat16
        x0 = dev_bf16(synth.activations(wl, seed)) if x_override is None else x_override
        wd = dev(synth.weights(wl, seed))
        b0 = dev(synth.bias(wl, seed))
        fmt = kq.KQ_W8_PER_CHANNEL if wl.fmt == "w8" else kq.KQ_W4_AFFINE_G64
        self.fmt = fmt
        # int4 weights on the tiled GEMM: the linear hands that kernel its
        # codes in the split order, so the kernel-only leg does the same
        self.order = (kq.KQ_CODES_SPLIT8 if fmt == kq.KQ_W4_AFFINE_G64
                      and kq.kq_route(wl.M, wl.N, wl.K, fmt)["kind"] == "gemm"
                      else kq.KQ_CODES_NATURAL)
        wq, sc, gb = kq.kq_quantize_weights(wd, fmt)
        del wd
        ws_bytes = kq.kq_workspace_bytes(wl.M, wl.N, wl.K, fmt)  # any route of the shape
        ysz = wl.M * wl.N * (4 if wl.out == "f32" else 2)
        per_copy = (x0.numel() * 2 + wq.numel() + sc.numel() * sc.element_size()
                    + (0 if gb is None else gb.numel() * 2) + 4 * wl.N + ysz + ws_bytes)
        self.R = max(1, min(max_copies, math.ceil(ROTATE_BYTES / per_copy)))
        self.copies = []
        for r in range(self.R):
            c = {
                "x": x0 if r == 0 else x0.clone(),
                "wq": wq if r == 0 else wq.clone(),
                "sc": sc if r == 0 else sc.clone(),
                "gb": None if gb is None else (gb if r == 0 else gb.clone()),
                "b": b0 if r == 0 else b0.clone(),
                "y": torch.empty((wl.M, wl.N), dtype=self.out_dtype, device="cuda"),
                "ws": torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device="cuda"),
            }
            a, sx, gs = kq.kq_quantize_act_ordered(c["x"], self.order,
                                                   group_sums=(fmt == kq.KQ_W4_AFFINE_G64))
            c.update(a=a, sx=sx, gs=gs)
            self.copies.append(c)
        torch.cuda.synchronize()

    def step(self, i: int) -> None:
        c = self.copies[i % self.R]
        kq = self.kq
        if self.fmt == kq.KQ_W8_PER_CHANNEL:
            kq.kq_w8a8_linear(c["x"], c["wq"], c["sc"], c["b"], out_dtype=self.out_dtype,
                              out=c["y"], workspace=c["ws"])
        else:
            kq.kq_w4a8_linear(c["x"], c["wq"], c["sc"], c["gb"], c["b"], out_dtype=self.out_dtype,
                              out=c["y"], workspace=c["ws"])

    def quant(self, i: int) -> None:
        """The activation quantize kernel alone (into the copy's codes)."""
        c = self.copies[i % self.R]
        self.kq.kq_quantize_act_ordered(c["x"], self.order, out=(c["a"], c["sx"], c["gs"]),
                                        group_sums=c["gs"] is not None)

    def add_gate(self, gate_rows: int, seed: int = 0) -> None:
        """fp32 gates [ceil(M/gate_rows), N] for the gated residual calls."""
        import synth
        self.gate_rows = gate_rows
        g = dev(synth.random_f32((-(-self.wl.M // gate_rows), self.wl.N), seed=seed + 40,
                                 scale=0.5))
        for r, c in enumerate(self.copies):
            c["gate"] = g if r == 0 else g.clone()

    def gated(self, i: int) -> None:
        """The DiT residual update in place: y += gate[m / L] * linear(x)."""
        c = self.copies[i % self.R]
        self.kq.kq_linear_gated(self.fmt, c["x"], c["wq"], c["sc"], c["gb"], c["b"],
                                residual=c["y"], gate=c["gate"], gate_rows=self.gate_rows,
                                out_dtype=self.out_dtype, out=c["y"], workspace=c["ws"])

    def gemm(self, i: int) -> None:
        c = self.copies[i % self.R]
        kq = self.kq
        if self.fmt == kq.KQ_W8_PER_CHANNEL:
            kq.kq_w8a8_gemm(c["a"], c["sx"], c["wq"], c["sc"], c["b"], out_dtype=self.out_dtype,
                            out=c["y"])
        else:
            kq.kq_w4a8_gemm_ordered(c["a"], c["sx"], c["gs"], c["wq"], c["sc"], c["gb"],
                                    self.order, c["b"], out_dtype=self.out_dtype, out=c["y"])

    def output_hash(self) -> str:
        """sha256 of copy 0's output after one call."""
        import torch
        self.step(0)
        torch.cuda.synchronize()
        y = self.copies[0]["y"]
        raw = y.view(torch.int16 if y.dtype == torch.bfloat16 else torch.int32).cpu().numpy()
        return hashlib.sha256(raw.tobytes()).hexdigest()


class PreparedAttention:
    """Device-resident q/k/v, output and workspace of one attention
    workload (its working set is far above the Infinity Cache, so one
    copy)."""

    def __init__(self, wl, seed=0):
        import torch
        import synth
        import w8a8_gemm_dit_amd as kq

        self.wl, self.kq = wl, kq
        q, k, v = synth.attention_inputs(wl.B, wl.H, wl.Lq, wl.Lk, seed=seed)
        self.q, self.k, self.v = (torch.from_numpy(t).cuda() for t in (q, k, v))
        del q, k, v
        self.out = torch.empty_like(self.q)
        self.ws = kq.kq_sage_prepare(self.q, self.k, self.v, wl.q_block, wl.k_block)
        torch.cuda.synchronize()

    def step(self, i: int) -> None:
        """The whole call: preparation + attention."""
        self.kq.kq_sage_attention(self.q, self.k, self.v, q_block=self.wl.q_block,
                                  k_block=self.wl.k_block, out=self.out, workspace=self.ws)

    def attend(self, i: int) -> None:
        """The attention kernel alone, on the prepared workspace."""
        w = self.wl
        self.kq.kq_sage_attend(self.ws, w.B, w.H, w.Lq, w.Lk, out=self.out, k_block=w.k_block)

    def output_hash(self) -> str:
        import torch
        self.step(0)
        torch.cuda.synchronize()
        raw = self.out.view(torch.int16).cpu().numpy()
        return hashlib.sha256(raw.tobytes()).hexdigest()


def attention_peak_tops() -> float:
    """Dense MFMA bound of the INT8 attention: half its operations run at
    the INT8 rate (QK^T), half at the FP16 rate (P.V)."""
    return 1.0 / (0.5 / PEAK_INT8_TOPS + 0.5 / PEAK_FP16_TFLOPS)


# ------------------------------------------------------------ timing
def graph_capture(fn, steps: int):
    """Capture `steps` calls of fn(i) in one HIP graph (after one call
    outside the capture that touches everything)."""
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i)
    torch.cuda.synchronize()
    return g


def warm_replays(g, seconds: float, min_replays: int = 3) -> int:
    """Untimed replays for at least `seconds` (and `min_replays`)."""
    import torch

    t0 = time.perf_counter()
    n = 0
    while n < min_replays or time.perf_counter() - t0 < seconds:
        g.replay()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def graph_replay_time(g, steps: int) -> float:
    """One timed replay of a captured graph of `steps` calls, bracketed by
    synchronizations and events on the replaying (current) stream; returns
    ms per call."""
    import torch

    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


MIN_SAMPLE_MS = 1.0  # a timed sample (one replay) lasts at least this long
MAX_CALLS_PER_SAMPLE = 4000


def measure(fn, steps: int, n_samples: int, warm_s: float, sink: SampleSink, workload: str,
            leg: str) -> dict:
    """Capture, warm for warm_s, then n_samples timed replays of `steps`
    calls; raw samples go to the sink first.  Returns the summary with the
    median in "ms".  A replay shorter than MIN_SAMPLE_MS is re-captured with
    proportionally more calls (fast shapes get more calls per sample, so
    every sample spans at least a millisecond of GPU time)."""
    g = graph_capture(fn, steps)
    nw = warm_replays(g, warm_s)
    t = graph_replay_time(g, steps) * steps
    if t < MIN_SAMPLE_MS and steps < MAX_CALLS_PER_SAMPLE:
        steps = min(MAX_CALLS_PER_SAMPLE, math.ceil(steps * MIN_SAMPLE_MS / max(t, 1e-4)))
        del g
        g = graph_capture(fn, steps)
        nw += warm_replays(g, min(warm_s, 0.1))
    xs = []
    for i in range(n_samples):
        v = graph_replay_time(g, steps)
        sink.add(workload, leg, i, steps, v)
        xs.append(v)
    del g
    s = summarize(xs, steps)
    s["warm_replays"] = nw
    s["calls_per_sample"] = steps
    s["ms"] = s["median_ms_per_step"]
    return s


def eager_time(fn, steps: int) -> float:
    import torch

    st = torch.cuda.current_stream()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for i in range(steps):
        fn(i)
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


# ------------------------------------------------------------ floors
def mfma_floor(sink: SampleSink) -> dict:
    """INT8 MFMA rate of a loop with no memory traffic (2 waves per SIMD)."""
    import w8a8_gemm_dit_amd as kq

    iters, grid = 4000, 512
    ops = (1 << 21) * iters * grid       # 8 waves x 8 MFMAs x 2^15 ops per iteration
    m = measure(lambda i: kq.kq_probe_mfma_i8(iters, grid), 4, 9, 0.2, sink, "probe_mfma_i8",
                "kernel")
    tops = ops / (m["ms"] * 1e-3) / 1e12
    return {"tops": round(tops, 1), "pct_of_peak": round(100 * tops / PEAK_INT8_TOPS, 2),
            "ms": m["ms"], "kernel": "probe_mfma_i8", "grid": grid, "iters": iters}


def read_floor(nbytes: int, grid: int, threads: int, sink: SampleSink, tag: str) -> dict:
    """HBM read rate of a plain streaming read of nbytes with this grid,
    rotated over enough buffers that the Infinity Cache cannot hold them."""
    import torch
    import w8a8_gemm_dit_amd as kq

    nbytes = (nbytes + 15) // 16 * 16
    R = max(1, min(16, math.ceil(ROTATE_BYTES / nbytes)))
    bufs = [torch.full((nbytes,), r + 1, dtype=torch.uint8, device="cuda") for r in range(R)]
    sinks = [torch.zeros((grid,), dtype=torch.int32, device="cuda") for _ in range(R)]
    m = measure(lambda i: kq.kq_probe_read(bufs[i % R], grid, threads, sinks[i % R]), 4 * R, 9,
                0.2, sink, tag, "kernel")
    gbs = nbytes / (m["ms"] * 1e-3) / 1e9
    del bufs, sinks
    return {"gbs": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
            "us": round(m["ms"] * 1e3, 3), "bytes": nbytes, "grid": grid, "threads": threads,
            "kernel": "probe_read"}


# ------------------------------------------------------------ CPU baseline
def cpu_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max((d.get("num_threads", 1) for d in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def cpu_oracle(wl, rows=None, budget_s: float = 2.0, max_runs: int = 50, x_bits=None) -> dict:
    """The oracle as it stands (numpy: fp32 quantizers, fp64 product, output
    rounding) on the first `rows` rows of the workload (all rows if None),
    repeated until about budget_s; the median run time scaled to the whole
    workload when rows < M ("extrapolated")."""
    import numpy as np
    import oracle
    import synth

    M = wl.M if rows is None else min(rows, wl.M)
    xb = synth.activations(wl, rows=M) if x_bits is None else x_bits[:M]
    w, b = synth.weights(wl), synth.bias(wl)
    if wl.fmt == "w8":
        q8, sw = oracle.quantize_w8(w)
        run = lambda: oracle.w8a8_linear_exact(xb, q8, sw, b)      # noqa: E731
    else:
        _, gs, gb, q = oracle.quantize_w4(w)
        run = lambda: oracle.w4a8_linear_exact(xb, q, gs, gb, b)   # noqa: E731
    del w
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        y = run()
        y32 = oracle.round_f32(y)
        if wl.out == "bf16":
            oracle.round_bf16_bits(y32)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= max_runs:
            break
    med = statistics.median(times)
    per_call = med * wl.M / M
    return {"value": round(wl.ops / per_call / 1e12, 5), "unit": "TOPS",
            "s_per_call": round(per_call, 5), "rows_timed": M, "extrapolated": M < wl.M,
            "runs": len(times)}


def cpu_baseline(wl, budget_s: float = 12.0) -> dict:
    """The headline cpu_baseline object: the oracle on a bounded sample of
    the headline workload (its first 512 rows, scaled to all M rows)."""
    r = cpu_oracle(wl, rows=512, budget_s=budget_s)
    return {
        "value": r["value"], "unit": "TOPS", "cores": int(cpu_threads()), "kind": "oracle",
        "sample": (f"first 512 of {wl.M} rows of {wl.name} (per-token quantize + fp64 product + "
                   f"bf16 rounding), median of {r['runs']} runs, scaled by M/512 "
                   f"(extrapolated): {r['s_per_call']:.3f} s per full call; host "
                   f"{platform.processor() or platform.machine()}, "
                   f"{len(os.sched_getaffinity(0))} cores visible"),
    }


# ------------------------------------------------------------ traffic
_KERNEL_SOURCES = {
    "gemm_w8a8": ("gemm_w8a8.hip", "kq_common.hpp"),
    "gemm_w4a8": ("gemm_w4a8.hip", "kq_common.hpp"),
    "gemv": ("gemv.hip", "kq_common.hpp"),
    "thin_fused": ("thin_fused.hip", "kq_common.hpp"),
    "quant_act": ("quant.hip", "kq_common.hpp"),
}


def kernel_source_hash(kernel: str) -> str:
    """sha256 (16 hex digits) of the sources of the named kernel."""
    files = next((v for k, v in _KERNEL_SOURCES.items() if kernel.startswith(k)), None)
    if files is None:
        return ""
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "w8a8_gemm_dit_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` at `workload` from the committed
    counter summary, or None if absent or taken on a different source."""
    p = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(f"{kernel}@{workload}")
    except Exception:
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


# ------------------------------------------------------------ trace summaries
def summarize_trace(path: str) -> int:
    """Per (kernel, grid) dispatch counts and average durations from a
    rocprofv3 --kernel-trace CSV (the file or a directory holding one), as
    a markdown table."""
    import csv
    import glob

    files = [path] if os.path.isfile(path) else glob.glob(
        os.path.join(path, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        print(f"no kernel_trace.csv under {path}", file=sys.stderr)
        return 1
    agg = {}
    for fn in files:
        with open(fn) as f:
            for r in csv.DictReader(f):
                name = r.get("Kernel_Name", "?")
                grid = "x".join(r.get(k, "?") for k in ("Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"))
                d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
                agg.setdefault((name, grid), []).append(d)
    print("| kernel | grid (threads x,y,z) | dispatches | average us | median us |")
    print("|---|---|---:|---:|---:|")
    for (name, grid), ds in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        short = name if len(name) < 90 else name[:87] + "..."
        print(f"| `{short}` | {grid} | {len(ds)} | {sum(ds) / len(ds) / 1e3:.2f} | "
              f"{statistics.median(ds) / 1e3:.2f} |")
    return 0


# ------------------------------------------------------------ counter summaries
def short_kernel_name(name: str) -> str:
    """The launch name of a libkq kernel (the route's name for it, as KQ_LOG
    prints it) from its full template name; the full name if unknown."""
    import re

    m = re.search(r"gemm_w8a8_kernel<(\d+), (\d+), (\d+), (\d+)", name)
    if m:
        bm, bn, wm, wn = (int(v) for v in m.groups())
        return f"gemm_w8a8_{bm}x{bn}" + ("w8" if bm == bn == 256 and wm * wn == 8 else "")
    m = re.search(r"gemm_w4a8_kernel<(\d+), (\d+),", name)
    if m:
        return f"gemm_w4a8_{m.group(1)}x{m.group(2)}"
    if "gemv_lane_kernel" in name:
        return "gemv_w4a8_lane"
    if "gemv_lane8_kernel" in name:
        return "gemv_w8a8_lane"
    m = re.search(r"gemv_kernel<(true|false)", name)
    if m:
        return "gemv_w4a8" if m.group(1) == "true" else "gemv_w8a8"
    if "quant_act" in name:
        return "quant_act"
    if "thin_fused" in name:
        return "thin_fused"
    return name


def _counter_values(path: str, counter: str) -> dict:
    """(kernel, grid threads) -> per-dispatch values (KiB) of one counter
    from rocprofv3 --pmc CSV output under path."""
    import csv
    import glob

    out = {}
    for fn in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        with open(fn) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                key = (r["Kernel_Name"], int(r["Grid_Size"]))
                out.setdefault(key, {})[r["Dispatch_Id"]] = (
                    out.get(key, {}).get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"]))
    return {k: list(v.values()) for k, v in out.items()}


def summarize_counters(dirs: str, copy_mib: int, workload: str, traffic_out: str) -> int:
    """Markdown table of FETCH_SIZE / WRITE_SIZE per kernel from four
    rocprofv3 --pmc passes (dirs = FETCH,WRITE,COPY_FETCH,COPY_WRITE), each
    counter scaled by what it reads for a plain device copy of copy_mib MiB.
    With a workload name and traffic_out, the libkq kernels' bytes per
    launch go into that JSON file under "kernel@workload", with the hash of
    their sources."""
    fd, wd, cfd, cwd = dirs.split(",")
    fetch, write = _counter_values(fd, "FETCH_SIZE"), _counter_values(wd, "WRITE_SIZE")
    cfetch, cwrite = _counter_values(cfd, "FETCH_SIZE"), _counter_values(cwd, "WRITE_SIZE")

    def copy_avg(vals):
        xs = [v for (n, _), d in vals.items() if "copy" in n.lower() for v in d]
        return sum(xs) / len(xs) if xs else float("nan")

    nkib = copy_mib * 1024
    sf, sw = nkib / copy_avg(cfetch), nkib / copy_avg(cwrite)
    print(f"Scale: a {copy_mib} MiB device copy ({nkib} KiB read and written) reads "
          f"{nkib / sf:.0f} KiB of FETCH_SIZE and {nkib / sw:.0f} KiB of WRITE_SIZE, so "
          f"FETCH_SIZE is multiplied by {sf:.4f} and WRITE_SIZE by {sw:.4f}.\n")
    print("| kernel | grid threads | dispatches | FETCH_SIZE KiB (avg) | WRITE_SIZE KiB (avg) "
          "| scaled MB read | scaled MB written |")
    print("|---|---:|---:|---:|---:|---:|---:|")
    rec = {}
    for key in sorted(fetch, key=lambda k: -sum(fetch[k]) / len(fetch[k])):
        name, grid = key
        f = sum(fetch[key]) / len(fetch[key])
        w = sum(write.get(key, [0.0])) / max(1, len(write.get(key, [])))
        short = short_kernel_name(name)
        shown = short if short != name else (name if len(name) < 60 else name[:57] + "...")
        print(f"| `{shown}` | {grid} | {len(fetch[key])} | {f:.0f} | {w:.0f} | "
              f"{f * sf * 1024 / 1e6:.1f} | {w * sw * 1024 / 1e6:.1f} |")
        if short != name and kernel_source_hash(short):
            fb, wb = f * sf * 1024, w * sw * 1024
            prev = rec.get(short)
            if prev is None or prev["dispatches"] < len(fetch[key]):
                rec[short] = {"bytes_per_launch": round(fb + wb), "fetch_bytes": round(fb),
                              "write_bytes": round(wb), "dispatches": len(fetch[key]),
                              "grid_threads": grid, "source_hash": kernel_source_hash(short)}
    if workload and traffic_out:
        data = json.load(open(traffic_out)) if os.path.exists(traffic_out) else {}
        data = {k: v for k, v in data.items() if "@" in k}  # entries keyed by workload only
        for short, r in rec.items():
            data[f"{short}@{workload}"] = r
        with open(traffic_out, "w") as fh:
            json.dump(data, fh, indent=1, sort_keys=True)
            fh.write("\n")
        print(f"\n{len(rec)} kernel(s) of {workload} written to {traffic_out}", file=sys.stderr)
    return 0


def summarize_pmc(path: str, workload: str = "", clock_out: str = "") -> int:
    """Per (kernel, grid) averages over dispatches of every counter in a
    rocprofv3 --pmc CSV output directory, as a markdown table.  With a
    workload name and clock_out, the libkq kernels' sustained clock and MFMA /
    VALU busy shares are recorded in clock_out (keyed kernel@workload, with
    the kernel's source hash)."""
    import csv
    import glob

    vals, counters, dur = {}, [], {}
    for fn in glob.glob(os.path.join(path, "**", "*kernel_trace.csv"), recursive=True):
        with open(fn) as f:
            for r in csv.DictReader(f):
                dur[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    for fn in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        with open(fn) as f:
            for r in csv.DictReader(f):
                c = r["Counter_Name"]
                if c not in counters:
                    counters.append(c)
                key = (short_kernel_name(r["Kernel_Name"]), int(r["Grid_Size"]))
                d = vals.setdefault(key, {}).setdefault(c, {})
                d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not vals:
        print(f"no counter_collection.csv under {path}", file=sys.stderr)
        return 1
    # With the dispatches' durations (--kernel-trace in the same run):
    # GRBM_GUI_ACTIVE summed over the 8 XCDs / duration = the shader clock,
    # and the MFMA / VALU busy shares of those cycles over 1024 SIMDs
    # (SQ_ACTIVE_INST_VALU counts quad-cycles).
    derived = ["avg us"] if dur else []
    if dur and "GRBM_GUI_ACTIVE" in counters:
        derived.append("clock GHz")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in counters:
            derived.append("MFMA busy %")
        if "SQ_ACTIVE_INST_VALU" in counters:
            derived.append("VALU busy %")
    rec = {}
    print("| kernel | grid threads | dispatches | " + " | ".join(counters + derived) + " |")
    print("|---|---:|---:|" + "---:|" * (len(counters) + len(derived)))
    for (name, grid), cs in sorted(vals.items(), key=lambda kv: kv[0]):
        ids = sorted(set().union(*(v.keys() for v in cs.values())))
        cells = [f"{sum(cs[c].values()) / len(cs[c]):.4g}" if c in cs else "" for c in counters]
        ds = [dur[i] for i in ids if i in dur]
        if derived and ds:
            us = sum(ds) / len(ds)
            cells.append(f"{us:.2f}")
            if "clock GHz" in derived:
                gui = sum(cs["GRBM_GUI_ACTIVE"].values()) / len(cs["GRBM_GUI_ACTIVE"]) / 8
                r = {"clock_ghz": round(gui / us / 1e3, 3), "avg_us": round(us, 3),
                     "cycles": round(gui), "dispatches": len(ds)}
                cells.append(f"{gui / us / 1e3:.2f}")
                if "MFMA busy %" in derived:
                    m = sum(cs["SQ_VALU_MFMA_BUSY_CYCLES"].values()) / len(cs["SQ_VALU_MFMA_BUSY_CYCLES"])
                    cells.append(f"{100 * m / 1024 / gui:.1f}")
                    r["mfma_busy_pct"] = round(100 * m / 1024 / gui, 2)
                if "VALU busy %" in derived:
                    v = sum(cs["SQ_ACTIVE_INST_VALU"].values()) / len(cs["SQ_ACTIVE_INST_VALU"])
                    cells.append(f"{100 * 4 * v / 1024 / gui:.1f}")
                    r["valu_busy_pct"] = round(100 * 4 * v / 1024 / gui, 2)
                if kernel_source_hash(name):
                    r["source_hash"] = kernel_source_hash(name)
                    prev = rec.get(name)
                    if prev is None or prev["dispatches"] < r["dispatches"]:
                        rec[name] = r
        elif derived:
            cells += [""] * len(derived)
        shown = name if len(name) < 60 else name[:57] + "..."
        print(f"| `{shown}` | {grid} | {len(ids)} | " + " | ".join(cells) + " |")
    if workload and clock_out:
        data = json.load(open(clock_out)) if os.path.exists(clock_out) else {}
        for k, r in rec.items():
            data[f"{k}@{workload}"] = r
        with open(clock_out, "w") as fh:
            json.dump(data, fh, indent=1, sort_keys=True)
        print(f"\n{len(rec)} kernel(s) of {workload} written to {clock_out}", file=sys.stderr)
    return 0


def recorded_clock(kernel: str, workload: str):
    """The sustained clock record of `kernel` at `workload` from the committed
    counter summary, or None if absent or taken on a different source."""
    p = os.path.join(ROOT, "profiles", "sustained_clock.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(f"{kernel}@{workload}")
    except Exception:
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash(kernel):
        return None
    return rec


# ------------------------------------------------------------ hashes
def output_hashes(workloads=None) -> dict:
    import torch
    import synth

    out = {}
    names = list(synth.WORKLOADS) + list(synth.ATTN_WORKLOADS)
    for name in names:
        if workloads and name not in workloads:
            continue
        if name in synth.WORKLOADS:
            p = Prepared(synth.WORKLOADS[name], max_copies=1)
        else:
            p = PreparedAttention(synth.ATTN_WORKLOADS[name])
        out[name] = p.output_hash()
        log(f"hash {name}: {out[name][:16]}")
        del p
        torch.cuda.empty_cache()
    return out


# ------------------------------------------------------------ main
def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="calls per timed sample (graph replay)")
    ap.add_argument("--warmup", type=int, default=5, help="eager warmup calls before capture")
    ap.add_argument("--samples", type=int, default=9,
                    help="timed samples (replays of --steps calls) of the headline legs; "
                         "value is their median")
    ap.add_argument("--quick", action="store_true", help="headline only, no extra workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="few eager steps of every workload, for profiler runs")
    ap.add_argument("--workload", default="", metavar="NAME",
                    help="with --profile or the hash modes: only this workload")
    ap.add_argument("--samples-out", default="", metavar="PATH",
                    help="JSONL file the raw samples are appended to as they are taken "
                         "(default: a file in the temporary directory, named on stderr)")
    ap.add_argument("--reaggregate", default="", metavar="PATH",
                    help="rebuild the per-leg medians and CIs from a raw-sample file (no GPU)")
    ap.add_argument("--save-hashes", default="", metavar="PATH",
                    help="write the sha256 of every workload's output at seed 0 and exit")
    ap.add_argument("--check-hashes", default="", metavar="PATH",
                    help="recompute the output hashes and compare them with PATH; exit 1 on "
                         "any difference")
    ap.add_argument("--summarize-trace", default="", metavar="PATH",
                    help="per-kernel averages from a rocprofv3 kernel-trace CSV (no GPU)")
    ap.add_argument("--summarize-counters", default="", metavar="F,W,CF,CW",
                    help="FETCH_SIZE/WRITE_SIZE table from four rocprofv3 --pmc output "
                         "directories (the run, then the copy probe; no GPU)")
    ap.add_argument("--summarize-pmc", default="", metavar="DIR",
                    help="per-kernel averages of every counter in a rocprofv3 --pmc output "
                         "directory (no GPU)")
    ap.add_argument("--clock-out", default="", metavar="JSON",
                    help="with --summarize-pmc and --workload: record the libkq kernels' "
                         "sustained clock and MFMA / VALU busy shares in this file")
    ap.add_argument("--copy-mib", type=int, default=256,
                    help="size of the copy probe the counters are scaled by")
    ap.add_argument("--traffic-out", default="", metavar="JSON",
                    help="with --summarize-counters and --workload: record the libkq "
                         "kernels' bytes per launch in this file")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 3 plain device-to-device copies of MIB MiB, the known-size "
                         "reference that scales HBM byte counters")
    args = ap.parse_args()
    if args.reaggregate:
        return reaggregate(args.reaggregate)
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace)
    if args.summarize_pmc:
        return summarize_pmc(args.summarize_pmc, args.workload, args.clock_out)
    if args.summarize_counters:
        return summarize_counters(args.summarize_counters, args.copy_mib, args.workload,
                                  args.traffic_out)
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; this build runs on one GPU "
              "(the linear would shard by output rows or columns with no collective).",
              file=sys.stderr)
        return 2

    import torch
    import synth
    import w8a8_gemm_dit_amd as kq

    torch.cuda.set_device(0)
    if not kq.kq_is_available():
        print("bench.py: device 0 is not a gfx950 GPU", file=sys.stderr)
        return 1
    log(f"device {torch.cuda.get_device_name(0)}")

    if args.copy_probe > 0:
        n = args.copy_probe << 20
        src = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: 3 copies of {n} bytes")
        return 0

    if args.save_hashes or args.check_hashes:
        only = {args.workload} if args.workload else None
        hashes = output_hashes(only)
        if args.save_hashes:
            with open(args.save_hashes, "w") as f:
                json.dump(hashes, f, indent=1, sort_keys=True)
            print(json.dumps({"saved": len(hashes), "path": args.save_hashes}))
            return 0
        ref = json.load(open(args.check_hashes))
        same = [k for k in hashes if ref.get(k) == hashes[k]]
        diff = [k for k in hashes if k in ref and ref[k] != hashes[k]]
        missing = [k for k in hashes if k not in ref]
        print(json.dumps({"bit_identical": f"{len(same)}/{len(hashes)}", "different": diff,
                          "not_in_reference": missing}))
        return 0 if not diff and not missing else 1

    if args.profile:
        for name, wl in synth.WORKLOADS.items():
            if args.workload and name != args.workload:
                continue
            p = Prepared(wl)
            for i in range(max(args.steps, 1)):
                p.step(i)
            for i in range(max(args.steps, 1)):
                p.gemm(i)
            torch.cuda.synchronize()
            log(f"profiled {name}")
            del p
            torch.cuda.empty_cache()
        for name, wl in synth.ATTN_WORKLOADS.items():
            if args.workload and name != args.workload:
                continue
            p = PreparedAttention(wl)
            for i in range(max(args.steps, 1)):
                p.step(i)
            torch.cuda.synchronize()
            log(f"profiled {name}")
            del p
            torch.cuda.empty_cache()
        return 0

    sink = SampleSink(args.samples_out or os.path.join(
        tempfile.gettempdir(), f"kq_bench_samples_{os.getpid()}.jsonl"))
    log(f"raw samples -> {sink.path} (run {sink.run})")
    n_head = max(9, args.samples)
    steps = max(1, args.steps)

    # ---- headline: the whole linear call, then its GEMM kernel alone
    wl = synth.WORKLOADS[synth.HEADLINE]
    p = Prepared(wl)
    log(f"{wl.name}: {p.R} rotation copies")
    for i in range(args.warmup):
        p.step(i)
    torch.cuda.synchronize()
    call = measure(p.step, steps, n_head, HEADLINE_WARM_S, sink, wl.name, "call")
    gemm = measure(p.gemm, steps, n_head, HEADLINE_WARM_S, sink, wl.name, "gemm_kernel")
    quant = measure(p.quant, steps, 5, EXTRA_WARM_S, sink, wl.name, "quant_kernel")
    ms_eager = eager_time(p.step, steps)
    ms, ms_gemm = call["ms"], gemm["ms"]
    log(f"call {ms * 1e3:.2f} us/step (median of {call['n']}, CI "
        f"[{call['ci95_ms_per_step'][0] * 1e3:.2f}, {call['ci95_ms_per_step'][1] * 1e3:.2f}]), "
        f"gemm {ms_gemm * 1e3:.2f} us, quantize {quant['ms'] * 1e3:.2f} us, eager "
        f"{ms_eager * 1e3:.2f} us")
    route = kq.kq_route(wl.M, wl.N, wl.K, kq.KQ_W8_PER_CHANNEL)
    gemm_name = f"gemm_w8a8_{route['tile_m']}x{route['tile_n']}" + (
        "w8" if route["tile_m"] == route["tile_n"] == 256 and route["threads"] == 512 else "")
    head_copies = p.R
    del p
    torch.cuda.empty_cache()
    tops = wl.ops / (ms * 1e-3) / 1e12
    gemm_tops = wl.ops / (ms_gemm * 1e-3) / 1e12

    floors = {}
    if not args.quick:
        floors["mfma_i8"] = mfma_floor(sink)
        log(f"MFMA-only loop: {floors['mfma_i8']['tops']} TOPS")
        floors["hbm_read"] = read_floor(256 << 20, 2048, 512, sink, "probe_read_256MiB")
        log(f"streaming read: {floors['hbm_read']['gbs']} GB/s")

    result = {
        "metric": METRIC,
        "value": round(tops, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": wl.name, "M": wl.M, "K": wl.K, "N": wl.N,
                   "weights": "int8 per output channel", "activations": "bf16 -> int8 per token",
                   "x": "Student-t nu=4", "out": wl.out,
                   "pct_of_int8_peak": round(100 * tops / PEAK_INT8_TOPS, 2),
                   "eager_ms_per_step": round(ms_eager, 6), "rotation_copies": head_copies,
                   "timing": (f"median of {call['n']} samples of {steps} calls (one graph "
                              f"replay each) after {call['warm_replays']} untimed replays "
                              f">= {HEADLINE_WARM_S} s")},
        "samples": {**{k: v for k, v in call.items() if k != "ms"},
                    "median_tops": round(tops, 3), "raw_samples_file": sink.path,
                    "method": "replays of the timed graph; distribution-free order-statistic "
                              "interval for the median"},
        "roofline": {
            "kernel": gemm_name,
            "bound": "mfma",
            "achieved": round(gemm_tops, 2),
            "peak": PEAK_INT8_TOPS,
            "unit": "TOP/s",
            "frac": round(gemm_tops / PEAK_INT8_TOPS, 4),
            "traffic": recorded_traffic(gemm_name, wl.name),
            "avg_launch_us": round(ms_gemm * 1e3, 3),
            "launch_ci95_us": [round(x * 1e3, 3) for x in gemm["ci95_ms_per_step"]],
            "algorithmic_ops": wl.ops,
            "algorithmic_bytes": 2 * wl.M * wl.N + wl.M * wl.K + 4 * wl.M + weight_bytes(wl) + 4 * wl.N,
        },
        "call_split": {"quantize_kernel_us": round(quant["ms"] * 1e3, 3),
                       "gemm_kernel_us": round(ms_gemm * 1e3, 3),
                       "call_us": round(ms * 1e3, 3)},
    }
    clk = recorded_clock(gemm_name, wl.name)
    if clk:
        # the peak scaled to the clock the kernel sustains under load (the
        # published peak assumes 2.4 GHz; the package power limit lowers it)
        # A counter run serializes dispatches; the kernel's cycle count from
        # it over the launch time measured here gives the clock it holds
        # in the timed region (its cycles barely move with the clock when
        # it is compute bound); the higher of the two readings is used
        ghz = clk["clock_ghz"]
        if clk.get("cycles"):
            ghz = max(ghz, clk["cycles"] / (ms_gemm * 1e6))
        peak_clk = PEAK_INT8_TOPS * min(ghz, 2.4) / 2.4
        result["roofline"]["sustained_clock_ghz"] = round(ghz, 3)
        result["roofline"]["counter_run_clock_ghz"] = clk["clock_ghz"]
        result["roofline"]["peak_at_sustained_clock"] = round(peak_clk, 1)
        result["roofline"]["frac_at_sustained_clock"] = round(gemm_tops / peak_clk, 4)
        if "mfma_busy_pct" in clk:
            result["roofline"]["mfma_busy_pct"] = clk["mfma_busy_pct"]
    if "mfma_i8" in floors:
        result["roofline"]["measured_mfma_only_tops"] = floors["mfma_i8"]["tops"]
        result["roofline"]["frac_of_measured"] = round(gemm_tops / floors["mfma_i8"]["tops"], 4)
        result["floors"] = floors

    if not args.quick:
        extra = {}
        steps_x = max(10, steps)
        up_out = None
        for name, w in synth.WORKLOADS.items():
            if name == synth.HEADLINE:
                continue
            xo = up_out if name.startswith("dit_mlp_down_w4a8") else None
            pw = Prepared(w, x_override=xo)
            if name.startswith("dit_mlp_up_w4a8"):
                pw.step(0)
                torch.cuda.synchronize()
                up_out = pw.copies[0]["y"].clone()      # the down projection's input
            for i in range(3):
                pw.step(i)
            c = measure(pw.step, steps_x, 5, EXTRA_WARM_S, sink, name, "call")
            t = c["ms"]
            r = kq.kq_route(w.M, w.N, w.K, pw.fmt)
            e = {"ms_per_call": round(t, 5), "ci95_ms": c["ci95_ms_per_step"],
                 "route": r["kind"], "tile": f"{r['tile_m']}x{r['tile_n']}", "splits": r["splits"],
                 "rotation_copies": pw.R}
            if r["kind"] == "fused":
                # one kernel per call: the call is the kernel; the two-kernel
                # route (quantize + GEMV) is timed beside it
                tg = t
                e["kernel_ms_method"] = "the call (one kernel)"
                with env_lever("KQ_FUSE", "0"):
                    e["two_kernel_ms_per_call"] = round(
                        measure(pw.step, steps_x, 5, EXTRA_WARM_S, sink, name, "call_two_kernel")["ms"], 5)
            elif r["splits"] > 1:
                # split K: the product is the tile kernel plus the fold; the
                # entry point on pre-quantized codes never splits, so the
                # route's kernels are the call minus the quantize kernel
                tq = measure(pw.quant, steps_x, 5, EXTRA_WARM_S, sink, name, "quant_kernel")["ms"]
                tg = t - tq
                e["kernel_ms_method"] = "call minus the quantize kernel timed alone (split K + fold)"
                e["quantize_ms"] = round(tq, 5)
            else:
                tg = measure(pw.gemm, steps_x, 5, EXTRA_WARM_S, sink, name, "kernel")["ms"]
                e["kernel_ms_method"] = "the product kernel on pre-quantized codes"
            gbs = algorithmic_bytes(w) / (t * 1e-3) / 1e9
            e.update({
                "kernel_ms": round(tg, 5),
                "tops": round(w.ops / (t * 1e-3) / 1e12, 2),
                "pct_int8_peak": round(100 * w.ops / (t * 1e-3) / 1e12 / PEAK_INT8_TOPS, 2),
                "kernel_tops": round(w.ops / (tg * 1e-3) / 1e12, 2),
                "kernel_pct_int8_peak": round(100 * w.ops / (tg * 1e-3) / 1e12 / PEAK_INT8_TOPS, 2),
                "gbs": round(gbs, 1), "pct_hbm_peak": round(100 * gbs / PEAK_HBM_GBS, 2),
            })
            if w.M <= 16:
                # the same bytes as a plain streaming read with the GEMV's grid
                fl = read_floor(weight_bytes(w), r["grid"], r["threads"], sink,
                                f"probe_read_{name}")
                e["read_floor_same_grid"] = fl
                e["vs_read_floor"] = round(tg * 1e3 / fl["us"], 3)
            if name == "dit_proj_w8a8_4096x3072x3072":
                # NEXT-1 on the tiled GEMM: any in-GEMM quantization needs the
                # rows' absmax first, i.e. a pass over x; this is the fastest
                # such pass (a plain streaming read of the 2*M*K bytes of x)
                fx = read_floor(2 * w.M * w.K, 2048, 512, sink, f"probe_read_x_{name}")
                e["x_read_floor"] = fx
                e["call_minus_kernel_us"] = round((t - tg) * 1e3, 3)
            if name == "dit_proj_w8a8_4096x3072x3072" and w.out == "bf16":
                # the gated residual epilogue, updating the residual stream in
                # place (4 samples of 1024 tokens: one gate row each)
                L = 1024
                pw.add_gate(L)
                tgd = measure(pw.gated, steps_x, 5, EXTRA_WARM_S, sink, name, "gated")["ms"]
                extra_b = 2 * w.M * w.N + 4 * (-(-w.M // L)) * w.N
                extra[name + "+gated_residual"] = {
                    "ms_per_call": round(tgd, 5), "gate_rows": L, "in_place": True,
                    "tops": round(w.ops / (tgd * 1e-3) / 1e12, 2),
                    "overhead_vs_plain_pct": round(100 * (tgd - t) / t, 2),
                    "gbs": round((algorithmic_bytes(w) + extra_b) / (tgd * 1e-3) / 1e9, 1),
                }
            extra[name] = e
            log(f"{name}: {t * 1e3:.2f} us/call, kernel {tg * 1e3:.2f} us "
                f"({e['kernel_tops']} TOPS, {gbs:.0f} GB/s per call)")
            del pw
            torch.cuda.empty_cache()
        del up_out
        peak_att = attention_peak_tops()
        for name, w in synth.ATTN_WORKLOADS.items():
            pa = PreparedAttention(w)
            pa.step(0)
            steps_a = max(3, steps // 4)
            t = measure(pa.step, steps_a, 5, EXTRA_WARM_S, sink, name, "call")["ms"]
            ta = measure(pa.attend, steps_a, 5, EXTRA_WARM_S, sink, name, "kernel")["ms"]
            extra[name] = {
                "ms_per_call": round(t, 5), "kernel_ms": round(ta, 5),
                "B": w.B, "H": w.H, "Lq": w.Lq, "Lk": w.Lk,
                "q_block": w.q_block, "k_block": w.k_block,
                "tops": round(w.ops / (t * 1e-3) / 1e12, 2),
                "kernel_tops": round(w.ops / (ta * 1e-3) / 1e12, 2),
                "mfma_peak_tops": round(peak_att, 1),
                "pct_mfma_peak": round(100 * w.ops / (ta * 1e-3) / 1e12 / peak_att, 2),
            }
            log(f"{name}: {t * 1e3:.1f} us/call, attention kernel {ta * 1e3:.1f} us "
                f"({extra[name]['kernel_tops']} TOPS, {extra[name]['pct_mfma_peak']}% of "
                f"{peak_att:.0f})")
            del pa
            torch.cuda.empty_cache()
        result["extra"] = extra

    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(wl)
        log(f"cpu oracle {wl.name}: {result['cpu_baseline']['value']} TOPS")
        if not args.quick:
            per = {}
            for name, w in synth.WORKLOADS.items():
                if name == synth.HEADLINE:
                    continue
                rows = 512 if w.M > 512 and w.fmt == "w4" or w.M > 4096 else None
                xb = None
                if name.startswith("dit_mlp_down_w4a8"):
                    xb = _oracle_up_output(synth, rows or 512)
                per[name] = cpu_oracle(w, rows=rows, budget_s=1.0, max_runs=5, x_bits=xb)
                log(f"cpu oracle {name}: {per[name]['value']} TOPS"
                    f"{' (extrapolated)' if per[name]['extrapolated'] else ''}")
            result["cpu_baseline"]["per_workload"] = per
    print(json.dumps(result), flush=True)
    return 0


def _oracle_up_output(synth, rows: int):
    """bf16 bits of the oracle's up-projection output on its first `rows`
    rows: the down projection's input on the CPU side."""
    import oracle

    up = next(w for n, w in synth.WORKLOADS.items() if n.startswith("dit_mlp_up_w4a8"))
    xb = synth.activations(up, rows=rows)
    _, gs, gb, q = oracle.quantize_w4(synth.weights(up))
    y = oracle.w4a8_linear_exact(xb, q, gs, gb, synth.bias(up))
    return oracle.round_bf16_bits(oracle.round_f32(y))


if __name__ == "__main__":
    sys.exit(main())
