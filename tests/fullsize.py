"""Oracle results of the full-size benchmark workloads, by blocks of rows,
for the GPU parity tests (test infrastructure: calls only oracle/ and
synth/).

Quantization is per row, so a block of rows of a linear is the linear of
those rows alone.  The int4 oracle takes tens of seconds per thousand rows
at the MLP shapes (one numpy pass per 64-group over the whole output), so
blocks are computed in parallel worker processes (spawned: they never
touch the GPU).  The MLP down projection's input is the oracle's own up
projection output rounded to bf16, row for row (the two linears of a DiT
MLP with nothing named in between).
"""
from __future__ import annotations

import concurrent.futures as cf
import functools
import multiprocessing as mp

import numpy as np

UP = "dit_mlp_up_w4a8_2048x4096x12288"
DOWN = "dit_mlp_down_w4a8_2048x12288x4096"


@functools.lru_cache(maxsize=4)
def quantized_weights(name: str):
    """The oracle's quantized weights of a workload (int8: (q8, sw);
    int4: (packed, gs, gb, q))."""
    import oracle
    import synth

    wl = synth.WORKLOADS[name]
    w = synth.weights(wl)
    return oracle.quantize_w8(w) if wl.fmt == "w8" else oracle.quantize_w4(w)


def activations(name: str, r0: int, r1: int) -> np.ndarray:
    """bf16 bits of rows [r0, r1) of the workload's input."""
    import oracle
    import synth

    if name == DOWN:
        up = synth.WORKLOADS[UP]
        _, gs, gb, q = quantized_weights(UP)
        xu = synth.activations(up, rows=r1)[r0:r1]
        yu = oracle.w4a8_linear_exact(xu, q, gs, gb, synth.bias(up))
        return oracle.round_bf16_bits(oracle.round_f32(yu))
    return synth.activations(synth.WORKLOADS[name], rows=r1)[r0:r1]


def block(name: str, r0: int, r1: int):
    """(x bits, y64, T) of rows [r0, r1): the input rows, the exact linear
    and its term magnitude."""
    import oracle
    import synth

    wl = synth.WORKLOADS[name]
    xb = activations(name, r0, r1)
    b = synth.bias(wl)
    if wl.fmt == "w8":
        q8, sw = quantized_weights(name)
        return (xb, oracle.w8a8_linear_exact(xb, q8, sw, b),
                oracle.w8a8_magnitude(xb, q8, sw, b))
    _, gs, gb, q = quantized_weights(name)
    return (xb, oracle.w4a8_linear_exact(xb, q, gs, gb, b),
            oracle.w4a8_magnitude(xb, q, gs, gb, b))


def _worker_init():
    # one BLAS thread per worker: the workers already use every core
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def blocks(name: str, rows: int, block_rows: int, workers: int):
    """Yield (r0, r1, x bits, y64, T) over the first `rows` rows; int4
    workloads in `workers` spawned processes, int8 ones in this process
    (BLAS-bound)."""
    import synth

    M = synth.WORKLOADS[name].M
    edges = [(r, min(M, r + block_rows)) for r in range(0, min(rows, M), block_rows)]
    if synth.WORKLOADS[name].fmt == "w8" or workers <= 1:
        for r0, r1 in edges:
            yield (r0, r1, *block(name, r0, r1))
        return
    ctx = mp.get_context("spawn")
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=ctx,
                                initializer=_worker_init) as ex:
        futs = [(r0, r1, ex.submit(block, name, r0, r1)) for r0, r1 in edges]
        for r0, r1, f in futs:
            yield (r0, r1, *f.result())
