"""GPU test of kq_w8a8_linear_noalloc, the entry point that allocates
nothing: through the C ABI, against kq_w8a8_linear (the same kernels on a
caller workspace) bit for bit and against the oracle's bars, on calls in a
row whose later shapes are smaller, on every route kind, and at the
scratch limit."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
import w8a8_gemm_dit_amd as kq
from tests.parity import check_bf16, check_f32, dev, dev_bf16, host, host_bf16_bits

pytestmark = pytest.mark.gpu

# (M, K, N, out): a GEMM shape, then smaller ones on other routes: split K
# (128 rows, K = 12288), the GEMV (10 rows), the fused GEMV (3 rows) and
# fused thin N (48 columns)
SEQUENCE = [(1000, 1024, 768, "bf16"), (300, 512, 512, "f32"), (128, 12288, 384, "bf16"),
            (10, 2048, 1000, "f32"), (3, 1024, 4096, "bf16"), (200, 1024, 48, "bf16")]


def _raw_call(x, wq, sw, b, y, dtype):
    M, K = x.shape
    N = wq.shape[0]
    return kq.lib().kq_w8a8_linear_noalloc(
        ctypes.c_void_p(x.data_ptr()), M, K, N, ctypes.c_void_p(wq.data_ptr()),
        ctypes.c_void_p(sw.data_ptr()), ctypes.c_void_p(b.data_ptr()),
        ctypes.c_void_p(y.data_ptr()), dtype,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_noalloc_matches_workspace_entry_point_on_calls_in_a_row():
    for i, (M, K, N, out) in enumerate(SEQUENCE):
        print(f"[noalloc] call {i}: M={M} K={K} N={N} {out}", flush=True)
        xb = synth.random_bf16((M, K), seed=900 + i, dist="student_t4")
        w = synth.random_f32((N, K), seed=950 + i, scale=0.02)
        b = synth.random_f32((N,), seed=990 + i, scale=0.1)
        q8, sw = oracle.quantize_w8(w)
        x, wq, swd, bd = dev_bf16(xb), dev(q8), dev(sw), dev(b)
        dt = torch.float32 if out == "f32" else torch.bfloat16
        code = kq.KQ_DTYPE_F32 if out == "f32" else kq.KQ_DTYPE_BF16
        y = torch.full((M, N), float("nan"), dtype=dt, device="cuda")
        assert _raw_call(x, wq, swd, bd, y, code) == kq.KQ_SUCCESS, kq.kq_last_error()
        ref = kq.kq_w8a8_linear(x, wq, swd, bd, out_dtype=dt)
        torch.cuda.synchronize()
        view = torch.int32 if out == "f32" else torch.int16
        assert torch.equal(y.view(view), ref.view(view)), (M, K, N)
        y64 = oracle.w8a8_linear_exact(xb, q8, sw, b)
        T = oracle.w8a8_magnitude(xb, q8, sw, b)
        if out == "f32":
            check_f32(host(y), y64, T, f"noalloc {M}x{K}x{N}")
        else:
            check_bf16(host_bf16_bits(y), y64, T, f"noalloc {M}x{K}x{N}")


def test_noalloc_at_and_over_the_scratch_limit():
    # the largest M with K = 4096 whose codes and scales fit the scratch
    K, N = 4096, 1024
    limit = kq.KQ_NOALLOC_SCRATCH_BYTES
    need = lambda m: kq.kq_workspace_bytes(m, N, K, kq.KQ_W8_PER_CHANNEL)  # noqa: E731
    lo, hi = 1, 1 << 16
    while hi - lo > 1:                      # the largest M that fits
        mid = (lo + hi) // 2
        lo, hi = (mid, hi) if need(mid) <= limit else (lo, mid)
    M = lo
    assert need(M) <= limit < need(M + 1)
    print(f"[noalloc] near the limit: M={M} K={K} N={N}", flush=True)
    xb = synth.random_bf16((M, K), seed=1)
    w = synth.random_f32((N, K), seed=2, scale=0.02)
    q8, sw = oracle.quantize_w8(w)
    x, wq, swd = dev_bf16(xb), dev(q8), dev(sw)
    y = kq.kq_w8a8_linear_noalloc(x, wq, swd, out_dtype=torch.bfloat16)
    ref = kq.kq_w8a8_linear(x, wq, swd, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), ref.view(torch.int16))
    rows = np.array([0, 1, M // 2, M - 1])
    check_bf16(host_bf16_bits(y)[rows], oracle.w8a8_linear_exact(xb[rows], q8, sw),
               oracle.w8a8_magnitude(xb[rows], q8, sw), "noalloc near the limit")
    # one more row no longer fits: rejected before anything runs
    M2 = M + 1
    assert kq.kq_workspace_bytes(M2, N, K, kq.KQ_W8_PER_CHANNEL) > limit
    x2 = torch.zeros((M2, K), dtype=torch.bfloat16, device="cuda")
    y2 = torch.zeros((M2, N), dtype=torch.bfloat16, device="cuda")
    st = _raw_call(x2, wq, swd, swd[:N], y2, kq.KQ_DTYPE_BF16)
    assert st == kq.KQ_ERR_UNSUPPORTED
    assert "needs" in kq.kq_last_error() and "scratch" in kq.kq_last_error()
    torch.cuda.synchronize()
    assert not y2.view(torch.int16).any()
