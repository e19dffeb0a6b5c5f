"""GPU parity at the limits of the linears' shapes: the longest K the
int32 accumulator admits (65536, MLX pull request 4722, "Selector rules":
K/64 <= 1024) with every code at +-127, so |acc| reaches 65536*127*127 =
1,057,030,144 (below 2^31); the smallest shapes (K = 64, N = 1, M = 1).
int32 accumulators and per-group products bit-exact; outputs within the
oracle's bars."""
import numpy as np
import pytest
import torch

import oracle
import synth
import w8a8_gemm_dit_amd as kq
from tests.parity import check_f32, dev, dev_bf16, host

pytestmark = pytest.mark.gpu


def setup_module(module):
    print(f"[limits] device: {torch.cuda.get_device_name(0)}", flush=True)
    assert kq.kq_is_available(), "libkq reports no gfx950 device"


def _saturating(M, K, N, seed):
    """x rows of +-1 (amax 1: codes +-127) and weight rows of +-0.02 (codes
    +-127); row m of x takes the signs of weight row m % N, so those dot
    products reach the full +-K*127*127, the others mix signs."""
    rng = np.random.default_rng(seed)
    sw_sign = np.where(rng.random((N, K)) < 0.5, -1.0, 1.0).astype(np.float32)
    w = sw_sign * np.float32(0.02)
    xs = np.where(rng.random((M, K)) < 0.5, -1.0, 1.0).astype(np.float32)
    for m in range(0, M, 3):
        xs[m] = sw_sign[m % N]
    return synth.to_bf16_bits(xs), w


@pytest.mark.parametrize("split", [None, "1", "4", "16"])
@pytest.mark.parametrize("M,N", [(64, 64), (17, 40)])
def test_w8a8_longest_k_accumulators(M, N, split, kq_env):
    K = 65536
    kq_env(KQ_FORCE_ROUTE="gemm", KQ_TILE=None, KQ_SPLIT=split)
    xb, w = _saturating(M, K, N, seed=M + N)
    q8, sw = oracle.quantize_w8(w)
    a, sx, _ = oracle.quantize_act(xb)
    ref = oracle.w8a8_acc(a, q8)
    assert np.abs(ref).max() == K * 127 * 127
    print(f"[limits] w8a8 K={K} {M}x{N} split={split}", flush=True)
    acc = kq.kq_w8a8_linear(dev_bf16(xb), dev(q8), dev(sw), out_dtype=torch.int32)
    torch.cuda.synchronize()
    assert np.array_equal(host(acc), ref)
    y = kq.kq_w8a8_linear(dev_bf16(xb), dev(q8), dev(sw), out_dtype=torch.float32)
    torch.cuda.synchronize()
    y64 = oracle.w8a8_linear_exact(xb, q8, sw, None)
    check_f32(host(y), y64, oracle.w8a8_magnitude(xb, q8, sw, None), f"w8a8 K={K}")


@pytest.mark.parametrize("split", [None, "1", "5"])
def test_w4a8_longest_k(split, kq_env):
    M, K, N = 33, 65536, 48
    kq_env(KQ_FORCE_ROUTE="gemm", KQ_TILE=None, KQ_SPLIT=split)
    xb, w = _saturating(M, K, N, seed=5)
    p, gs, gb, q = oracle.quantize_w4(w)
    a, _, _ = oracle.quantize_act(xb)
    print(f"[limits] w4a8 K={K} split={split}", flush=True)
    P = kq.kq_w4a8_linear(dev_bf16(xb), dev(p), dev(gs), dev(gb), out_dtype=torch.int32)
    torch.cuda.synchronize()
    assert np.array_equal(host(P), oracle.w4a8_group_acc(a, q))
    y = kq.kq_w4a8_linear(dev_bf16(xb), dev(p), dev(gs), dev(gb), out_dtype=torch.float32)
    torch.cuda.synchronize()
    y64 = oracle.w4a8_linear_exact(xb, q, gs, gb, None)
    check_f32(host(y), y64, oracle.w4a8_magnitude(xb, q, gs, gb, None), f"w4a8 K={K}")


@pytest.mark.parametrize("fmt", ["w8", "w4"])
@pytest.mark.parametrize("route", [None, "gemm", "gemv"])
def test_smallest_shape(fmt, route, kq_env):
    M, K, N = 1, 64, 1
    kq_env(KQ_FORCE_ROUTE=route, KQ_TILE=None, KQ_SPLIT=None)
    xb = synth.random_bf16((M, K), seed=3, dist="student_t4")
    w = synth.random_f32((N, K), seed=4, scale=0.02)
    b = synth.random_f32((N,), seed=5, scale=0.1)
    print(f"[limits] smallest {fmt} route={route}", flush=True)
    if fmt == "w8":
        q8, sw = oracle.quantize_w8(w)
        a, _, _ = oracle.quantize_act(xb)
        acc = kq.kq_w8a8_linear(dev_bf16(xb), dev(q8), dev(sw), out_dtype=torch.int32)
        y = kq.kq_w8a8_linear(dev_bf16(xb), dev(q8), dev(sw), dev(b), out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert np.array_equal(host(acc), oracle.w8a8_acc(a, q8))
        check_f32(host(y), oracle.w8a8_linear_exact(xb, q8, sw, b),
                  oracle.w8a8_magnitude(xb, q8, sw, b), "w8a8 1x64x1")
    else:
        p, gs, gb, q = oracle.quantize_w4(w)
        a, _, _ = oracle.quantize_act(xb)
        P = kq.kq_w4a8_linear(dev_bf16(xb), dev(p), dev(gs), dev(gb), out_dtype=torch.int32)
        y = kq.kq_w4a8_linear(dev_bf16(xb), dev(p), dev(gs), dev(gb), dev(b), out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert np.array_equal(host(P), oracle.w4a8_group_acc(a, q))
        check_f32(host(y), oracle.w4a8_linear_exact(xb, q, gs, gb, b),
                  oracle.w4a8_magnitude(xb, q, gs, gb, b), "w4a8 1x64x1")
