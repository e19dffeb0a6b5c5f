"""GPU parity of the entry points on pre-quantized activations
(kq_w8a8_gemm / kq_w4a8_gemm: codes, token scales and group sums from
kq_quantize_act) against the oracle, on every route they take: the GEMV
(M <= 32, or thin N, where the linears would take the fused kernel) and the
GEMM tiles (never split: these entry points take no workspace).

For int8 weights the result must equal the linear's bit for bit (same
codes, same exact sums, same epilogue expression); for int4 weights the
per-group products must, and the outputs meet the oracle's bars."""
import numpy as np
import pytest
import torch

import oracle
import synth
import w8a8_gemm_dit_amd as kq
from tests.parity import check_bf16, check_f32, dev, dev_bf16, host, host_bf16_bits

pytestmark = pytest.mark.gpu


def setup_module(module):
    print(f"[prequant] device: {torch.cuda.get_device_name(0)}", flush=True)
    assert kq.kq_is_available(), "libkq reports no gfx950 device"


# (M, K, N, route the linear takes): a few rows (the linear's GEMV quantizes
# x itself; these entry points take the plain GEMV), 16 rows, thin N (fused
# for the linear), GEMM with ragged tiles, a shape the linear would split
SHAPES = [(3, 512, 200, "fused"), (16, 512, 200, "gemv"), (300, 640, 48, "fused"),
          (257, 320, 129, "gemm"),
          (64, 1024, 1000, "gemm"), (128, 12288, 256, "gemm")]


def _operands(M, K, N, seed):
    xb = synth.random_bf16((M, K), seed=seed, dist="student_t4")
    w = synth.random_f32((N, K), seed=seed + 1, scale=0.02)
    b = synth.random_f32((N,), seed=seed + 2, scale=0.1)
    return xb, w, b


@pytest.mark.parametrize("M,K,N,route", SHAPES)
def test_w8a8_gemm_matches_linear_and_oracle(M, K, N, route, kq_env):
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_SPLIT=None, KQ_FUSE=None)
    assert kq.kq_route(M, N, K, kq.KQ_W8_PER_CHANNEL)["kind"] == route
    print(f"[prequant] w8 {M}x{K}x{N}", flush=True)
    xb, w, b = _operands(M, K, N, seed=M + K + N)
    q8, sw = oracle.quantize_w8(w)
    x = dev_bf16(xb)
    a, sx, _ = kq.kq_quantize_act(x)
    args = (a, sx, dev(q8), dev(sw))
    acc = kq.kq_w8a8_gemm(*args, out_dtype=torch.int32)
    yf = kq.kq_w8a8_gemm(*args, dev(b), out_dtype=torch.float32)
    yb = kq.kq_w8a8_gemm(*args, dev(b), out_dtype=torch.bfloat16)
    lf = kq.kq_w8a8_linear(x, dev(q8), dev(sw), dev(b), out_dtype=torch.float32)
    lb = kq.kq_w8a8_linear(x, dev(q8), dev(sw), dev(b), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    a_ref, _, _ = oracle.quantize_act(xb)
    assert np.array_equal(host(acc), oracle.w8a8_acc(a_ref, q8))
    assert np.array_equal(host(yf).view(np.uint32), host(lf).view(np.uint32))
    assert np.array_equal(host_bf16_bits(yb), host_bf16_bits(lb))
    y64 = oracle.w8a8_linear_exact(xb, q8, sw, b)
    T = oracle.w8a8_magnitude(xb, q8, sw, b)
    check_f32(host(yf), y64, T, f"w8 gemm {M}x{K}x{N}")
    check_bf16(host_bf16_bits(yb), y64, T, f"w8 gemm {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N,route", SHAPES)
def test_w4a8_gemm_matches_oracle(M, K, N, route, kq_env):
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_SPLIT=None, KQ_FUSE=None)
    print(f"[prequant] w4 {M}x{K}x{N}", flush=True)
    xb, w, b = _operands(M, K, N, seed=2 * M + K + N)
    p, gs, gb, q = oracle.quantize_w4(w)
    x = dev_bf16(xb)
    a, sx, gsum = kq.kq_quantize_act(x, group_sums=True)
    args = (a, sx, gsum, dev(p), dev(gs), dev(gb))
    P = kq.kq_w4a8_gemm(*args, out_dtype=torch.int32)
    yf = kq.kq_w4a8_gemm(*args, dev(b), out_dtype=torch.float32)
    yb = kq.kq_w4a8_gemm(*args, dev(b), out_dtype=torch.bfloat16)
    PL = kq.kq_w4a8_linear(x, dev(p), dev(gs), dev(gb), out_dtype=torch.int32)
    torch.cuda.synchronize()
    a_ref, _, _ = oracle.quantize_act(xb)
    P_ref = oracle.w4a8_group_acc(a_ref, q)
    assert np.array_equal(host(P), P_ref)
    assert np.array_equal(host(PL), P_ref)
    y64 = oracle.w4a8_linear_exact(xb, q, gs, gb, b)
    T = oracle.w4a8_magnitude(xb, q, gs, gb, b)
    check_f32(host(yf), y64, T, f"w4 gemm {M}x{K}x{N}")
    check_bf16(host_bf16_bits(yb), y64, T, f"w4 gemm {M}x{K}x{N}")


def test_prequantized_errors():
    """Missing scales or group sums are rejected before any launch."""
    a = torch.zeros((4, 128), dtype=torch.int8, device="cuda")
    wq = torch.zeros((16, 128), dtype=torch.int8, device="cuda")
    sw = torch.ones((16,), dtype=torch.float32, device="cuda")
    y = torch.empty((4, 16), dtype=torch.bfloat16, device="cuda")
    st = kq.lib().kq_w8a8_gemm(kq._ptr(a), None, 4, 128, 16, kq._ptr(wq), kq._ptr(sw), None,
                              kq._ptr(y), kq.KQ_DTYPE_BF16, kq._stream())
    assert st != 0 and "null scale or group-sum pointer" in kq.kq_last_error()
    with pytest.raises(ValueError, match=r"\[kq_w8a8_gemm\] K=100 must be a positive multiple of 64"):
        kq.kq_w8a8_gemm(torch.zeros((4, 100), dtype=torch.int8, device="cuda"),
                        torch.ones((4,), dtype=torch.float32, device="cuda"),
                        torch.zeros((16, 100), dtype=torch.int8, device="cuda"), sw)


# ------------------------------------------------------- split code order
# KQ_CODES_SPLIT8: bytes 8j + i of a row hold the code of k = 8j + SPLIT8[i]
SPLIT8 = np.array([0, 2, 4, 6, 1, 3, 5, 7])


def _split8(a):
    M, K = a.shape
    return a.reshape(M, K // 8, 8)[:, :, SPLIT8].reshape(M, K)


def test_split8_permutation_is_the_header_one():
    # the natural codes 0..15 of one row come out as 0 2 4 6 1 3 5 7 8 10 ...
    assert _split8(np.arange(16).reshape(1, 16)).tolist() == [
        [0, 2, 4, 6, 1, 3, 5, 7, 8, 10, 12, 14, 9, 11, 13, 15]]


@pytest.mark.parametrize("M,K", [(1, 64), (7, 520), (16, 5120), (300, 4096), (64, 12288),
                                 (3, 24)])
def test_quantize_act_split_order(M, K):
    """Split-order codes are the natural codes permuted within each run of 8;
    scales and group sums are unchanged, bit for bit."""
    print(f"[prequant] split quantize {M}x{K}", flush=True)
    xb = synth.random_bf16((M, K), seed=M * 7 + K, dist="student_t4")
    a_ref, s_ref, g_ref = oracle.quantize_act(xb)
    sums = K % 64 == 0
    a, sx, gs = kq.kq_quantize_act_ordered(dev_bf16(xb), kq.KQ_CODES_SPLIT8, group_sums=sums)
    torch.cuda.synchronize()
    assert np.array_equal(host(a), _split8(a_ref))
    assert np.array_equal(host(sx).view(np.uint32), s_ref.view(np.uint32))
    if sums:
        assert np.array_equal(host(gs), g_ref)


@pytest.mark.parametrize("tile", [None, "128x256", "128x128", "64x128"])
@pytest.mark.parametrize("M,K,N", [(1, 512, 200), (16, 512, 200), (257, 320, 129),
                                   (130, 2048, 200), (96, 2112, 272), (128, 12288, 256)])
def test_w4a8_gemm_split_order(M, K, N, tile, kq_env):
    """The int4 GEMM on split-order codes: per-group products bit-exact
    against the oracle, outputs bit-identical to the same tile on the
    natural codes and within the oracle's bars."""
    kq_env(KQ_FORCE_ROUTE="gemm", KQ_TILE=tile, KQ_SPLIT=None, KQ_FUSE=None)
    print(f"[prequant] split w4 gemm {M}x{K}x{N} tile {tile}", flush=True)
    xb, w, b = _operands(M, K, N, seed=3 * M + K + 5 * N)
    p, gs, gb, q = oracle.quantize_w4(w)
    x = dev_bf16(xb)
    an, sx, gsum = kq.kq_quantize_act(x, group_sums=True)
    asp, sx2, gsum2 = kq.kq_quantize_act_ordered(x, kq.KQ_CODES_SPLIT8, group_sums=True)
    W = (dev(p), dev(gs), dev(gb))
    S = kq.KQ_CODES_SPLIT8
    P = kq.kq_w4a8_gemm_ordered(asp, sx2, gsum2, *W, S, out_dtype=torch.int32)
    yf = kq.kq_w4a8_gemm_ordered(asp, sx2, gsum2, *W, S, dev(b), out_dtype=torch.float32)
    yb = kq.kq_w4a8_gemm_ordered(asp, sx2, gsum2, *W, S, dev(b), out_dtype=torch.bfloat16)
    nf = kq.kq_w4a8_gemm(an, sx, gsum, *W, dev(b), out_dtype=torch.float32)
    nb = kq.kq_w4a8_gemm(an, sx, gsum, *W, dev(b), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    a_ref, _, _ = oracle.quantize_act(xb)
    assert np.array_equal(host(P), oracle.w4a8_group_acc(a_ref, q))
    assert np.array_equal(host(yf).view(np.uint32), host(nf).view(np.uint32))
    assert np.array_equal(host_bf16_bits(yb), host_bf16_bits(nb))
    y64 = oracle.w4a8_linear_exact(xb, q, gs, gb, b)
    T = oracle.w4a8_magnitude(xb, q, gs, gb, b)
    check_f32(host(yf), y64, T, f"split w4 gemm {M}x{K}x{N}")
    check_bf16(host_bf16_bits(yb), y64, T, f"split w4 gemm {M}x{K}x{N}")


def test_split_order_small_m_takes_the_gemm(kq_env):
    """Without a forced route, split-order codes at M <= 16 (where natural
    codes take the GEMV) still go through the tiled GEMM."""
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_SPLIT=None, KQ_FUSE=None)
    M, K, N = 4, 1024, 96
    xb, w, b = _operands(M, K, N, seed=77)
    p, gs, gb, q = oracle.quantize_w4(w)
    asp, sx, gsum = kq.kq_quantize_act_ordered(dev_bf16(xb), kq.KQ_CODES_SPLIT8, group_sums=True)
    P = kq.kq_w4a8_gemm_ordered(asp, sx, gsum, dev(p), dev(gs), dev(gb), kq.KQ_CODES_SPLIT8,
                                out_dtype=torch.int32)
    torch.cuda.synchronize()
    a_ref, _, _ = oracle.quantize_act(xb)
    assert np.array_equal(host(P), oracle.w4a8_group_acc(a_ref, q))
