"""GPU parity of the gated residual epilogue (kq_linear_gated):
out = residual + gate[m // gate_rows] * linear(x), against the oracle's
fp64 gated_residual_exact, on every route (GEMM tiles, GEMV, fused thin N).

Tolerance: the plain linears' bars with the term magnitude widened to
|residual| + |gate| * T (oracle.gated_magnitude), the scale of an fp32
evaluation's rounding error once the fma adds the residual."""
import numpy as np
import pytest
import torch

import oracle
import synth
import w8a8_gemm_dit_amd as kq
from tests.parity import check_bf16, check_f32, dev, dev_bf16, host, host_bf16_bits

pytestmark = pytest.mark.gpu


def setup_module(module):
    print(f"[gated] device: {torch.cuda.get_device_name(0)}", flush=True)
    assert kq.kq_is_available(), "libkq reports no gfx950 device"


def _operands(fmt, M, K, N, seed):
    xb = synth.random_bf16((M, K), seed=seed)
    w = synth.random_f32((N, K), seed=seed + 1, scale=0.02)
    b = synth.random_f32((N,), seed=seed + 2, scale=0.1)
    if fmt == "w8":
        q8, sw = oracle.quantize_w8(w)
        y64 = oracle.w8a8_linear_exact(xb, q8, sw, b)
        T = oracle.w8a8_magnitude(xb, q8, sw, b)
        args = (kq.KQ_W8_PER_CHANNEL, dev_bf16(xb), dev(q8), dev(sw), None)
    else:
        p, gs, gb, q = oracle.quantize_w4(w)
        y64 = oracle.w4a8_linear_exact(xb, q, gs, gb, b)
        T = oracle.w4a8_magnitude(xb, q, gs, gb, b)
        args = (kq.KQ_W4_AFFINE_G64, dev_bf16(xb), dev(p), dev(gs), dev(gb))
    return args, dev(b), y64, T


def _residual_gate(M, N, seed, with_residual, gate_rows):
    r = synth.random_bf16((M, N), seed=seed + 3) if with_residual else None
    g = None
    if gate_rows:
        g = synth.random_f32((-(-M // gate_rows), N), seed=seed + 4, scale=0.5)
    return r, g


def _check(y, out, y64, T, r, g, L, what):
    ref = oracle.gated_residual_exact(y64, r, g, L)
    Tg = oracle.gated_magnitude(T, r, g, L)
    torch.cuda.synchronize()
    if out == "f32":
        check_f32(host(y), ref, Tg, what)
    else:
        check_bf16(host_bf16_bits(y), ref, Tg, what)


# (M, K, N, route): GEMM with whole and ragged tiles, GEMV, fused thin N
SHAPES = [(300, 640, 200, "gemm"), (513, 320, 260, "gemm"), (256, 512, 256, "gemm"),
          (5, 1024, 200, "gemv"), (16, 256, 130, "gemv"), (300, 512, 48, "fused"),
          (3, 1024, 200, "fused"),
          (96, 2112, 272, "gemm")]
# (residual?, gate_rows or 0 for no gate)
VARIANTS = [(True, 1), (True, 128), (False, 1), (True, 0), (True, 7)]


@pytest.mark.parametrize("res,L", VARIANTS)
@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", ["w8", "w4"])
@pytest.mark.parametrize("M,K,N,route", SHAPES)
def test_gated_matches_oracle(M, K, N, route, fmt, out, res, L, kq_env):
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None)
    assert kq.kq_route(M, N, K, kq.KQ_W8_PER_CHANNEL)["kind"] == route
    seed = 11 * M + K + 3 * N
    args, b, y64, T = _operands(fmt, M, K, N, seed)
    r, g = _residual_gate(M, N, seed, res, L)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    y = kq.kq_linear_gated(*args, bias=b, residual=None if r is None else dev_bf16(r),
                           gate=None if g is None else dev(g), gate_rows=max(L, 1), out_dtype=dt)
    _check(y, out, y64, T, r, g, max(L, 1), f"gated {fmt} {out} {M}x{K}x{N} res={res} L={L}")


@pytest.mark.parametrize("tile", ["256x256", "256x256w8", "256x192", "256x128", "128x128", "64x64"])
@pytest.mark.parametrize("M,K,N", [(300, 448, 200), (257, 128, 129), (512, 256, 512)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gated_w8_every_tile(M, K, N, tile, out, kq_env):
    """Each W8A8 tile, whole tiles (staged bf16 epilogue) and ragged ones
    (odd N: the per-element path)."""
    kq_env(KQ_FORCE_ROUTE="gemm", KQ_TILE=tile)
    seed = M + 5 * K + N
    args, b, y64, T = _operands("w8", M, K, N, seed)
    r, g = _residual_gate(M, N, seed, True, 64)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    y = kq.kq_linear_gated(*args, bias=b, residual=dev_bf16(r), gate=dev(g), gate_rows=64,
                           out_dtype=dt)
    _check(y, out, y64, T, r, g, 64, f"gated w8 tile {tile} {M}x{K}x{N}")


@pytest.mark.parametrize("tile", ["128x256", "128x128", "64x128"])
@pytest.mark.parametrize("M,K,N", [(300, 448, 200), (257, 128, 129), (256, 1024, 512)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_gated_w4_every_tile(M, K, N, tile, out, kq_env):
    kq_env(KQ_FORCE_ROUTE="gemm", KQ_TILE=tile)
    seed = 2 * M + K + N
    args, b, y64, T = _operands("w4", M, K, N, seed)
    r, g = _residual_gate(M, N, seed, True, 100)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    y = kq.kq_linear_gated(*args, bias=b, residual=dev_bf16(r), gate=dev(g), gate_rows=100,
                           out_dtype=dt)
    _check(y, out, y64, T, r, g, 100, f"gated w4 tile {tile} {M}x{K}x{N}")


@pytest.mark.parametrize("fmt", ["w8", "w4"])
@pytest.mark.parametrize("M,K,N,route", [(512, 512, 512, "gemm"), (300, 320, 260, "gemm"),
                                          (7, 512, 200, "gemv"), (300, 256, 64, "fused")])
def test_gated_in_place(M, K, N, route, fmt, kq_env):
    """The residual stream updated in place (out is the residual tensor),
    a DiT block's x = x + gate * linear(...)."""
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None)
    assert kq.kq_route(M, N, K, kq.KQ_W8_PER_CHANNEL)["kind"] == route
    seed = M + K + 7 * N
    args, b, y64, T = _operands(fmt, M, K, N, seed)
    r, g = _residual_gate(M, N, seed, True, 128)
    stream = dev_bf16(r)
    ptr = stream.data_ptr()
    y = kq.kq_linear_gated(*args, bias=b, residual=stream, gate=dev(g), gate_rows=128,
                           out_dtype=torch.bfloat16, out=stream)
    assert y.data_ptr() == ptr
    _check(y, "bf16", y64, T, r, g, 128, f"in-place {fmt} {M}x{K}x{N}")


@pytest.mark.parametrize("fmt", ["w8", "w4"])
@pytest.mark.parametrize("M,K,N", [(300, 640, 200), (5, 1024, 200), (300, 512, 48)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_gated_without_terms_is_the_plain_linear(M, K, N, fmt, out, kq_env):
    """residual = gate = NULL reproduces the plain linear bit for bit, and a
    zero residual with a unit gate gives the same numbers."""
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None)
    args, b, _, _ = _operands(fmt, M, K, N, seed=M + K + N)
    fmtc, x, wq, sc, gb = args
    if fmt == "w8":
        plain = kq.kq_w8a8_linear(x, wq, sc, b, out_dtype=out)
    else:
        plain = kq.kq_w4a8_linear(x, wq, sc, gb, bias=b, out_dtype=out)
    none = kq.kq_linear_gated(*args, bias=b, out_dtype=out)
    ones = kq.kq_linear_gated(*args, bias=b, residual=torch.zeros((M, N), dtype=torch.bfloat16,
                                                                  device="cuda"),
                              gate=torch.ones((1, N), dtype=torch.float32, device="cuda"),
                              gate_rows=M, out_dtype=out)
    torch.cuda.synchronize()
    assert torch.equal(plain.view(torch.int16) if out == torch.bfloat16 else plain.view(torch.int32),
                       none.view(torch.int16) if out == torch.bfloat16 else none.view(torch.int32))
    # 1 * v + 0 == v exactly in fp32 (a -0 result becomes +0; compare values)
    assert torch.equal(plain.float(), ones.float())


def test_gated_zero_gate_returns_the_residual(kq_env):
    """gate = 0 leaves exactly the residual (bf16 in, bf16 out)."""
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None)
    M, K, N = 300, 256, 200
    args, b, _, _ = _operands("w8", M, K, N, seed=77)
    r = synth.random_bf16((M, N), seed=78)
    g = np.zeros((3, N), np.float32)
    y = kq.kq_linear_gated(*args, bias=b, residual=dev_bf16(r), gate=dev(g), gate_rows=100)
    torch.cuda.synchronize()
    # values, not bits: r + (+-0) may turn a -0 residual into +0
    got = oracle.bf16_bits_to_f32(host_bf16_bits(y))
    assert np.array_equal(got, oracle.bf16_bits_to_f32(r))
