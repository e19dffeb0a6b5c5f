"""GPU parity of the split-K GEMM (int8 weights): each K slice writes exact
int32 partial sums and the fold applies the unsplit epilogue expression, so
every output is bit-identical to the unsplit product's; against the oracle
the usual bars apply (int32 bit-exact, fp32 1e-5 of the term magnitude,
bf16 1 ulp)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import w8a8_gemm_dit_amd as kq
from tests.parity import check_bf16, check_f32, dev, dev_bf16, host, host_bf16_bits

pytestmark = pytest.mark.gpu


def setup_module(module):
    print(f"[splitk] device: {torch.cuda.get_device_name(0)}", flush=True)
    assert kq.kq_is_available(), "libkq reports no gfx950 device"


def _problem(M, K, N, seed):
    xb = synth.random_bf16((M, K), seed=seed)
    w = synth.random_f32((N, K), seed=seed + 1, scale=0.02)
    b = synth.random_f32((N,), seed=seed + 2, scale=0.1)
    q8, sw = oracle.quantize_w8(w)
    return xb, q8, sw, b


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu()


@pytest.mark.parametrize("M,K,N", [(128, 12288, 3072), (64, 4096, 4096), (200, 8192, 1000)])
def test_automatic_split_matches_unsplit_bitwise(M, K, N, kq_env):
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_SPLIT=None)
    assert kq.kq_route(M, N, K, kq.KQ_W8_PER_CHANNEL)["splits"] > 1
    xb, q8, sw, b = _problem(M, K, N, seed=M + N)
    args = (dev_bf16(xb), dev(q8), dev(sw), dev(b))
    outs = {}
    for split in (None, "1"):
        kq_env(KQ_SPLIT=split)
        outs[split] = [kq.kq_w8a8_linear(*args, out_dtype=dt) for dt in (torch.float32, torch.bfloat16)]
        outs[split].append(kq.kq_w8a8_linear(*args[:3], out_dtype=torch.int32))
    torch.cuda.synchronize()
    for a, c in zip(outs[None], outs["1"]):
        assert torch.equal(_bits(a), _bits(c))
    a, _, _ = oracle.quantize_act(xb)
    assert np.array_equal(host(outs[None][2]), oracle.w8a8_acc(a, q8))
    y64 = oracle.w8a8_linear_exact(xb, q8, sw, b)
    T = oracle.w8a8_magnitude(xb, q8, sw, b)
    check_f32(host(outs[None][0]), y64, T, f"split {M}x{K}x{N} f32")
    check_bf16(host_bf16_bits(outs[None][1]), y64, T, f"split {M}x{K}x{N} bf16")


@pytest.mark.parametrize("tile", ["256x256", "256x256w8", "256x192", "256x128", "128x128", "64x64"])
@pytest.mark.parametrize("split", ["2", "3", "7", "16"])
@pytest.mark.parametrize("M,K,N", [(257, 1088, 200), (100, 2304, 129)])
def test_forced_splits_every_tile(M, K, N, tile, split, kq_env):
    """Ragged M and N, slice counts that leave a short last slice (and a
    last slice whose step count is not a multiple of 4)."""
    kq_env(KQ_FORCE_ROUTE="gemm", KQ_TILE=tile, KQ_SPLIT=split)
    r = kq.kq_route(M, N, K, kq.KQ_W8_PER_CHANNEL)
    assert r["splits"] > 1
    xb, q8, sw, b = _problem(M, K, N, seed=3 * M + N + int(split))
    args = (dev_bf16(xb), dev(q8), dev(sw), dev(b))
    ys = [kq.kq_w8a8_linear(*args, out_dtype=dt) for dt in (torch.float32, torch.bfloat16)]
    acc = kq.kq_w8a8_linear(*args[:3], out_dtype=torch.int32)
    kq_env(KQ_SPLIT="1")
    ref = [kq.kq_w8a8_linear(*args, out_dtype=dt) for dt in (torch.float32, torch.bfloat16)]
    torch.cuda.synchronize()
    for a, c in zip(ys, ref):
        assert torch.equal(_bits(a), _bits(c)), (tile, split)
    a, _, _ = oracle.quantize_act(xb)
    assert np.array_equal(host(acc), oracle.w8a8_acc(a, q8))
    y64 = oracle.w8a8_linear_exact(xb, q8, sw, b)
    check_f32(host(ys[0]), y64, oracle.w8a8_magnitude(xb, q8, sw, b), f"{tile} split {split}")


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_split_with_gated_epilogue(out, kq_env):
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_SPLIT=None)
    M, K, N = 128, 12288, 3072
    assert kq.kq_route(M, N, K, kq.KQ_W8_PER_CHANNEL)["splits"] > 1
    xb, q8, sw, b = _problem(M, K, N, seed=11)
    r = synth.random_bf16((M, N), seed=12)
    g = synth.random_f32((2, N), seed=13, scale=0.5)
    args = (kq.KQ_W8_PER_CHANNEL, dev_bf16(xb), dev(q8), dev(sw), None)
    y = kq.kq_linear_gated(*args, bias=dev(b), residual=dev_bf16(r), gate=dev(g), gate_rows=64,
                           out_dtype=out)
    kq_env(KQ_SPLIT="1")
    y1 = kq.kq_linear_gated(*args, bias=dev(b), residual=dev_bf16(r), gate=dev(g), gate_rows=64,
                            out_dtype=out)
    torch.cuda.synchronize()
    assert torch.equal(_bits(y), _bits(y1))
    ref = oracle.gated_residual_exact(oracle.w8a8_linear_exact(xb, q8, sw, b), r, g, 64)
    T = oracle.gated_magnitude(oracle.w8a8_magnitude(xb, q8, sw, b), r, g, 64)
    if out == torch.float32:
        check_f32(host(y), ref, T, "split gated f32")
    else:
        check_bf16(host_bf16_bits(y), ref, T, "split gated bf16")


def test_workspace_too_small_for_the_partials_is_an_error(kq_env):
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_SPLIT=None)
    M, K, N = 128, 12288, 3072
    xb, q8, sw, b = _problem(M, K, N, seed=21)
    need = kq.kq_workspace_bytes(M, N, K, kq.KQ_W8_PER_CHANNEL)
    small = torch.empty((need - 256,), dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="workspace"):
        kq.kq_w8a8_linear(dev_bf16(xb), dev(q8), dev(sw), dev(b), workspace=small)


# ---------------------------------------------------------------- int4
def _problem4(M, K, N, seed):
    xb = synth.random_bf16((M, K), seed=seed)
    w = synth.random_f32((N, K), seed=seed + 1, scale=0.02)
    b = synth.random_f32((N,), seed=seed + 2, scale=0.1)
    p, gs, gb, q = oracle.quantize_w4(w)
    return xb, p, gs, gb, q, b


def _check4(xb, q, gs, gb, b, yf, yb, P, what):
    a, _, _ = oracle.quantize_act(xb)
    assert np.array_equal(host(P), oracle.w4a8_group_acc(a, q)), what
    y64 = oracle.w4a8_linear_exact(xb, q, gs, gb, b)
    T = oracle.w4a8_magnitude(xb, q, gs, gb, b)
    check_f32(host(yf), y64, T, what + " f32")
    check_bf16(host_bf16_bits(yb), y64, T, what + " bf16")


@pytest.mark.parametrize("M,K,N", [(128, 12288, 3072), (64, 4096, 4096), (300, 2112, 640)])
def test_int4_automatic_split(M, K, N, kq_env):
    """fp32 slice sums folded in slice order: within the oracle's bars (not
    bitwise the unsplit order), per-group products bit-exact."""
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_SPLIT=None)
    assert kq.kq_route(M, N, K, kq.KQ_W4_AFFINE_G64)["splits"] > 1
    xb, p, gs, gb, q, b = _problem4(M, K, N, seed=M + K)
    args = (dev_bf16(xb), dev(p), dev(gs), dev(gb))
    yf = kq.kq_w4a8_linear(*args, bias=dev(b), out_dtype=torch.float32)
    yb = kq.kq_w4a8_linear(*args, bias=dev(b), out_dtype=torch.bfloat16)
    P = kq.kq_w4a8_linear(*args, out_dtype=torch.int32)
    torch.cuda.synchronize()
    _check4(xb, q, gs, gb, b, yf, yb, P, f"int4 split {M}x{K}x{N}")


@pytest.mark.parametrize("tile", ["128x256", "128x128", "64x128"])
@pytest.mark.parametrize("split", ["2", "3", "7"])
@pytest.mark.parametrize("M,K,N", [(257, 3200, 200), (100, 2112, 129)])
def test_int4_forced_splits_every_tile(M, K, N, tile, split, kq_env):
    """Ragged M and N; 50 and 33 groups, so the last slice holds a partial
    16-group chunk (or a single group)."""
    kq_env(KQ_FORCE_ROUTE="gemm", KQ_TILE=tile, KQ_SPLIT=split)
    assert kq.kq_route(M, N, K, kq.KQ_W4_AFFINE_G64)["splits"] > 1
    xb, p, gs, gb, q, b = _problem4(M, K, N, seed=2 * M + N + int(split))
    args = (dev_bf16(xb), dev(p), dev(gs), dev(gb))
    yf = kq.kq_w4a8_linear(*args, bias=dev(b), out_dtype=torch.float32)
    yb = kq.kq_w4a8_linear(*args, bias=dev(b), out_dtype=torch.bfloat16)
    P = kq.kq_w4a8_linear(*args, out_dtype=torch.int32)
    torch.cuda.synchronize()
    _check4(xb, q, gs, gb, b, yf, yb, P, f"int4 {tile} split {split}")


def test_int4_split_with_gated_epilogue(kq_env):
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_SPLIT=None)
    M, K, N = 128, 12288, 3072
    assert kq.kq_route(M, N, K, kq.KQ_W4_AFFINE_G64)["splits"] > 1
    xb, p, gs, gb, q, b = _problem4(M, K, N, seed=41)
    r = synth.random_bf16((M, N), seed=42)
    g = synth.random_f32((1, N), seed=43, scale=0.5)
    y = kq.kq_linear_gated(kq.KQ_W4_AFFINE_G64, dev_bf16(xb), dev(p), dev(gs), dev(gb),
                           bias=dev(b), residual=dev_bf16(r), gate=dev(g), gate_rows=M,
                           out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.gated_residual_exact(oracle.w4a8_linear_exact(xb, q, gs, gb, b), r, g, M)
    T = oracle.gated_magnitude(oracle.w4a8_magnitude(xb, q, gs, gb, b), r, g, M)
    check_bf16(host_bf16_bits(y), ref, T, "int4 split gated")


# The 4-buffer ring (tiles up to 128x128 on grids of at most one workgroup
# per CU, K/64 a multiple of 8 in every slice): the same sums and epilogue
# as the 2-buffer ring, so every output bit agrees with KQ_DEEP_RING=0.
@pytest.mark.parametrize("tile", ["128x128", "64x64"])
@pytest.mark.parametrize("split", [None, "1", "2", "6"])
@pytest.mark.parametrize("M,K,N", [(128, 12288, 3072), (100, 4096, 500), (256, 512, 129),
                                   (64, 3584, 1000)])
def test_deep_ring_matches_two_buffer_ring(M, K, N, tile, split, kq_env):
    kq_env(KQ_FORCE_ROUTE="gemm", KQ_TILE=tile, KQ_SPLIT=split, KQ_DEEP_RING=None)
    print(f"[splitk] deep ring {M}x{K}x{N} tile {tile} split {split}", flush=True)
    xb, q8, sw, b = _problem(M, K, N, seed=3 * M + K + N)
    args = (dev_bf16(xb), dev(q8), dev(sw), dev(b))
    outs = {}
    for deep in (None, "0"):
        kq_env(KQ_DEEP_RING=deep)
        outs[deep] = [kq.kq_w8a8_linear(*args, out_dtype=dt) for dt in (torch.float32, torch.bfloat16)]
        outs[deep].append(kq.kq_w8a8_linear(*args[:3], out_dtype=torch.int32))
    torch.cuda.synchronize()
    for a, c in zip(outs[None], outs["0"]):
        assert torch.equal(_bits(a), _bits(c))
    a, _, _ = oracle.quantize_act(xb)
    assert np.array_equal(host(outs[None][2]), oracle.w8a8_acc(a, q8))
    y64 = oracle.w8a8_linear_exact(xb, q8, sw, b)
    T = oracle.w8a8_magnitude(xb, q8, sw, b)
    check_f32(host(outs[None][0]), y64, T, f"deep ring {M}x{K}x{N} f32")
    check_bf16(host_bf16_bits(outs[None][1]), y64, T, f"deep ring {M}x{K}x{N} bf16")
