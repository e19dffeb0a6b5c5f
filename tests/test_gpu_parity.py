"""GPU parity: libkq (through its C ABI and the thin binding) against the
CPU oracle on identical seeded inputs."""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
import w8a8_gemm_dit_amd as kq
from tests.parity import check_bf16, check_f32, dev, dev_bf16, host, host_bf16_bits

pytestmark = pytest.mark.gpu


def setup_module(module):
    print(f"[parity] device: {torch.cuda.get_device_name(0)}", flush=True)
    assert kq.kq_is_available(), "libkq reports no gfx950 device"


# -------------------------------------------------------------- quantizers
K_SWEEP = [1, 7, 8, 31, 33, 63, 64, 65, 127, 128, 511, 512, 520, 3072, 4096, 5120,
           12288, 16384, 20000, 20001]


@pytest.mark.parametrize("K", K_SWEEP)
@pytest.mark.parametrize("M", [1, 5, 256, 257])
def test_quantize_act_k_sweep(M, K):
    xb = synth.random_bf16((M, K), seed=1000 + K + M, scale=2.0, dist="student_t4")
    a_ref, sx_ref, g_ref = oracle.quantize_act(xb)
    a, sx, g = kq.kq_quantize_act(dev_bf16(xb), group_sums=(K % 64 == 0))
    torch.cuda.synchronize()
    assert np.array_equal(host(a), a_ref)
    assert np.array_equal(host(sx).view(np.uint32), sx_ref.view(np.uint32))
    if K % 64 == 0:
        assert np.array_equal(host(g), g_ref)


def test_quantize_act_special_rows():
    K = 3072
    x = synth.bf16_bits_to_f32(synth.random_bf16((8, K), seed=7)).copy()
    x[0] = 0.0                               # zero row
    x[1] = 0.0
    x[1, 17] = 1e-38                         # 127/amax overflows -> zero row
    x[2] *= np.float32(1e-36)                # tiny, still quantizes
    x[3] = 0.0
    x[3, ::7] = np.float32(2.0 ** -130)      # subnormal values (bf16 keeps them)
    x[4, 5] = np.float32(3.0e38)             # huge outlier
    x[5] = np.round(x[5] * 40)               # ties at .5 after scaling
    x[6] *= np.float32(-1.0)
    xb = synth.to_bf16_bits(x)
    a_ref, sx_ref, g_ref = oracle.quantize_act(xb)
    a, sx, g = kq.kq_quantize_act(dev_bf16(xb), group_sums=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(a), a_ref)
    assert np.array_equal(host(sx).view(np.uint32), sx_ref.view(np.uint32))
    assert np.array_equal(host(g), g_ref)


@pytest.mark.parametrize("N,K", [(1, 64), (33, 192), (257, 3072), (48, 5120), (130, 12288)])
def test_quantize_weights_bit_exact(N, K):
    w = synth.random_f32((N, K), seed=N + K, scale=0.02)
    w[0, :64] = 0.0                           # degenerate group / row part
    if N > 2:
        w[2] = 0.0                            # zero row -> scale 0
    wd = dev(w)
    q8, sw, none = kq.kq_quantize_weights(wd, kq.KQ_W8_PER_CHANNEL)
    q4, gs, gb = kq.kq_quantize_weights(wd, kq.KQ_W4_AFFINE_G64)
    torch.cuda.synchronize()
    assert none is None
    q8_ref, sw_ref = oracle.quantize_w8(w)
    assert np.array_equal(host(q8), q8_ref)
    assert np.array_equal(host(sw).view(np.uint32), sw_ref.view(np.uint32))
    p_ref, gs_ref, gb_ref, _ = oracle.quantize_w4(w)
    assert np.array_equal(host(q4), p_ref)
    assert np.array_equal(host(gs).view(np.uint16), gs_ref.view(np.uint16))
    assert np.array_equal(host(gb).view(np.uint16), gb_ref.view(np.uint16))


# ---------------------------------------------------------------- linears
def _problem(M, K, N, seed, dist="normal", with_bias=True):
    xb = synth.random_bf16((M, K), seed=seed, dist=dist)
    w = synth.random_f32((N, K), seed=seed + 1, scale=0.02)
    b = synth.random_f32((N,), seed=seed + 2, scale=0.1) if with_bias else None
    return xb, w, b


# K covers both GEMM loop variants (K % 256 == 0, and 1-3 trailing 64-steps)
SHAPES = [(64, 512, 512), (1, 64, 16), (17, 64, 33), (100, 192, 200), (257, 128, 129),
          (300, 256, 48), (64, 1024, 1000), (513, 320, 260), (300, 448, 200), (130, 576, 72),
          (70, 640, 70)]
TILES = [None, "256x256", "256x256w8", "256x192", "256x128", "128x128", "64x64"]


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_w8a8_accumulators_bit_exact(M, K, N, tile, kq_env):
    kq_env(KQ_TILE=tile, KQ_FORCE_ROUTE="gemm")
    xb, w, _ = _problem(M, K, N, seed=M * 7 + K + N)
    q8, sw = oracle.quantize_w8(w)
    a, _, _ = oracle.quantize_act(xb)
    acc = kq.kq_w8a8_linear(dev_bf16(xb), dev(q8), dev(sw), out_dtype=torch.int32)
    torch.cuda.synchronize()
    assert np.array_equal(host(acc), oracle.w8a8_acc(a, q8))


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("tile", [None, "256x256", "256x256w8", "256x192", "64x64"])
@pytest.mark.parametrize("M,K,N", SHAPES[:6])
def test_w8a8_outputs(M, K, N, tile, out, kq_env):
    kq_env(KQ_TILE=tile, KQ_FORCE_ROUTE="gemm")
    xb, w, b = _problem(M, K, N, seed=M + 3 * K + N, with_bias=(M % 2 == 0))
    q8, sw = oracle.quantize_w8(w)
    y64 = oracle.w8a8_linear_exact(xb, q8, sw, b)
    T = oracle.w8a8_magnitude(xb, q8, sw, b)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    y = kq.kq_w8a8_linear(dev_bf16(xb), dev(q8), dev(sw), None if b is None else dev(b), out_dtype=dt)
    torch.cuda.synchronize()
    if out == "f32":
        check_f32(host(y), y64, T, f"w8a8 {M}x{K}x{N}")
    else:
        check_bf16(host_bf16_bits(y), y64, T, f"w8a8 {M}x{K}x{N}")


# K spanning several 16-group chunks of the int4 GEMM, whole and partial
SHAPES_W4 = SHAPES + [(130, 2048, 200), (96, 2112, 272)]


@pytest.mark.parametrize("tile", [None, "128x256", "128x128", "64x128"])
@pytest.mark.parametrize("M,K,N", SHAPES_W4)
def test_w4a8_group_products_bit_exact(M, K, N, tile, kq_env):
    kq_env(KQ_TILE=tile, KQ_FORCE_ROUTE="gemm")
    xb, w, _ = _problem(M, K, N, seed=M + K * 5 + N)
    p, gs, gb, q = oracle.quantize_w4(w)
    a, _, _ = oracle.quantize_act(xb)
    P = kq.kq_w4a8_linear(dev_bf16(xb), dev(p), dev(gs), dev(gb), out_dtype=torch.int32)
    torch.cuda.synchronize()
    assert np.array_equal(host(P), oracle.w4a8_group_acc(a, q))


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("tile", [None, "128x256", "128x128", "64x128"])
@pytest.mark.parametrize("M,K,N", SHAPES[:6] + SHAPES_W4[-2:])
def test_w4a8_outputs(M, K, N, tile, out, kq_env):
    kq_env(KQ_TILE=tile, KQ_FORCE_ROUTE="gemm")
    xb, w, b = _problem(M, K, N, seed=2 * M + K + N, with_bias=(M % 2 == 1))
    p, gs, gb, q = oracle.quantize_w4(w)
    y64 = oracle.w4a8_linear_exact(xb, q, gs, gb, b)
    T = oracle.w4a8_magnitude(xb, q, gs, gb, b)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    y = kq.kq_w4a8_linear(dev_bf16(xb), dev(p), dev(gs), dev(gb), None if b is None else dev(b),
                          out_dtype=dt)
    torch.cuda.synchronize()
    if out == "f32":
        check_f32(host(y), y64, T, f"w4a8 {M}x{K}x{N}")
    else:
        check_bf16(host_bf16_bits(y), y64, T, f"w4a8 {M}x{K}x{N}")


# ------------------------------------------------------------------ GEMV
@pytest.mark.parametrize("M", [1, 2, 4, 7, 16])
@pytest.mark.parametrize("K,N", [(64, 16), (320, 100), (5120, 256), (4160, 33)])
def test_gemv_w4_bit_exact_and_outputs(M, K, N):
    xb, w, b = _problem(M, K, N, seed=M + K + 11 * N)
    p, gs, gb, q = oracle.quantize_w4(w)
    a, _, _ = oracle.quantize_act(xb)
    args = (kq.KQ_W4_AFFINE_G64, dev_bf16(xb), dev(p), dev(gs), dev(gb))
    P = kq.kq_gemv_small_m(*args, out_dtype=torch.int32)
    yf = kq.kq_gemv_small_m(*args, bias=dev(b), out_dtype=torch.float32)
    yb = kq.kq_gemv_small_m(*args, bias=dev(b), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(host(P), oracle.w4a8_group_acc(a, q))
    y64 = oracle.w4a8_linear_exact(xb, q, gs, gb, b)
    T = oracle.w4a8_magnitude(xb, q, gs, gb, b)
    check_f32(host(yf), y64, T, "gemv w4 f32")
    check_bf16(host_bf16_bits(yb), y64, T, "gemv w4 bf16")


@pytest.mark.parametrize("M", [1, 3, 16])
@pytest.mark.parametrize("K,N", [(64, 16), (5120, 300)])
def test_gemv_w8(M, K, N):
    xb, w, b = _problem(M, K, N, seed=M + K + 13 * N)
    q8, sw = oracle.quantize_w8(w)
    a, _, _ = oracle.quantize_act(xb)
    args = (kq.KQ_W8_PER_CHANNEL, dev_bf16(xb), dev(q8), dev(sw), None)
    acc = kq.kq_gemv_small_m(*args, out_dtype=torch.int32)
    yf = kq.kq_gemv_small_m(*args, bias=dev(b), out_dtype=torch.float32)
    yb = kq.kq_gemv_small_m(*args, bias=dev(b), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(host(acc), oracle.w8a8_acc(a, q8))
    y64 = oracle.w8a8_linear_exact(xb, q8, sw, b)
    T = oracle.w8a8_magnitude(xb, q8, sw, b)
    check_f32(host(yf), y64, T, "gemv w8 f32")
    check_bf16(host_bf16_bits(yb), y64, T, "gemv w8 bf16")


@pytest.mark.parametrize("fmt", ["w8", "w4"])
@pytest.mark.parametrize("M,K,N", [(300, 640, 48), (2048, 512, 64), (33, 128, 40), (17, 5120, 16)])
def test_thin_n_linears_take_the_gemv(M, K, N, fmt, kq_env):
    """Thin N at any M with the fused route off (KQ_FUSE=0): 16-row blocks
    of the GEMV kernel (ragged last block) after the quantize kernel,
    against the oracle; int32 bit-exact, outputs within tolerance."""
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_FUSE="0")
    assert kq.kq_route(M, N, K, kq.KQ_W8_PER_CHANNEL)["kind"] == "gemv"
    xb, w, b = _problem(M, K, N, seed=3 * M + K + N)
    a, _, _ = oracle.quantize_act(xb)
    x = dev_bf16(xb)
    if fmt == "w8":
        q8, sw = oracle.quantize_w8(w)
        acc = kq.kq_w8a8_linear(x, dev(q8), dev(sw), out_dtype=torch.int32)
        yf = kq.kq_w8a8_linear(x, dev(q8), dev(sw), dev(b), out_dtype=torch.float32)
        yb = kq.kq_w8a8_linear(x, dev(q8), dev(sw), dev(b), out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert np.array_equal(host(acc), oracle.w8a8_acc(a, q8))
        y64 = oracle.w8a8_linear_exact(xb, q8, sw, b)
        T = oracle.w8a8_magnitude(xb, q8, sw, b)
    else:
        p, gs, gb, q = oracle.quantize_w4(w)
        args = (x, dev(p), dev(gs), dev(gb))
        P = kq.kq_w4a8_linear(*args, out_dtype=torch.int32)
        yf = kq.kq_w4a8_linear(*args, bias=dev(b), out_dtype=torch.float32)
        yb = kq.kq_w4a8_linear(*args, bias=dev(b), out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert np.array_equal(host(P), oracle.w4a8_group_acc(a, q))
        y64 = oracle.w4a8_linear_exact(xb, q, gs, gb, b)
        T = oracle.w4a8_magnitude(xb, q, gs, gb, b)
    check_f32(host(yf), y64, T, f"thin {fmt} f32")
    check_bf16(host_bf16_bits(yb), y64, T, f"thin {fmt} bf16")


@pytest.mark.parametrize("fmt", ["w8", "w4"])
@pytest.mark.parametrize("M", [17, 24, 32])
def test_gemv_route_up_to_32_rows(M, fmt, kq_env):
    """17..32 rows still take the GEMV kernel (two 16-row blocks, the
    second ragged), against the oracle."""
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_SPLIT=None)
    K, N = 1024, 1000
    assert kq.kq_route(M, N, K, kq.KQ_W8_PER_CHANNEL)["kind"] == "gemv"
    xb, w, b = _problem(M, K, N, seed=M + 17)
    a, _, _ = oracle.quantize_act(xb)
    x = dev_bf16(xb)
    if fmt == "w8":
        q8, sw = oracle.quantize_w8(w)
        acc = kq.kq_w8a8_linear(x, dev(q8), dev(sw), out_dtype=torch.int32)
        yb = kq.kq_w8a8_linear(x, dev(q8), dev(sw), dev(b), out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert np.array_equal(host(acc), oracle.w8a8_acc(a, q8))
        y64, T = oracle.w8a8_linear_exact(xb, q8, sw, b), oracle.w8a8_magnitude(xb, q8, sw, b)
    else:
        p, gs, gb, q = oracle.quantize_w4(w)
        P = kq.kq_w4a8_linear(x, dev(p), dev(gs), dev(gb), out_dtype=torch.int32)
        yb = kq.kq_w4a8_linear(x, dev(p), dev(gs), dev(gb), bias=dev(b), out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert np.array_equal(host(P), oracle.w4a8_group_acc(a, q))
        y64, T = oracle.w4a8_linear_exact(xb, q, gs, gb, b), oracle.w4a8_magnitude(xb, q, gs, gb, b)
    check_bf16(host_bf16_bits(yb), y64, T, f"gemv {M} rows {fmt}")


@pytest.mark.parametrize("M", [3, 8])
def test_gemv_and_gemm_routes_agree_bitwise(M, kq_env):
    # The same per-group products whichever kernel runs (decode steps stay
    # bit-identical across routes, as MLX pull request 4722 checks).
    K, N = 1024, 200
    xb, w, b = _problem(M, K, N, seed=99)
    p, gs, gb, q = oracle.quantize_w4(w)
    args = (dev_bf16(xb), dev(p), dev(gs), dev(gb))
    kq_env(KQ_FORCE_ROUTE="gemv")
    P1 = host(kq.kq_w4a8_linear(*args, out_dtype=torch.int32))
    kq_env(KQ_FORCE_ROUTE="gemm")
    P2 = host(kq.kq_w4a8_linear(*args, out_dtype=torch.int32))
    assert np.array_equal(P1, P2)


# ------------------------------------------------------------- behaviour
def test_route_log_names_kernels(kq_env, capfd):
    kq_env(KQ_LOG="1", KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_FUSE=None)
    xb, w, b = _problem(5, 256, 96, seed=5)  # N > 64: M = 300 takes the GEMM
    p, gs, gb, _ = oracle.quantize_w4(w)
    kq.kq_w4a8_linear(dev_bf16(xb), dev(p), dev(gs), dev(gb))
    xb2 = synth.random_bf16((300, 256), seed=6)
    kq.kq_w4a8_linear(dev_bf16(xb2), dev(p), dev(gs), dev(gb))
    xb3 = synth.random_bf16((4, 256), seed=7)
    kq.kq_w4a8_linear(dev_bf16(xb3), dev(p), dev(gs), dev(gb))
    torch.cuda.synchronize()
    lines = capfd.readouterr().err.splitlines()
    m5 = [l for l in lines if "kq_w4a8_linear M=5 " in l]
    m300 = [l for l in lines if "kq_w4a8_linear M=300 " in l]
    m4 = [l for l in lines if "kq_w4a8_linear M=4 " in l]
    assert m5 and "route=gemv" in m5[0] and "quant_act" in m5[0] and "gemv_w4a8" in m5[0]
    assert m300 and "route=gemm" in m300[0] and "gemm_w4a8_" in m300[0]
    assert m4 and "route=fused" in m4[0] and "gemv_xq_w4a8" in m4[0]


def test_empty_and_error_paths():
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros((64, 128), dtype=torch.int8, device="cuda")
    sw = torch.ones((64,), dtype=torch.float32, device="cuda")
    y = kq.kq_w8a8_linear(x, wq, sw)
    assert y.shape == (0, 64)
    xb = torch.zeros((4, 100), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="K=100 must be a positive multiple of 64"):
        kq.kq_w8a8_linear(xb, torch.zeros((64, 100), dtype=torch.int8, device="cuda"), sw)
    # a misaligned x (an offset view of a larger buffer)
    big = torch.zeros((4 * 128 + 8,), dtype=torch.bfloat16, device="cuda")
    xm = big[1:1 + 4 * 128].view(4, 128)
    with pytest.raises(ValueError, match="16-byte aligned"):
        kq.kq_w8a8_linear(xm, wq, sw)


def test_deterministic_bits():
    M, K, N = 512, 1024, 768
    xb, w, b = _problem(M, K, N, seed=42)
    q8, sw = oracle.quantize_w8(w)
    p, gs, gb, _ = oracle.quantize_w4(w)
    x = dev_bf16(xb)
    r1 = kq.kq_w8a8_linear(x, dev(q8), dev(sw), dev(b)).clone()
    r2 = kq.kq_w8a8_linear(x, dev(q8), dev(sw), dev(b)).clone()
    s1 = kq.kq_w4a8_linear(x, dev(p), dev(gs), dev(gb), dev(b)).clone()
    s2 = kq.kq_w4a8_linear(x, dev(p), dev(gs), dev(gb), dev(b)).clone()
    torch.cuda.synchronize()
    assert torch.equal(r1.view(torch.int16), r2.view(torch.int16))
    assert torch.equal(s1.view(torch.int16), s2.view(torch.int16))


# ------------------------------------------------------ full-size workloads
def _workers():
    n = len(os.sched_getaffinity(0))
    return max(1, min(8, n // 2))


@pytest.mark.parametrize("name", [n for n in synth.WORKLOADS])
def test_workload_full_size_every_row(name):
    """Full-size launch, as the benchmark runs it: the weights bit-exact in
    full and EVERY output element against the oracle (computed by blocks of
    rows, which the per-row quantization makes independent).  The MLP down
    projection takes the oracle's up projection output as its input."""
    from tests import fullsize

    wl = synth.WORKLOADS[name]
    print(f"[parity] workload {name} (every row)", flush=True)
    w = synth.weights(wl)
    b = synth.bias(wl)
    out_dt = torch.float32 if wl.out == "f32" else torch.bfloat16
    wd = dev(w)
    if wl.fmt == "w8":
        q8, sw, _ = kq.kq_quantize_weights(wd, kq.KQ_W8_PER_CHANNEL)
        q8_ref, sw_ref = fullsize.quantized_weights(name)
        assert np.array_equal(host(q8), q8_ref)
        assert np.array_equal(host(sw).view(np.uint32), sw_ref.view(np.uint32))
        run = lambda x: kq.kq_w8a8_linear(x, q8, sw, dev(b), out_dtype=out_dt)  # noqa: E731
    else:
        p, gs, gb = kq.kq_quantize_weights(wd, kq.KQ_W4_AFFINE_G64)
        p_ref, gs_ref, gb_ref, _ = fullsize.quantized_weights(name)
        assert np.array_equal(host(p), p_ref)
        assert np.array_equal(host(gs).view(np.uint16), gs_ref.view(np.uint16))
        assert np.array_equal(host(gb).view(np.uint16), gb_ref.view(np.uint16))
        run = lambda x: kq.kq_w4a8_linear(x, p, gs, gb, dev(b), out_dtype=out_dt)  # noqa: E731
    del wd
    got = list(fullsize.blocks(name, wl.M, 2048 if wl.fmt == "w8" else 256, _workers()))
    xb = np.concatenate([g[2] for g in got])      # the input rows, in order
    assert xb.shape == (wl.M, wl.K)
    y = run(dev_bf16(xb))
    torch.cuda.synchronize()
    y_host = host(y) if wl.out == "f32" else host_bf16_bits(y)
    for r0, r1, _, y64, T in got:
        if wl.out == "f32":
            check_f32(y_host[r0:r1], y64, T, f"{name} rows {r0}:{r1}")
        else:
            check_bf16(y_host[r0:r1], y64, T, f"{name} rows {r0}:{r1}")


@pytest.mark.parametrize("name,split", [
    ("dit_proj_w8a8_4096x3072x3072", None),
    ("dit_4k_w8a8_16384x3072x12288", None),
    ("short_seq_w8a8_128x12288x3072", None),
    ("short_seq_w8a8_128x12288x3072", "1"),
])
def test_workload_full_size_w8a8_accumulators(name, split, kq_env):
    """The int32 accumulators of a full-size int8 workload, every element
    bit-exact: the big tiles' XCD-remapped tile walk at the DiT shapes, and
    a K = 12288 product both split (the automatic route) and unsplit."""
    from tests import fullsize

    kq_env(KQ_SPLIT=split)
    wl = synth.WORKLOADS[name]
    print(f"[parity] workload {name} int32 accumulators (KQ_SPLIT={split})", flush=True)
    xb = synth.activations(wl)
    q8_ref, sw_ref = fullsize.quantized_weights(name)
    acc = kq.kq_w8a8_linear(dev_bf16(xb), dev(q8_ref), dev(sw_ref), out_dtype=torch.int32)
    torch.cuda.synchronize()
    acc = host(acc)
    for r0 in range(0, wl.M, 2048):
        r1 = min(wl.M, r0 + 2048)
        a, _, _ = oracle.quantize_act(xb[r0:r1], with_group_sums=False)
        assert np.array_equal(acc[r0:r1], oracle.w8a8_acc(a, q8_ref)), (name, r0)


@pytest.mark.parametrize("name", ["dit_mlp_up_w4a8_2048x4096x12288",
                                  "dit_mlp_down_w4a8_2048x12288x4096"])
def test_workload_full_size_w4a8_group_products(name):
    """The per-group int32 products P [K/64, M, N] of a full-size int4
    workload, every element bit-exact (compared one group at a time)."""
    from tests import fullsize

    wl = synth.WORKLOADS[name]
    print(f"[parity] workload {name} per-group products", flush=True)
    xb = synth.activations(wl)          # int products: any input of the shape
    p_ref, gs_ref, gb_ref, q_ref = fullsize.quantized_weights(name)
    P = kq.kq_w4a8_linear(dev_bf16(xb), dev(p_ref), dev(gs_ref), dev(gb_ref),
                          out_dtype=torch.int32)
    torch.cuda.synchronize()
    a, _, _ = oracle.quantize_act(xb, with_group_sums=False)
    for g in range(wl.K // 64):
        sl = slice(64 * g, 64 * g + 64)
        want = oracle.w4a8_group_acc(a[:, sl], q_ref[:, sl])[0]
        assert np.array_equal(host(P[g]), want), (name, g)
    del P


# ------------------------------------------------------- golden fixture
def _golden_case():
    import json

    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "small_cases.json")
    with open(path) as f:
        d = json.load(f)

    def arr(key, dtype, shape):
        return np.array([int(h, 16) for h in d[key]], dtype=dtype).reshape(shape)

    return d, arr


@pytest.mark.parametrize("route", ["gemm", "gemv"])
def test_golden_small_cases(route, kq_env):
    """The stored fixture (oracle results, tests/golden/make_golden.py) on
    the GPU: codes, scales, sums, weights, accumulators and group products
    bit-exact; fp32 outputs within 1e-5 of the stored ones (relative to the
    term magnitude) and bf16 outputs within 1 ulp."""
    kq_env(KQ_FORCE_ROUTE=route)
    d, arr = _golden_case()
    M, K, N = d["shape"]["M"], d["shape"]["K"], d["shape"]["N"]
    G = K // 64
    print(f"[parity] golden small cases, route {route}", flush=True)
    xb = arr("x_bf16_bits", np.uint16, (M, K))
    w = arr("w_f32_bits", np.uint32, (N, K)).view(np.float32)
    b = arr("bias_f32_bits", np.uint32, (N,)).view(np.float32)
    x = dev_bf16(xb)
    a, sx, gsum = kq.kq_quantize_act(x, group_sums=True)
    q8, sw, _ = kq.kq_quantize_weights(dev(w), kq.KQ_W8_PER_CHANNEL)
    p4, gs, gb = kq.kq_quantize_weights(dev(w), kq.KQ_W4_AFFINE_G64)
    torch.cuda.synchronize()
    assert host(a).astype(int).ravel().tolist() == d["act_codes"]
    assert np.array_equal(host(sx).view(np.uint32), arr("act_scale_f32_bits", np.uint32, (M,)))
    assert host(gsum).astype(int).ravel().tolist() == d["act_group_sums"]
    assert host(q8).astype(int).ravel().tolist() == d["w8_codes"]
    assert np.array_equal(host(sw).view(np.uint32), arr("w8_scale_f32_bits", np.uint32, (N,)))
    assert host(p4).astype(int).ravel().tolist() == d["w4_packed"]
    assert np.array_equal(host(gs).view(np.uint16), arr("w4_scale_f16_bits", np.uint16, (N, G)))
    assert np.array_equal(host(gb).view(np.uint16), arr("w4_offset_f16_bits", np.uint16, (N, G)))

    # magnitudes for the fp32 tolerance, from the stored quantized operands
    q8h = np.array(d["w8_codes"], np.int8).reshape(N, K)
    swh = arr("w8_scale_f32_bits", np.uint32, (N,)).view(np.float32)
    q4h = oracle.unpack_w4(np.array(d["w4_packed"], np.uint8).reshape(N, K // 2))
    gsh = arr("w4_scale_f16_bits", np.uint16, (N, G)).view(np.float16)
    gbh = arr("w4_offset_f16_bits", np.uint16, (N, G)).view(np.float16)
    T8 = oracle.w8a8_magnitude(xb, q8h, swh, b)
    T4 = oracle.w4a8_magnitude(xb, q4h, gsh, gbh, b)

    def check(y_f32, y_bf16, key32, key16, T):
        r32 = arr(key32, np.uint32, (M, N)).view(np.float32).astype(np.float64)
        err = np.abs(host(y_f32).astype(np.float64) - r32)
        assert (err <= 1e-5 * np.maximum(np.abs(r32), T)).all(), key32
        r16 = arr(key16, np.uint16, (M, N))
        g = oracle.bf16_bits_to_f32(host_bf16_bits(y_bf16)).astype(np.float64)
        r = oracle.bf16_bits_to_f32(r16).astype(np.float64)
        assert (np.abs(g - r) <= oracle.bf16_ulp(r16)).all(), key16

    bd = dev(b)
    acc = kq.kq_w8a8_linear(x, q8, sw, out_dtype=torch.int32)
    y32 = kq.kq_w8a8_linear(x, q8, sw, bd, out_dtype=torch.float32)
    y16 = kq.kq_w8a8_linear(x, q8, sw, bd, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert host(acc).astype(np.int64).ravel().tolist() == d["w8a8_acc"]
    check(y32, y16, "w8a8_y_f32_bits", "w8a8_y_bf16_bits", T8)
    P = kq.kq_w4a8_linear(x, p4, gs, gb, out_dtype=torch.int32)
    y32 = kq.kq_w4a8_linear(x, p4, gs, gb, bd, out_dtype=torch.float32)
    y16 = kq.kq_w4a8_linear(x, p4, gs, gb, bd, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert host(P).astype(np.int64).ravel().tolist() == d["w4a8_group_products_gmn"]
    check(y32, y16, "w4a8_y_f32_bits", "w4a8_y_bf16_bits", T4)


@pytest.mark.parametrize("fmt", ["w4", "w8"])
def test_golden_rows_on_gemv(fmt):
    """The fixture's first four rows (plain, all zero, subnormal, ties at
    amax 127) through kq_gemv_small_m."""
    d, arr = _golden_case()
    M, K, N = 4, d["shape"]["K"], d["shape"]["N"]
    Mf, G = d["shape"]["M"], K // 64
    xb = arr("x_bf16_bits", np.uint16, (Mf, K))[:M]
    b = arr("bias_f32_bits", np.uint32, (N,)).view(np.float32)
    x = dev_bf16(xb)
    if fmt == "w4":
        p4 = np.array(d["w4_packed"], np.uint8).reshape(N, K // 2)
        gs = arr("w4_scale_f16_bits", np.uint16, (N, G)).view(np.float16)
        gb = arr("w4_offset_f16_bits", np.uint16, (N, G)).view(np.float16)
        args = (kq.KQ_W4_AFFINE_G64, x, dev(p4), dev(gs), dev(gb))
        ref_int = np.array(d["w4a8_group_products_gmn"], np.int64).reshape(G, Mf, N)[:, :M]
        q4 = oracle.unpack_w4(p4)
        T = oracle.w4a8_magnitude(xb, q4, gs, gb, b)
        k32, k16 = "w4a8_y_f32_bits", "w4a8_y_bf16_bits"
    else:
        q8 = np.array(d["w8_codes"], np.int8).reshape(N, K)
        sw = arr("w8_scale_f32_bits", np.uint32, (N,)).view(np.float32)
        args = (kq.KQ_W8_PER_CHANNEL, x, dev(q8), dev(sw), None)
        ref_int = np.array(d["w8a8_acc"], np.int64).reshape(Mf, N)[:M]
        T = oracle.w8a8_magnitude(xb, q8, sw, b)
        k32, k16 = "w8a8_y_f32_bits", "w8a8_y_bf16_bits"
    P = kq.kq_gemv_small_m(*args, out_dtype=torch.int32)
    yf = kq.kq_gemv_small_m(*args, bias=dev(b), out_dtype=torch.float32)
    yb = kq.kq_gemv_small_m(*args, bias=dev(b), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(host(P).astype(np.int64), ref_int)
    r32 = arr(k32, np.uint32, (Mf, N)).view(np.float32)[:M].astype(np.float64)
    assert (np.abs(host(yf).astype(np.float64) - r32) <= 1e-5 * np.maximum(np.abs(r32), T)).all()
    r16 = arr(k16, np.uint16, (Mf, N))[:M]
    g = oracle.bf16_bits_to_f32(host_bf16_bits(yb)).astype(np.float64)
    r = oracle.bf16_bits_to_f32(r16).astype(np.float64)
    assert (np.abs(g - r) <= oracle.bf16_ulp(r16)).all()


# -------------------------------------------- persistent tile loop (int8)
# More whole 256x192 tiles than CUs with K % 256 == 0 takes the persistent
# kernel (one workgroup per CU looping over tiles, the next tile's first
# operands fetched during the current tile's last steps) under KQ_PERSIST=1;
# KQ_PERSIST=0 gives the one-tile-per-workgroup kernel.  Shapes: whole tiles (persistent:
# 320, 288 and 270 tiles, K from 512 to 3072), then ragged M and N and N not
# a multiple of 4 (which keep the one-tile kernel).
PERSIST_SHAPES = [(2560, 512, 6144), (4096, 3072, 3456), (2304, 1024, 5760), (4100, 1024, 3000),
                  (4100, 256, 2998)]


@pytest.mark.parametrize("M,K,N", PERSIST_SHAPES)
def test_persistent_gemm_matches_oracle_and_one_tile_kernel(M, K, N, kq_env):
    print(f"[parity] persistent {M}x{K}x{N}", flush=True)
    kq_env(KQ_TILE="256x192", KQ_PERSIST="1")
    xb, w, b = _problem(M, K, N, seed=M + N)
    q8, sw = oracle.quantize_w8(w)
    x, wq, swd, bd = dev_bf16(xb), dev(q8), dev(sw), dev(b)
    acc = kq.kq_w8a8_linear(x, wq, swd, out_dtype=torch.int32)
    y16 = kq.kq_w8a8_linear(x, wq, swd, bd, out_dtype=torch.bfloat16)
    y32 = kq.kq_w8a8_linear(x, wq, swd, bd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    a, _, _ = oracle.quantize_act(xb, with_group_sums=False)
    assert np.array_equal(host(acc), oracle.w8a8_acc(a, q8))
    y64 = oracle.w8a8_linear_exact(xb, q8, sw, b)
    T = oracle.w8a8_magnitude(xb, q8, sw, b)
    check_bf16(host_bf16_bits(y16), y64, T, f"persistent bf16 {M}x{K}x{N}")
    check_f32(host(y32), y64, T, f"persistent f32 {M}x{K}x{N}")
    kq_env(KQ_PERSIST="0")
    r16 = kq.kq_w8a8_linear(x, wq, swd, bd, out_dtype=torch.bfloat16)
    r32 = kq.kq_w8a8_linear(x, wq, swd, bd, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y16.view(torch.int16), r16.view(torch.int16))
    assert torch.equal(y32.view(torch.int32), r32.view(torch.int32))


def test_persistent_gemm_gated_in_place(kq_env):
    M, K, N, L = 4100, 1024, 3000, 100
    print(f"[parity] persistent gated {M}x{K}x{N} L={L}", flush=True)
    kq_env(KQ_TILE="256x192")
    xb, w, b = _problem(M, K, N, seed=5)
    q8, sw = oracle.quantize_w8(w)
    r = synth.random_bf16((M, N), seed=6)
    gate = synth.random_f32((-(-M // L), N), seed=7, scale=0.5)
    x, wq, swd, bd = dev_bf16(xb), dev(q8), dev(sw), dev(b)
    y = dev_bf16(r)
    kq.kq_linear_gated(kq.KQ_W8_PER_CHANNEL, x, wq, swd, None, bd, residual=y, gate=dev(gate),
                       gate_rows=L, out_dtype=torch.bfloat16, out=y)
    torch.cuda.synchronize()
    y64 = oracle.gated_residual_exact(oracle.w8a8_linear_exact(xb, q8, sw, b), r, gate, L)
    T = oracle.gated_magnitude(oracle.w8a8_magnitude(xb, q8, sw, b), r, gate, L)
    check_bf16(host_bf16_bits(y), y64, T, "persistent gated in place")
