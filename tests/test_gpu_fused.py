"""GPU parity of the fused routes (route kind "fused"), where the linear's
product kernel quantizes x itself: the thin-N kernel (8 rows of x per
workgroup, all N <= 64 columns; M > 16, K <= 6144) and the GEMV with the
quantization in its prologue (M <= 4, K <= 6144), against the oracle and
against the two-kernel routes (quantize kernel + GEMV, KQ_FUSE=0).

Bars as in the other parity tests: int32 accumulators and per-group
products bit-exact (they pin the codes the kernel forms in registers), the
token scales it stores bit-exact, fp32 outputs within 1e-5 of the term
magnitude, bf16 outputs within 1 ulp."""
import numpy as np
import pytest
import torch

import oracle
import synth
import w8a8_gemm_dit_amd as kq
from tests.parity import check_bf16, check_f32, dev, dev_bf16, host, host_bf16_bits

pytestmark = pytest.mark.gpu


def setup_module(module):
    print(f"[fused] device: {torch.cuda.get_device_name(0)}", flush=True)
    assert kq.kq_is_available(), "libkq reports no gfx950 device"


# (M, K, N): ragged 8-row blocks, 1-4 column blocks (ragged), K from one group
# (15 idle slices) through uneven slices (17 groups) to the 6144 limit
SHAPES = [(17, 64, 1), (33, 128, 16), (300, 640, 48), (2048, 512, 64), (100, 1088, 33),
          (65, 5120, 48), (40, 6144, 64), (257, 960, 17), (18, 1024, 40), (31, 192, 5)]


def _fmt_code(fmt):
    return kq.KQ_W8_PER_CHANNEL if fmt == "w8" else kq.KQ_W4_AFFINE_G64


def _run(fmt, xb, w, b, out_dtype, workspace=None):
    x = dev_bf16(xb)
    if fmt == "w8":
        q8, sw = oracle.quantize_w8(w)
        return kq.kq_w8a8_linear(x, dev(q8), dev(sw), None if b is None else dev(b),
                                 out_dtype=out_dtype, workspace=workspace)
    p, gs, gb, _ = oracle.quantize_w4(w)
    return kq.kq_w4a8_linear(x, dev(p), dev(gs), dev(gb), None if b is None else dev(b),
                             out_dtype=out_dtype, workspace=workspace)


def _exact(fmt, xb, w, b):
    if fmt == "w8":
        q8, sw = oracle.quantize_w8(w)
        return oracle.w8a8_linear_exact(xb, q8, sw, b), oracle.w8a8_magnitude(xb, q8, sw, b)
    _, gs, gb, q = oracle.quantize_w4(w)
    return oracle.w4a8_linear_exact(xb, q, gs, gb, b), oracle.w4a8_magnitude(xb, q, gs, gb, b)


def _int_ref(fmt, xb, w):
    a, _, _ = oracle.quantize_act(xb)
    if fmt == "w8":
        q8, _ = oracle.quantize_w8(w)
        return oracle.w8a8_acc(a, q8)
    _, _, _, q = oracle.quantize_w4(w)
    return oracle.w4a8_group_acc(a, q)


def _check_all(fmt, xb, w, b, what):
    M, K = xb.shape
    N = w.shape[0]
    fc = _fmt_code(fmt)
    ws = torch.zeros((kq.kq_workspace_bytes(M, N, K, fc),), dtype=torch.uint8, device="cuda")
    acc = _run(fmt, xb, w, None, torch.int32, workspace=ws)
    yf = _run(fmt, xb, w, b, torch.float32)
    yb = _run(fmt, xb, w, b, torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(host(acc), _int_ref(fmt, xb, w)), f"{what}: int32 results"
    # the route keeps only the token scales, at the start of the workspace
    _, sx_ref, _ = oracle.quantize_act(xb)
    sx = ws[: 4 * M].view(torch.float32)
    assert np.array_equal(host(sx).view(np.uint32), sx_ref.view(np.uint32)), f"{what}: scales"
    y64, T = _exact(fmt, xb, w, b)
    check_f32(host(yf), y64, T, f"{what} f32")
    check_bf16(host_bf16_bits(yb), y64, T, f"{what} bf16")


@pytest.mark.parametrize("fmt", ["w8", "w4"])
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_fused_matches_oracle(M, K, N, fmt, kq_env):
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_FUSE=None)
    r = kq.kq_route(M, N, K, _fmt_code(fmt))
    assert (r["kind"], r["grid"]) == ("fused", -(-M // 8))
    seed = 5 * M + K + 3 * N
    dist = "student_t4" if (M + N) % 2 else "normal"
    xb = synth.random_bf16((M, K), seed=seed, dist=dist)
    w = synth.random_f32((N, K), seed=seed + 1, scale=0.02)
    b = synth.random_f32((N,), seed=seed + 2, scale=0.1)
    print(f"[fused] {fmt} {M}x{K}x{N} {dist}", flush=True)
    _check_all(fmt, xb, w, b, f"fused {fmt} {M}x{K}x{N}")


@pytest.mark.parametrize("fmt", ["w8", "w4"])
def test_fused_special_rows(fmt, kq_env):
    """Rows the quantizer treats specially, inside the fused kernel: zero
    rows, a row whose 127/amax overflows (zero codes and scale), tiny and
    subnormal rows, a huge outlier, ties at .5, negated rows."""
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_FUSE=None)
    M, K, N = 40, 3072, 48
    x = synth.bf16_bits_to_f32(synth.random_bf16((M, K), seed=17)).copy()
    x[0] = 0.0
    x[1] = 0.0
    x[1, 17] = 1e-38
    x[2] *= np.float32(1e-36)
    x[3] = 0.0
    x[3, ::7] = np.float32(2.0 ** -130)
    x[4, 5] = np.float32(3.0e38)
    x[5] = np.round(x[5] * 40)
    x[6] *= np.float32(-1.0)
    x[39] = 0.0                       # last row of a ragged block
    xb = synth.to_bf16_bits(x)
    w = synth.random_f32((N, K), seed=18, scale=0.02)
    b = synth.random_f32((N,), seed=19, scale=0.1)
    assert kq.kq_route(M, N, K, _fmt_code(fmt))["kind"] == "fused"
    _check_all(fmt, xb, w, b, f"fused special rows {fmt}")


@pytest.mark.parametrize("M,K,N", [(300, 640, 48), (100, 1088, 33), (2048, 5120, 48)])
def test_fused_and_two_kernel_routes_agree(M, K, N, kq_env):
    """Same codes, same exact int32 sums and the same epilogue expression:
    for int8 weights the fused and the two-kernel routes agree bit for bit;
    for int4 weights the per-group products do (the fp32 sums run in a
    different slice order)."""
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None)
    seed = M + 2 * K + N
    xb = synth.random_bf16((M, K), seed=seed, dist="student_t4")
    w = synth.random_f32((N, K), seed=seed + 1, scale=0.02)
    b = synth.random_f32((N,), seed=seed + 2, scale=0.1)
    outs = {}
    for fuse in (None, "0"):
        kq_env(KQ_FUSE=fuse)
        kind = kq.kq_route(M, N, K, kq.KQ_W8_PER_CHANNEL)["kind"]
        assert kind == ("fused" if fuse is None else "gemv")
        outs[kind] = [host(_run("w8", xb, w, b, dt)) for dt in (torch.float32, torch.int32)]
        outs[kind].append(host_bf16_bits(_run("w8", xb, w, b, torch.bfloat16)))
        outs[kind].append(host(_run("w4", xb, w, b, torch.int32)))
    torch.cuda.synchronize()
    for u, v in zip(outs["fused"], outs["gemv"]):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


@pytest.mark.parametrize("fmt", ["w8", "w4"])
def test_fused_without_bias_and_f32_output_vector(fmt, kq_env):
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_FUSE=None)
    M, K, N = 64, 512, 64
    xb = synth.random_bf16((M, K), seed=31)
    w = synth.random_f32((N, K), seed=32, scale=0.02)
    y = _run(fmt, xb, w, None, torch.float32)
    torch.cuda.synchronize()
    y64, T = _exact(fmt, xb, w, None)
    check_f32(host(y), y64, T, f"fused no bias {fmt}")


def test_fused_route_log(kq_env, capfd):
    kq_env(KQ_LOG="1", KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_FUSE=None)
    xb = synth.random_bf16((100, 256), seed=41)
    w = synth.random_f32((48, 256), seed=42, scale=0.02)
    _run("w8", xb, w, None, torch.bfloat16)
    _run("w4", xb, w, None, torch.bfloat16)
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    assert "kq_w8a8_linear M=100 N=48 K=256" in err and "route=fused" in err
    assert "thin_fused_w8a8" in err and "thin_fused_w4a8" in err


# ---------------------------------------------------- GEMV quantizing x itself
# (M, K, N): 1-4 rows, one group to the 6144 limit, ragged column blocks
GEMV_XQ = [(1, 64, 16), (2, 320, 200), (3, 1088, 33), (4, 5120, 256), (1, 6144, 100),
           (4, 192, 17), (2, 3072, 1000)]


@pytest.mark.parametrize("lane", [None, "0"])
@pytest.mark.parametrize("fmt", ["w8", "w4"])
@pytest.mark.parametrize("M,K,N", GEMV_XQ)
def test_gemv_xq_matches_oracle(M, K, N, fmt, lane, kq_env):
    """M <= 4: the GEMV quantizes its rows in its prologue (route "fused");
    M <= 2 on the lane-per-column kernels (2-row, 32-column tile) unless
    KQ_GEMV_LANE=0, else the MFMA GEMV (4-row tile of 32 columns for int4
    weights, 16 for int8); codes
    (through the int32 outputs) and scales bit-exact."""
    if lane == "0" and not M <= 2:
        pytest.skip("the lever changes only GEMVs at M <= 2")
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_FUSE=None, KQ_GEMV_LANE=lane)
    r = kq.kq_route(M, N, K, _fmt_code(fmt))
    if M <= 2 and lane is None:
        assert (r["kind"], r["tile_m"], r["grid"]) == ("fused", 2, -(-N // 32))
    else:
        cols = 32 if fmt == "w4" else 16
        assert (r["kind"], r["tile_m"], r["grid"]) == ("fused", 4, -(-N // cols))
    seed = 7 * M + K + N
    dist = "student_t4" if (M + K) % 2 else "normal"
    xb = synth.random_bf16((M, K), seed=seed, dist=dist)
    w = synth.random_f32((N, K), seed=seed + 1, scale=0.02)
    b = synth.random_f32((N,), seed=seed + 2, scale=0.1)
    print(f"[fused] gemv xq {fmt} {M}x{K}x{N} {dist}", flush=True)
    _check_all(fmt, xb, w, b, f"gemv xq {fmt} {M}x{K}x{N}")


# M <= 2 on grids of at least one workgroup per CU (N >= 8161): the lane
# kernels keep a window of lines in flight per lane instead of issuing every
# line at once; one line window, a ragged line count, the K limit
GEMV_LANE_WIDE = [(1, 5120, 8192), (2, 1088, 8200), (1, 2112, 9000), (2, 6144, 8224)]


@pytest.mark.parametrize("fmt", ["w8", "w4"])
@pytest.mark.parametrize("M,K,N", GEMV_LANE_WIDE)
def test_gemv_lane_windowed_matches_oracle(M, K, N, fmt, kq_env):
    """The windowed lane kernels: int32 results and scales bit-exact,
    outputs within the oracle's bars."""
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_FUSE=None, KQ_GEMV_LANE=None)
    r = kq.kq_route(M, N, K, _fmt_code(fmt))
    assert (r["kind"], r["tile_m"]) == ("fused", 2) and r["grid"] >= 256
    seed = 11 * M + K + N
    xb = synth.random_bf16((M, K), seed=seed, dist="student_t4")
    w = synth.random_f32((N, K), seed=seed + 1, scale=0.02)
    b = synth.random_f32((N,), seed=seed + 2, scale=0.1)
    print(f"[fused] windowed lane {fmt} {M}x{K}x{N}", flush=True)
    _check_all(fmt, xb, w, b, f"windowed lane {fmt} {M}x{K}x{N}")


@pytest.mark.parametrize("fmt", ["w8", "w4"])
def test_gemv_xq_special_rows(fmt, kq_env):
    """A zero row, a row whose 127/amax overflows, a subnormal row and a huge
    outlier, quantized inside the GEMV."""
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_FUSE=None)
    M, K, N = 4, 3072, 48
    x = synth.bf16_bits_to_f32(synth.random_bf16((M, K), seed=23)).copy()
    x[0] = 0.0
    x[1] = 0.0
    x[1, 17] = 1e-38
    x[2] = 0.0
    x[2, ::7] = np.float32(2.0 ** -130)
    x[3, 5] = np.float32(3.0e38)
    xb = synth.to_bf16_bits(x)
    w = synth.random_f32((N, K), seed=24, scale=0.02)
    b = synth.random_f32((N,), seed=25, scale=0.1)
    assert kq.kq_route(M, N, K, _fmt_code(fmt))["kind"] == "fused"
    _check_all(fmt, xb, w, b, f"gemv xq special rows {fmt}")


@pytest.mark.parametrize("fmt", ["w8", "w4"])
@pytest.mark.parametrize("M,K,N", [(1, 5120, 512), (4, 1088, 200), (2, 3072, 1000),
                                   (1, 5120, 8192), (2, 3072, 8256)])
def test_gemv_xq_and_two_kernel_gemv_agree_bitwise(M, K, N, fmt, kq_env):
    """The same GEMV kernel, slices and sum order whether it quantizes x
    itself or reads the quantize kernel's codes: every output bit agrees,
    for int4 weights too."""
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None)
    seed = M + 3 * K + N
    xb = synth.random_bf16((M, K), seed=seed, dist="student_t4")
    w = synth.random_f32((N, K), seed=seed + 1, scale=0.02)
    b = synth.random_f32((N,), seed=seed + 2, scale=0.1)
    outs = {}
    for fuse in (None, "0"):
        kq_env(KQ_FUSE=fuse)
        kind = kq.kq_route(M, N, K, _fmt_code(fmt))["kind"]
        assert kind == ("fused" if fuse is None else "gemv")
        outs[kind] = [host(_run(fmt, xb, w, b, dt)) for dt in (torch.float32, torch.int32)]
        outs[kind].append(host_bf16_bits(_run(fmt, xb, w, b, torch.bfloat16)))
    torch.cuda.synchronize()
    for u, v in zip(outs["fused"], outs["gemv"]):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


@pytest.mark.parametrize("fmt", ["w8", "w4"])
def test_gemv_small_m_entry_quantizes_in_kernel(fmt, kq_env, capfd):
    """kq_gemv_small_m at M <= 4 runs the GEMV with the quantization in its
    prologue; KQ_FORCE_ROUTE=gemv gives the plain GEMV after the quantize
    kernel; every output bit agrees."""
    M, K, N = 3, 1024, 300
    xb = synth.random_bf16((M, K), seed=51, dist="student_t4")
    w = synth.random_f32((N, K), seed=52, scale=0.02)
    b = synth.random_f32((N,), seed=53, scale=0.1)
    x = dev_bf16(xb)
    if fmt == "w8":
        q8, sw = oracle.quantize_w8(w)
        args = (kq.KQ_W8_PER_CHANNEL, x, dev(q8), dev(sw), None)
    else:
        p, gs, gb, _ = oracle.quantize_w4(w)
        args = (kq.KQ_W4_AFFINE_G64, x, dev(p), dev(gs), dev(gb))
    outs = []
    for force in (None, "gemv"):
        kq_env(KQ_LOG="1", KQ_FORCE_ROUTE=force, KQ_TILE=None, KQ_FUSE=None)
        outs.append([host(kq.kq_gemv_small_m(*args, bias=dev(b), out_dtype=torch.float32)),
                     host(kq.kq_gemv_small_m(*args, out_dtype=torch.int32))])
    torch.cuda.synchronize()
    lines = [l for l in capfd.readouterr().err.splitlines() if "kq_gemv_small_m" in l]
    assert len(lines) == 4
    assert all("route=fused" in l and "gemv_xq_" in l for l in lines[:2])
    assert all("route=gemv" in l and "quant_act" in l for l in lines[2:])
    for u, v in zip(*outs):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))
    y64, T = _exact(fmt, xb, w, b)
    check_f32(outs[0][0], y64, T, f"kq_gemv_small_m {fmt}")
