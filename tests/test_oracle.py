"""CPU pins of the oracle: each check fixes the oracle to something other
than its own code (exact rational arithmetic, invariants the quantization
rule implies, integer arithmetic, closed forms, library routines)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import exact


def _bits(x32):
    return synth.to_bf16_bits(np.asarray(x32, np.float32))


# ------------------------------------------------- activation quantizer
@pytest.mark.parametrize("seed,shape,dist", [
    (1, (6, 37), "normal"), (2, (4, 64), "student_t4"), (3, (3, 129), "uniform"),
    (4, (5, 1), "normal"), (5, (2, 200), "normal"),
])
def test_quantize_act_matches_exact_bruteforce(seed, shape, dist):
    xb = synth.random_bf16(shape, seed, scale=3.0, dist=dist)
    x = oracle.bf16_bits_to_f32(xb)
    a, sx, _ = oracle.quantize_act(xb)
    for m in range(shape[0]):
        codes, scale = exact.quantize_row(x[m])
        assert list(a[m].astype(int)) == codes
        assert np.float32(sx[m]).view(np.uint32) == np.float32(scale).view(np.uint32)


def test_quantize_rounds_half_to_even_and_clamps():
    # amax = 127 gives inv = 1 exactly, so codes are rint(x) of the values.
    row = np.array([127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -127.0], np.float32)
    a, sx = oracle.quantize_rows_absmax(row[None, :])
    assert sx[0] == np.float32(1.0)
    assert list(a[0]) == [127, 0, 2, 2, 0, -2, -2, 126, -127]


def test_absmax_maps_to_127_and_codes_in_range():
    xb = synth.random_bf16((64, 300), 7, scale=5.0, dist="student_t4")
    x = oracle.bf16_bits_to_f32(xb)
    a, sx, _ = oracle.quantize_act(xb)
    assert a.min() >= -127 and a.max() <= 127
    idx = np.argmax(np.abs(x), axis=1)
    peak = a[np.arange(64), idx].astype(int)
    assert np.all(np.abs(peak) == 127)
    assert np.all(np.sign(peak) == np.sign(x[np.arange(64), idx]))


def test_dequantization_error_bound():
    # |x - sx*a| <= sx*(1/2 + 2^-15): 1/2 from rounding to a code, the rest
    # from fp32(127/amax)*fp32(amax/127) != 1 and the rounded product x*inv
    # (127*(2^-23 + 2^-24) < 2^-15).
    xb = synth.random_bf16((128, 513), 8, scale=0.7, dist="student_t4")
    x = oracle.bf16_bits_to_f32(xb).astype(np.float64)
    a, sx, _ = oracle.quantize_act(xb)
    err = np.abs(x - sx.astype(np.float64)[:, None] * a)
    assert np.all(err <= sx.astype(np.float64)[:, None] * (0.5 + 2.0 ** -15))
    # and the bound is nearly attained (codes really are nearest points)
    assert np.max(err / sx[:, None]) > 0.49


def test_sign_symmetry_and_power_of_two_scaling():
    xb = synth.random_bf16((16, 256), 9)
    x = oracle.bf16_bits_to_f32(xb)
    a, sx, _ = oracle.quantize_act(xb)
    an, sxn, _ = oracle.quantize_act(_bits(-x))
    assert np.array_equal(an, -a) and np.array_equal(sxn, sx)
    for k in (-20, -3, 5, 30):
        s = np.float32(2.0 ** k)
        ak, sxk, _ = oracle.quantize_act(_bits(x * s))
        assert np.array_equal(ak, a)
        assert np.array_equal(sxk, sx * s)


def test_zero_and_tiny_rows():
    x = np.zeros((3, 64), np.float32)
    x[1, 5] = np.float32(1e-38)     # 127/amax overflows fp32 -> zero row
    x[2, 7] = np.float32(1e-30)     # fine: a normal tiny row
    a, sx, A = oracle.quantize_act(_bits(x))
    assert sx[0] == 0 and not a[0].any() and A[0, 0] == 0
    assert sx[1] == 0 and not a[1].any()
    assert a[2, 7] == 127 and sx[2] > 0


def test_group_sums():
    xb = synth.random_bf16((5, 256), 10)
    a, _, A = oracle.quantize_act(xb)
    for m in range(5):
        for g in range(4):
            assert A[m, g] == sum(int(v) for v in a[m, 64 * g:64 * g + 64])
    _, _, none = oracle.quantize_act(synth.random_bf16((2, 100), 1))
    assert none is None


# ----------------------------------------------------------- int8 weights
def test_w8_matches_bruteforce_rows():
    w = synth.random_f32((5, 96), 11, scale=0.02)
    q8, sw = oracle.quantize_w8(w)
    for n in range(5):
        codes, scale = exact.quantize_row(w[n])
        assert list(q8[n].astype(int)) == codes and sw[n] == scale


# ----------------------------------------------------------- int4 weights
def test_w4_matches_bruteforce_groups():
    w = synth.random_f32((3, 192), 12, scale=0.02)
    w[1, 64:128] = np.float32(0.25)            # degenerate group: max == min
    packed, gs, gb, q = oracle.quantize_w4(w)
    for n in range(3):
        for g in range(3):
            codes, s, b = exact.quantize_group_w4(w[n, 64 * g:64 * g + 64])
            assert list(q[n, 64 * g:64 * g + 64].astype(int)) == codes
            assert gs[n, g].view(np.uint16) == np.float16(s).view(np.uint16)
            assert gb[n, g].view(np.uint16) == np.float16(b).view(np.uint16)
    assert gs[1, 1] == 0 and not q[1, 64:128].any()


def test_w4_pack_unpack_roundtrip_all_codes():
    lo, hi = np.meshgrid(np.arange(16), np.arange(16))
    q = np.stack([lo.ravel(), hi.ravel()], axis=1).reshape(1, -1).astype(np.uint8)
    p = oracle.pack_w4(q)
    assert p.shape == (1, 256)
    assert np.array_equal(np.sort(p[0]), np.arange(256, dtype=np.uint8))
    assert np.array_equal(oracle.unpack_w4(p), q)
    # low nibble = even k
    assert oracle.pack_w4(np.array([[3, 12]], np.uint8))[0, 0] == 0xC3


def test_w4_codes_span_grid_and_requantize():
    w = synth.random_f32((64, 512), 13, scale=0.02)
    packed, gs, gb, q = oracle.quantize_w4(w)
    n, k = w.shape
    qg = q.reshape(n, k // 64, 64)
    blocks = w.reshape(n, k // 64, 64).astype(np.float64)
    lo = blocks.min(2)
    s = gs.astype(np.float64)
    b = gb.astype(np.float64)
    # min element -> 0 when the offset rounding is under half a step;
    # max element -> 15 when the scale rounding (<= 2^-11 relative, times 15)
    # plus the offset rounding stays under half a step.
    off = np.abs(lo - b) / s
    assert np.all(qg.min(2)[off < 0.49] == 0)
    assert np.all(qg.max(2)[off + 15 * 2.0 ** -10 < 0.49] == 15)
    # re-quantizing the dequantized weights with the same scale/offset
    # returns the codes
    what = oracle.dequant_w4(q, gs, gb).astype(np.float32)
    g = np.arange(k) // 64
    inv = (np.float32(1) / gs.astype(np.float32))[:, g]
    t = (what - gb.astype(np.float32)[:, g]) * inv
    assert np.array_equal(np.clip(np.rint(t), 0, 15).astype(np.uint8), q)
    # dequantization error: nearest grid point up to the rounding slack
    err = np.abs(blocks - oracle.dequant_w4(q, gs, gb).reshape(n, k // 64, 64))
    assert np.all(err <= (0.5 * s + np.abs(lo - b) + 2.0 ** -9 * s * 15)[:, :, None])


def test_w4_exact_grid_is_recovered():
    rng = np.random.default_rng(14)
    n, k = 8, 256
    q = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
    q[:, 0::64] = 0
    q[:, 1::64] = 15
    e = rng.integers(6, 12, size=(n, k // 64))
    s = (2.0 ** -e).astype(np.float32)
    b = (np.float16(rng.standard_normal((n, k // 64)) * 0.05)).astype(np.float32)
    g = np.arange(k) // 64
    w = s[:, g] * q + b[:, g]                      # exact in fp32
    packed, gs, gb, q2 = oracle.quantize_w4(w)
    assert np.array_equal(q2, q)
    assert np.array_equal(gs.astype(np.float32), s)
    assert np.array_equal(gb.astype(np.float32), b)
    assert np.array_equal(oracle.dequant_w4(q, gs, gb), w.astype(np.float64))


# ------------------------------------------------------------ accumulators
def test_accumulators_against_python_integers():
    rng = np.random.default_rng(15)
    a = rng.integers(-127, 128, size=(3, 128)).astype(np.int8)
    q8 = rng.integers(-127, 128, size=(4, 128)).astype(np.int8)
    q4 = rng.integers(0, 16, size=(4, 128)).astype(np.uint8)
    acc = oracle.w8a8_acc(a, q8)
    P = oracle.w4a8_group_acc(a, q4)
    for m in range(3):
        for n in range(4):
            assert acc[m, n] == sum(int(a[m, k]) * int(q8[n, k]) for k in range(128))
            for g in range(2):
                assert P[g, m, n] == sum(int(a[m, k]) * int(q4[n, k])
                                         for k in range(64 * g, 64 * g + 64))


def test_accumulator_extremes_fit_int32():
    k = 65536
    a = np.full((1, k), -127, np.int8)
    q8 = np.full((2, k), 127, np.int8)
    q8[1] = -127
    acc = oracle.w8a8_acc(a, q8)
    assert acc[0, 0] == -127 * 127 * k and acc[0, 1] == 127 * 127 * k
    q4 = np.full((1, 128), 15, np.uint8)
    P = oracle.w4a8_group_acc(np.full((1, 128), 127, np.int8), q4)
    assert P[0, 0, 0] == 64 * 127 * 15


# ---------------------------------------------------------------- linears
def test_w8a8_integer_grid_reduces_to_integer_gemm():
    rng = np.random.default_rng(16)
    m, k, n = 9, 192, 11
    x = rng.integers(-127, 128, size=(m, k)).astype(np.float32)
    x[:, 3] = 127.0                                # amax 127 -> inv 1, sx 1
    w = rng.integers(-127, 128, size=(n, k)).astype(np.float32)
    w[:, 5] = -127.0
    bias = rng.standard_normal(n).astype(np.float32)
    q8, sw = oracle.quantize_w8(w)
    assert np.all(sw == 1) and np.array_equal(q8, w.astype(np.int8))
    y = oracle.w8a8_linear_exact(_bits(x), q8, sw, bias)
    ref = (x.astype(np.int64) @ w.astype(np.int64).T).astype(np.float64) + bias
    assert np.array_equal(y, ref)


def test_w4a8_exact_grid_reduces_to_fp64_gemm():
    rng = np.random.default_rng(17)
    m, k, n = 7, 256, 10
    q = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
    q[:, 0::64] = 0
    q[:, 1::64] = 15
    g = np.arange(k) // 64
    s = (2.0 ** -rng.integers(6, 10, size=(n, k // 64))).astype(np.float32)
    b = np.float16(rng.standard_normal((n, k // 64)) * 0.05).astype(np.float32)
    w = s[:, g] * q + b[:, g]
    x = rng.integers(-127, 128, size=(m, k)).astype(np.float32)
    x[:, 0] = -127.0
    bias = rng.standard_normal(n).astype(np.float32)
    _, gs, gb, q2 = oracle.quantize_w4(w)
    y = oracle.w4a8_linear_exact(_bits(x), q2, gs, gb, bias)
    ref = x.astype(np.float64) @ w.astype(np.float64).T + bias
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


def test_one_hot_rows_select_weight_columns():
    m, k, n = 4, 128, 6
    w = synth.random_f32((n, k), 18, scale=0.02)
    bias = synth.random_f32((n,), 19, scale=0.1)
    x = np.zeros((m, k), np.float32)
    cols = [0, 17, 64, 127]
    vals = [np.float32(3.0), np.float32(-0.125), np.float32(1e-3), np.float32(-70.0)]
    for i, (c, v) in enumerate(zip(cols, vals)):
        x[i, c] = v
    xb = _bits(x)
    xq = oracle.bf16_bits_to_f32(xb)
    q8, sw = oracle.quantize_w8(w)
    y = oracle.w8a8_linear_exact(xb, q8, sw, bias)
    _, gs, gb, q = oracle.quantize_w4(w)
    y4 = oracle.w4a8_linear_exact(xb, q, gs, gb, bias)
    what8 = oracle.dequant_w8(q8, sw)
    what4 = oracle.dequant_w4(q, gs, gb)
    for i, c in enumerate(cols):
        amax = abs(float(xq[i, c]))
        sx = float(np.float32(amax) / np.float32(127))
        sgn = float(np.sign(xq[i, c]))
        np.testing.assert_allclose(y[i], sgn * 127 * sx * what8[:, c] + bias, rtol=1e-14, atol=1e-14)
        np.testing.assert_allclose(y4[i], sgn * 127 * sx * what4[:, c] + bias, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("fmt", ["w8", "w4"])
def test_quantization_error_bound_against_fp64_gemm(fmt):
    # y_q - y = sum_k (x*(w_hat - w) - (x - x_hat)*w_hat), so
    # |y_q - y| <= sum_k |x||dw| + |dx||w_hat| (plus fp64 rounding).
    m, k, n = 32, 320, 48
    xb = synth.random_bf16((m, k), 20, dist="student_t4")
    x = oracle.bf16_bits_to_f32(xb).astype(np.float64)
    w = synth.random_f32((n, k), 21, scale=0.02)
    bias = synth.random_f32((n,), 22, scale=0.1)
    a, sx, _ = oracle.quantize_act(xb)
    xh = sx.astype(np.float64)[:, None] * a
    if fmt == "w8":
        q8, sw = oracle.quantize_w8(w)
        wh = oracle.dequant_w8(q8, sw)
        yq = oracle.w8a8_linear_exact(xb, q8, sw, bias)
    else:
        _, gs, gb, q = oracle.quantize_w4(w)
        wh = oracle.dequant_w4(q, gs, gb)
        yq = oracle.w4a8_linear_exact(xb, q, gs, gb, bias)
    y = x @ w.astype(np.float64).T + bias
    bound = np.abs(x) @ np.abs(wh - w).T + np.abs(x - xh) @ np.abs(wh).T
    assert np.all(np.abs(yq - y) <= bound * (1 + 1e-9) + 1e-12)
    # the bound is not vacuous: the quantized result is close
    rel = np.linalg.norm(yq - y) / np.linalg.norm(y)
    assert rel < (0.02 if fmt == "w8" else 0.1)


@pytest.mark.parametrize("fmt", ["w8", "w4"])
def test_factored_forms_match_plain_dequantized_product(fmt):
    # The oracle factors the scales out of exact integer sums; the plain
    # definition (float64 product of dequantized operands) must agree to
    # within that product's own rounding, K * 2^-52 * sum |x_hat||w_hat|.
    m, k, n = 24, 448, 40
    xb = synth.random_bf16((m, k), 29, dist="student_t4")
    w = synth.random_f32((n, k), 30, scale=0.02)
    bias = synth.random_f32((n,), 31, scale=0.1)
    a, sx, _ = oracle.quantize_act(xb)
    xh = sx.astype(np.float64)[:, None] * a
    if fmt == "w8":
        q8, sw = oracle.quantize_w8(w)
        wh = oracle.dequant_w8(q8, sw)
        y = oracle.w8a8_linear_exact(xb, q8, sw, bias)
    else:
        _, gs, gb, q = oracle.quantize_w4(w)
        wh = oracle.dequant_w4(q, gs, gb)
        y = oracle.w4a8_linear_exact(xb, q, gs, gb, bias)
    plain = oracle.linear_dequantized_fp64(xb, wh, bias)
    bound = k * 2.0 ** -52 * (np.abs(xh) @ np.abs(wh).T + np.abs(bias))
    assert np.all(np.abs(y - plain) <= bound)


def test_exact_zero_results_are_zero():
    # rows whose int8 products cancel exactly give exactly the bias
    k = 128
    x = np.zeros((1, k), np.float32)
    x[0, 0], x[0, 1] = 1.0, -1.0
    w = np.zeros((2, k), np.float32)
    w[:, 0] = w[:, 1] = 0.5
    w[1, 5] = 1.0
    q8, sw = oracle.quantize_w8(w)
    y = oracle.w8a8_linear_exact(_bits(x), q8, sw)
    assert np.all(y == 0.0)


def test_transposed_weight_is_caught():
    # a plausible slip (using w instead of w^T) must break the fp64 check
    m, k = 16, 64
    xb = synth.random_bf16((m, k), 23)
    w = synth.random_f32((k, k), 24, scale=0.02)
    q8, sw = oracle.quantize_w8(w)
    y = oracle.w8a8_linear_exact(xb, q8, sw)
    ref = oracle.bf16_bits_to_f32(xb).astype(np.float64) @ w.T.astype(np.float64)
    wrong = oracle.bf16_bits_to_f32(xb).astype(np.float64) @ w.astype(np.float64)
    assert np.linalg.norm(y - ref) < 0.1 * np.linalg.norm(y - wrong)


def test_magnitudes_bound_results():
    m, k, n = 8, 256, 16
    xb = synth.random_bf16((m, k), 25)
    w = synth.random_f32((n, k), 26, scale=0.02)
    bias = synth.random_f32((n,), 27, scale=0.1)
    q8, sw = oracle.quantize_w8(w)
    y8 = oracle.w8a8_linear_exact(xb, q8, sw, bias)
    assert np.all(np.abs(y8) <= oracle.w8a8_magnitude(xb, q8, sw, bias) * (1 + 1e-12))
    _, gs, gb, q = oracle.quantize_w4(w)
    y4 = oracle.w4a8_linear_exact(xb, q, gs, gb, bias)
    T4 = oracle.w4a8_magnitude(xb, q, gs, gb, bias)
    assert np.all(np.abs(y4) <= T4 * (1 + 1e-12))


# ------------------------------------------------------------ rounding
def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(28)
    v = rng.standard_normal(200000).astype(np.float32) * np.float32(1e3)
    u = v.view(np.uint32)
    u[:1000] = (u[:1000] & 0xFFFF0000) | 0x8000      # exact ties
    u[1000:2000] = (u[1000:2000] & 0xFFFF0000) | 0x7FFF
    v = u.view(np.float32)
    ours = oracle.round_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_ulp():
    bits = synth.to_bf16_bits(np.array([1.0, -1.0, 3.0, 1e-3], np.float32))
    np.testing.assert_array_equal(oracle.bf16_ulp(bits),
                                  [2 ** -7, 2 ** -7, 2 ** -6, 2.0 ** -17])


# ------------------------------------------------------- golden fixture
# tests/golden/small_cases.json is written by tests/golden/make_golden.py
# from oracle/ and synth/ only.  The first test catches any drift of the
# oracle's arithmetic; the second checks the fixture's hand-derivable rows
# against their closed forms, independently of the oracle.
def _golden():
    import importlib.util
    import json
    import os

    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(here, "make_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    with open(os.path.join(here, "small_cases.json")) as f:
        return mod, json.load(f)


def test_golden_fixture_is_reproduced_by_oracle(tmp_path, monkeypatch):
    mod, stored = _golden()
    monkeypatch.setattr(mod, "OUT", str(tmp_path / "again.json"))
    mod.main()
    import json

    with open(tmp_path / "again.json") as f:
        assert json.load(f) == stored


def test_golden_fixture_closed_forms():
    _, d = _golden()
    M, K, N = d["shape"]["M"], d["shape"]["K"], d["shape"]["N"]
    codes = np.array(d["act_codes"]).reshape(M, K)
    scale_bits = [int(h, 16) for h in d["act_scale_f32_bits"]]
    # row 3: amax = 127 gives inv = 127/127 = 1 and scale 127/127 = 1, so the
    # codes are rint(x) with ties to even: 2.5 -> 2, -2.5 -> -2, 3.5 -> 4,
    # +-0.5 -> 0, 1.5 -> 2
    assert scale_bits[3] == 0x3F800000
    assert codes[3, :7].tolist() == [127, 2, -2, 4, 0, 0, 2]
    assert not codes[3, 7:].any()
    # rows 1 (zeros) and 2 (bf16 subnormals: 127/amax > FLT_MAX): scale 0, codes 0
    assert scale_bits[1] == 0 and scale_bits[2] == 0
    assert not codes[1].any() and not codes[2].any()
    # every other row reaches +-127 at its absmax element
    for m in (0, 4, 5):
        assert np.abs(codes[m]).max() == 127
    # group sums are the sums of the codes
    gs = np.array(d["act_group_sums"]).reshape(M, K // 64)
    assert np.array_equal(gs, codes.reshape(M, K // 64, 64).sum(axis=2))
    # int8 weights: the all-zero channel 1 gets scale 0 and zero codes
    q8 = np.array(d["w8_codes"]).reshape(N, K)
    sw_bits = [int(h, 16) for h in d["w8_scale_f32_bits"]]
    assert sw_bits[1] == 0 and not q8[1].any()
    # int4: channel 2, group 1 is constant 0.0123, so its scale is 0, its
    # offset fp16(0.0123) and its codes 0
    gs4 = [int(h, 16) for h in d["w4_scale_f16_bits"]]
    gb4 = [int(h, 16) for h in d["w4_offset_f16_bits"]]
    G = K // 64
    assert gs4[2 * G + 1] == 0
    assert gb4[2 * G + 1] == int(np.array(0.0123, np.float16).view(np.uint16))
    packed = np.array(d["w4_packed"]).reshape(N, K // 2)
    assert not packed[2, 32:].any()
    # int32 accumulators are the exact integer products of the stored codes
    acc = np.array(d["w8a8_acc"]).reshape(M, N)
    assert np.array_equal(acc, codes.astype(np.int64) @ q8.astype(np.int64).T)


# ------------------------------------------------ gated residual epilogue
def test_gated_residual_identities():
    """No residual and no gate is the linear; gate 1 and residual 0 too;
    gate 0 leaves the residual exactly."""
    rng = np.random.default_rng(31)
    y = rng.standard_normal((6, 5))
    assert np.array_equal(oracle.gated_residual_exact(y), y)
    ones = np.ones((6, 5), np.float32)
    zeros_r = _bits(np.zeros((6, 5), np.float32))
    assert np.array_equal(oracle.gated_residual_exact(y, zeros_r, ones, 1), y)
    r = _bits(rng.standard_normal((6, 5)).astype(np.float32))
    out = oracle.gated_residual_exact(y, r, np.zeros((3, 5), np.float32), 2)
    assert np.array_equal(out, synth.bf16_bits_to_f32(r).astype(np.float64))


def test_gated_residual_integer_grid_is_exact_arithmetic():
    """Integer-grid linear (sx = sw = 1, so y is an exact integer GEMM plus
    an integer bias), power-of-two gates shared by 3 rows each, and integer
    residuals: the result is plain integer/dyadic arithmetic."""
    rng = np.random.default_rng(32)
    m, k, n, L = 9, 128, 7, 3
    x = rng.integers(-127, 128, size=(m, k)).astype(np.float32)
    x[:, 0] = 127.0
    w = rng.integers(-127, 128, size=(n, k)).astype(np.float32)
    w[:, 1] = 127.0
    bias = rng.integers(-50, 50, size=n).astype(np.float32)
    gate = (2.0 ** rng.integers(-3, 4, size=(m // L, n))).astype(np.float32)
    gate[0, 0] = -0.5
    r = rng.integers(-100, 100, size=(m, n)).astype(np.float32)
    q8, sw = oracle.quantize_w8(w)
    y = oracle.w8a8_linear_exact(_bits(x), q8, sw, bias)
    out = oracle.gated_residual_exact(y, _bits(r), gate, L)
    lin = x.astype(np.int64) @ w.astype(np.int64).T + bias.astype(np.int64)
    g = np.repeat(gate.astype(np.float64), L, axis=0)
    ref = r.astype(np.float64) + g * lin.astype(np.float64)   # exact: dyadic, < 2^53
    assert np.array_equal(out, ref)
    T = oracle.gated_magnitude(oracle.w8a8_magnitude(_bits(x), q8, sw, bias), _bits(r), gate, L)
    assert np.all(T >= np.abs(out) - 1e-9)


# ------------------------------------- tolerance scales, pinned on both sides
# The term magnitudes T set every fp32 bar (1e-5 * max(|y|, T)) and the bf16
# cancellation fallback of the GPU parity tests, so an inflated T would
# loosen every bar.  Each is pinned from above as well as from below: exact
# equality with Python-integer / rational sums on integer grids, an identity
# with the oracle's independently pinned result, and elementwise
# triangle-inequality bounds on random inputs small enough (tiny token
# scales) that a missing scale factor cannot hide under them.
def _grid_w4(rng, n, k):
    """int4 weights that are exactly gs*q + gb (gs a power of two, gb fp16)."""
    q = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
    q[:, 0::64] = 0
    q[:, 1::64] = 15
    g = np.arange(k) // 64
    s = (2.0 ** -rng.integers(6, 10, size=(n, k // 64))).astype(np.float32)
    b = np.float16(rng.standard_normal((n, k // 64)) * 0.05).astype(np.float32)
    return s[:, g] * q + b[:, g], q, s, b


def test_w8a8_magnitude_equals_integer_terms_on_grid():
    # sx = sw = 1 on the integer grid: T = |acc| + |bias| in Python integers
    rng = np.random.default_rng(33)
    m, k, n = 5, 192, 7
    x = rng.integers(-127, 128, size=(m, k)).astype(np.float32)
    x[:, 2] = -127.0
    w = rng.integers(-127, 128, size=(n, k)).astype(np.float32)
    w[:, 7] = 127.0
    bias = rng.integers(-5000, 5000, size=n).astype(np.float32)
    q8, sw = oracle.quantize_w8(w)
    T = oracle.w8a8_magnitude(_bits(x), q8, sw, bias)
    for i in range(m):
        for j in range(n):
            acc = sum(int(x[i, kk]) * int(w[j, kk]) for kk in range(k))
            assert T[i, j] == abs(acc) + abs(int(bias[j]))


def test_w4a8_magnitude_equals_rational_terms_on_grid():
    # x on the integer grid (sx = 1) and w = gs*q + gb exactly: T is the
    # rational sum over groups of |gs*P| + |gb*A| plus |bias|, every term a
    # dyadic number, so the fp64 value must be exact
    rng = np.random.default_rng(34)
    m, k, n = 4, 256, 5
    w, q, s, b = _grid_w4(rng, n, k)
    x = rng.integers(-127, 128, size=(m, k)).astype(np.float32)
    x[:, 0] = 127.0
    bias = np.float32(rng.standard_normal(n) * 0.1)
    _, gs, gb, q2 = oracle.quantize_w4(w)
    assert np.array_equal(q2, q)
    T = oracle.w4a8_magnitude(_bits(x), q2, gs, gb, bias)
    for i in range(m):
        for j in range(n):
            want = abs(Fraction(float(bias[j])))
            for g in range(k // 64):
                ks = range(64 * g, 64 * g + 64)
                P = sum(int(x[i, kk]) * int(q[j, kk]) for kk in ks)
                A = sum(int(x[i, kk]) for kk in ks)
                want += abs(Fraction(float(s[j, g])) * P) + abs(Fraction(float(b[j, g])) * A)
            assert Fraction(float(T[i, j])) == want


def test_w8a8_magnitude_is_the_terms_of_the_result():
    # y = sx*sw*acc + bias, so T = |sx*sw*acc| + |bias| = |y - bias| + |bias|
    # (y pinned independently above), to fp64 rounding
    m, k, n = 12, 320, 20
    xb = synth.random_bf16((m, k), 35, scale=0.01, dist="student_t4")
    w = synth.random_f32((n, k), 36, scale=0.02)
    bias = synth.random_f32((n,), 37, scale=0.1)
    q8, sw = oracle.quantize_w8(w)
    y = oracle.w8a8_linear_exact(xb, q8, sw, bias)
    T = oracle.w8a8_magnitude(xb, q8, sw, bias)
    want = np.abs(y - bias.astype(np.float64)) + np.abs(bias.astype(np.float64))
    assert np.all(np.abs(T - want) <= 4 * 2.0 ** -52 * want)


@pytest.mark.parametrize("fmt", ["w8", "w4"])
def test_magnitudes_between_result_and_elementwise_sums(fmt):
    # From below: T >= |y - bias| + |bias|.  From above, by the triangle
    # inequality on the dequantized operands: |sx*sw*acc| <= sum_k
    # |x_hat||w_hat|; |gs*P| + |gb*A| <= sum_{k in g} |a|(|gs*q| + |gb|).
    # The activations are small (sx ~ 3e-4), so a magnitude that lost its
    # token scale, or was scaled up, lands above the bound.
    m, k, n = 10, 384, 24
    xb = synth.random_bf16((m, k), 38, scale=0.01)
    w = synth.random_f32((n, k), 39, scale=0.02)
    bias = synth.random_f32((n,), 40, scale=0.1)
    a, sx, _ = oracle.quantize_act(xb)
    b64 = np.abs(bias.astype(np.float64))
    if fmt == "w8":
        q8, sw = oracle.quantize_w8(w)
        y = oracle.w8a8_linear_exact(xb, q8, sw, bias)
        T = oracle.w8a8_magnitude(xb, q8, sw, bias)
        xh = sx.astype(np.float64)[:, None] * a.astype(np.float64)
        upper = np.abs(xh) @ np.abs(oracle.dequant_w8(q8, sw)).T + b64
    else:
        _, gs, gb, q = oracle.quantize_w4(w)
        y = oracle.w4a8_linear_exact(xb, q, gs, gb, bias)
        T = oracle.w4a8_magnitude(xb, q, gs, gb, bias)
        g = np.arange(k) // 64
        wabs = (np.abs(gs.astype(np.float64)[:, g] * q) + np.abs(gb.astype(np.float64))[:, g])
        upper = sx.astype(np.float64)[:, None] * (np.abs(a.astype(np.float64)) @ wabs.T) + b64
    lower = np.abs(y - bias.astype(np.float64)) + b64
    assert np.all(T >= lower * (1 - 1e-12))
    assert np.all(T <= upper * (1 + 1e-12))
    assert np.max(upper / T) < 200       # the upper bound is not vacuous


def test_gated_magnitude_equals_integer_terms_on_grid():
    # integer grid, integer residuals, power-of-two gates shared by 2 rows:
    # T_gated = |r| + |g| * (|acc| + |bias|) in Python integers and dyadics
    rng = np.random.default_rng(41)
    m, k, n, L = 6, 128, 5, 2
    x = rng.integers(-127, 128, size=(m, k)).astype(np.float32)
    x[:, 1] = 127.0
    w = rng.integers(-127, 128, size=(n, k)).astype(np.float32)
    w[:, 4] = -127.0
    bias = rng.integers(-300, 300, size=n).astype(np.float32)
    gate = (2.0 ** rng.integers(-3, 4, size=(m // L, n))).astype(np.float32)
    gate[1, 2] = -4.0
    r = rng.integers(-200, 200, size=(m, n)).astype(np.float32)
    q8, sw = oracle.quantize_w8(w)
    T = oracle.gated_magnitude(oracle.w8a8_magnitude(_bits(x), q8, sw, bias), _bits(r), gate, L)
    for i in range(m):
        for j in range(n):
            acc = sum(int(x[i, kk]) * int(w[j, kk]) for kk in range(k))
            want = abs(int(r[i, j])) + abs(Fraction(float(gate[i // L, j]))) * (abs(acc) + abs(int(bias[j])))
            assert Fraction(float(T[i, j])) == want


def test_gated_magnitude_between_result_and_elementwise_sums():
    m, k, n, L = 8, 256, 12, 3
    xb = synth.random_bf16((m, k), 42, scale=0.01)
    w = synth.random_f32((n, k), 43, scale=0.02)
    bias = synth.random_f32((n,), 44, scale=0.1)
    gate = synth.random_f32((-(-m // L), n), 45, scale=0.5)
    r = synth.random_bf16((m, n), 46)
    q8, sw = oracle.quantize_w8(w)
    y = oracle.w8a8_linear_exact(xb, q8, sw, bias)
    out = oracle.gated_residual_exact(y, r, gate, L)
    T = oracle.gated_magnitude(oracle.w8a8_magnitude(xb, q8, sw, bias), r, gate, L)
    a, sx, _ = oracle.quantize_act(xb)
    xh = sx.astype(np.float64)[:, None] * a.astype(np.float64)
    lin_upper = np.abs(xh) @ np.abs(oracle.dequant_w8(q8, sw)).T + np.abs(bias.astype(np.float64))
    rows = np.arange(m) // L
    upper = (np.abs(oracle.bf16_bits_to_f32(r).astype(np.float64))
             + np.abs(gate.astype(np.float64))[rows] * lin_upper)
    assert np.all(T >= np.abs(out) * (1 - 1e-12))
    assert np.all(T <= upper * (1 + 1e-12))
