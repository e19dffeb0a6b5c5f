"""Writes tests/golden/small_cases.json: small, fixed inputs and the oracle's
results for them.  Calls only oracle/ and synth/ (the seeded input
generators); nothing here comes from the HIP path.

What the fixture pins, and from where:
  - per-token int8 activation codes, fp32 scales and 64-wide group sums
    ("qlip-mlx" README, w8a8_linear bullet: per-token activation
    quantization inside the kernel), including an all-zero row, a row of
    bf16 subnormals (127/amax overflows fp32, so the row quantizes to zero),
    a row with amax 127 whose codes are ties (round half to even), an
    outlier row and a row whose absmax is negative;
  - int8 per-output-channel weights ("qlip-mlx" README, "Quick start":
    quantize_weight_int8) and affine 4-bit g64 weights with fp16 scale and
    offset (MLX pull request 4722, serving test, affine 4-bit g64),
    including an all-zero weight row and a constant 64-group;
  - the int32 accumulators, the per-group int4 products and the linears'
    fp32 and bf16 outputs, each the exact dequantized product plus bias
    rounded once ("qlip-mlx" README, w8a8_linear bullet; mlx-kquant pull
    request 89 commit list: one output rounding).

Run from the repository root:  python3 tests/golden/make_golden.py
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "small_cases.json")
M, K, N = 6, 128, 4


def activation_bits() -> np.ndarray:
    x = synth.bf16_bits_to_f32(synth.random_bf16((M, K), seed=11)).copy()
    x[1, :] = 0.0                                   # all zero
    x[2, :] = 0.0
    x[2, 0:5] = np.float32(2.0 ** -133) * np.arange(1, 6, dtype=np.float32)  # subnormal: 127/amax overflows
    x[3, :] = 0.0                                    # amax 127: inv = 1, codes = rint(x)
    x[3, 0:7] = np.array([127.0, 2.5, -2.5, 3.5, 0.5, -0.5, 1.5], np.float32)  # ties to even
    x[4, 7] = np.float32(30.0) * abs(x[4, 7]) + np.float32(5.0)  # outlier
    x[5, :] = -np.abs(x[5, :])                       # absmax is a negative value
    return synth.to_bf16_bits(x)


def weights_f32() -> np.ndarray:
    w = synth.random_f32((N, K), seed=12, scale=0.02)
    w[1, :] = 0.0                                    # zero channel / zero groups
    w[2, 64:128] = np.float32(0.0123)                # constant 64-group (scale 0)
    return w


def hexbits(a: np.ndarray, dtype) -> list:
    return [format(int(v), "x") for v in np.ascontiguousarray(a).view(dtype).ravel()]


def main() -> None:
    xb = activation_bits()
    w = weights_f32()
    bias = synth.random_f32((N,), seed=13, scale=0.1)
    a, sx, gsum = oracle.quantize_act(xb)
    q8, sw = oracle.quantize_w8(w)
    p4, gs, gb, q4 = oracle.quantize_w4(w)
    acc = oracle.w8a8_acc(a, q8)
    P = oracle.w4a8_group_acc(a, q4)
    y8 = oracle.w8a8_linear_exact(xb, q8, sw, bias)
    y4 = oracle.w4a8_linear_exact(xb, q4, gs, gb, bias)
    y8_32 = oracle.round_f32(y8)
    y4_32 = oracle.round_f32(y4)
    doc = {
        "about": "inputs and oracle results for the small cases; written by "
                 "tests/golden/make_golden.py from oracle/ and synth/ only",
        "shape": {"M": M, "K": K, "N": N},
        "x_bf16_bits": hexbits(xb, np.uint16),
        "w_f32_bits": hexbits(w, np.uint32),
        "bias_f32_bits": hexbits(bias, np.uint32),
        "act_codes": a.astype(int).ravel().tolist(),
        "act_scale_f32_bits": hexbits(sx, np.uint32),
        "act_group_sums": gsum.astype(int).ravel().tolist(),
        "w8_codes": q8.astype(int).ravel().tolist(),
        "w8_scale_f32_bits": hexbits(sw, np.uint32),
        "w4_packed": p4.astype(int).ravel().tolist(),
        "w4_scale_f16_bits": hexbits(gs, np.uint16),
        "w4_offset_f16_bits": hexbits(gb, np.uint16),
        "w8a8_acc": acc.astype(np.int64).ravel().tolist(),
        "w4a8_group_products_gmn": P.astype(np.int64).ravel().tolist(),
        "w8a8_y_f32_bits": hexbits(y8_32, np.uint32),
        "w8a8_y_bf16_bits": hexbits(oracle.round_bf16_bits(y8_32), np.uint16),
        "w4a8_y_f32_bits": hexbits(y4_32, np.uint32),
        "w4a8_y_bf16_bits": hexbits(oracle.round_bf16_bits(y4_32), np.uint16),
    }
    with open(OUT, "w") as f:
        json.dump(doc, f, indent=0, separators=(",", ":"))
        f.write("\n")
    print(f"wrote {OUT}")


if __name__ == "__main__":
    main()
