"""CPU oracle of the INT8 quantized linear and the INT8 attention -- TEST
INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy implementation of what the GPU path
computes.  Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import it; the product path (the HIP library and its Python
binding) never does, and shares no code with it.

Every function pinned by the CPU test suite (see the headers of
kq_oracle.py and sage_oracle.py for which pin covers which function).
"""
from . import sage_oracle as sage  # noqa: F401
from .kq_oracle import (  # noqa: F401
    F32_MAX,
    quantize_rows_absmax,
    quantize_act,
    quantize_w8,
    quantize_w4,
    pack_w4,
    unpack_w4,
    dequant_w8,
    dequant_w4,
    w8a8_acc,
    w4a8_group_acc,
    w8a8_linear_exact,
    w4a8_linear_exact,
    linear_dequantized_fp64,
    w8a8_magnitude,
    w4a8_magnitude,
    gated_residual_exact,
    gated_magnitude,
    round_f32,
    round_bf16_bits,
    bf16_bits_to_f32,
    bf16_ulp,
)
