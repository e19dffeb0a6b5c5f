"""Helpers of the GPU parity tests: host<->device marshalling of seeded
inputs and the comparison rules against the oracle.

Bars (the GPU path against the oracle on identical inputs):
  - int8 codes, scales, group sums, int4 packing, int32 accumulators:
    bit-exact;
  - fp32 outputs: |y - y32| <= 1e-5 * max(|y32|, T), where y32 is the
    oracle's exact result rounded once to fp32 and T the term magnitude
    (|sx*sw*acc| + |bias| for int8 weights, sx*sum_g(|gs*P| + |gb*A|) +
    |bias| for int4), the scale of an fp32 evaluation's rounding error;
  - bf16 outputs: within 1 bf16 ulp of the oracle's bf16 result, except
    where |y32| < 2^-8 * T (cancellation: the fp32 error alone can exceed
    an ulp of the tiny result) where the fp32 rule plus one ulp applies.
"""
import numpy as np
import torch

import oracle


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def host_bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.float16:
        return t.detach().view(torch.int16).cpu().numpy().view(np.float16)
    return t.detach().cpu().numpy()


def check_f32(y_gpu: np.ndarray, y64: np.ndarray, T: np.ndarray, what: str = "") -> float:
    y32 = oracle.round_f32(y64).astype(np.float64)
    err = np.abs(np.asarray(y_gpu, np.float64) - y32)
    tol = 1e-5 * np.maximum(np.abs(y32), T)
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} fp32 elements out of tolerance; first {tuple(i)}: "
                             f"gpu {y_gpu[tuple(i)]!r} oracle {y32[tuple(i)]!r} T {T[tuple(i)]!r}")
    return float(np.max(err / np.maximum(np.maximum(np.abs(y32), T), 1e-300)))


def check_bf16(y_bits: np.ndarray, y64: np.ndarray, T: np.ndarray, what: str = "") -> int:
    y32 = oracle.round_f32(y64)
    r_bits = oracle.round_bf16_bits(y32)
    g = oracle.bf16_bits_to_f32(y_bits).astype(np.float64)
    r = oracle.bf16_bits_to_f32(r_bits).astype(np.float64)
    ulp = oracle.bf16_ulp(r_bits)
    ok = np.abs(g - r) <= ulp
    cancel = np.abs(y32.astype(np.float64)) < 2.0 ** -8 * T
    ok |= cancel & (np.abs(g - y32) <= ulp + 1e-5 * T)
    if not ok.all():
        i = np.argwhere(~ok)[0]
        raise AssertionError(f"{what}: {(~ok).sum()} bf16 elements beyond 1 ulp; first {tuple(i)}: "
                             f"gpu {g[tuple(i)]!r} oracle {r[tuple(i)]!r}")
    return int(np.sum(g != r))
