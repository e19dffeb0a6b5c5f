"""Seeded synthetic inputs for the INT8 quantized linear and the INT8
attention.

Shared by the CPU oracle's tests, the GPU parity tests and the benchmark.  It
holds no step of the method: it only draws activations, fp32 weights and
biases with the shapes and value distributions of diffusion-transformer
linear layers, and casts the activations to bf16.

Shapes and distributions (the workloads the pages measure on are DiT models;
their weights and prompts are not available, so these draws stand in):
  - "qlip-mlx" README, "Quick start": a bare-tensor W8A8 check at
    14040x5120 @ 5120x5120 bf16 shapes; W8A8/W4A8 linears replace DiT
    linear layers.
  - MLX pull request 4722, speed tables: prefill at M=2048, q/o 4096x4096,
    gate/up 4096x12288, down 12288x4096, thin-N 5120x48, decode at M=1.
  - "MiniMax-H3-Image M5 affine Q8 acceleration": about 16.5k token rows per
    4K image.

Recipe (seed 0 unless stated): numpy SeedSequence(seed).spawn(4) gives four
independent streams for (outlier channel indices, x, W, bias).  x is drawn in
fp32 (normal, or Student-t with 4 degrees of freedom), a fixed set of
"outlier" input channels (chosen uniformly without replacement) is multiplied
by a factor before the cast, then x is cast to bf16 with round-to-nearest-even
(torch).  W ~ N(0, 0.02) fp32 [N,K]; bias ~ N(0, 0.1) fp32 [N].
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    fmt: str            # "w8" (int8 per channel) or "w4" (int4 affine g64)
    out: str            # "f32" or "bf16"
    x_dist: str = "normal"   # "normal" or "student_t4"
    outliers: int = 0   # number of outlier input channels
    outlier_scale: float = 1.0

    @property
    def ops(self) -> int:
        """Integer operations of the matrix product (a multiply-add is two)."""
        return 2 * self.M * self.N * self.K


WORKLOADS = {
    w.name: w
    for w in [
        # Small correctness shape: 4 outlier channels x20, fp32 output.
        Workload("w8a8_64x512x512", 64, 512, 512, "w8", "f32",
                 outliers=4, outlier_scale=20.0),
        # DiT attention projection at 1024px (64x64 latent patches = 4096
        # tokens): 1% of the 3072 channels (31) are outliers x30.
        Workload("dit_proj_w8a8_4096x3072x3072", 4096, 3072, 3072, "w8", "bf16",
                 outliers=31, outlier_scale=30.0),
        # DiT MLP pair with int4 weights (gate/up then down).
        Workload("dit_mlp_up_w4a8_2048x4096x12288", 2048, 4096, 12288, "w4", "bf16"),
        Workload("dit_mlp_down_w4a8_2048x12288x4096", 2048, 12288, 4096, "w4", "bf16"),
        # Large-sequence linear (2048px / 4K scale), heavy-tailed activations.
        Workload("dit_4k_w8a8_16384x3072x12288", 16384, 3072, 12288, "w8", "bf16",
                 x_dist="student_t4"),
        Workload("thin_n_w8a8_2048x5120x48", 2048, 5120, 48, "w8", "bf16",
                 x_dist="student_t4"),
        # A short sequence through a long-K projection (128 tokens, e.g. a
        # text-conditioning stream, through an MLP down-projection): 24
        # output tiles of 128x128, so the GEMM splits K.
        Workload("short_seq_w8a8_128x12288x3072", 128, 12288, 3072, "w8", "bf16"),
        # adaLN modulation of a DiT block: the conditioning vector of each
        # sample (batch 2) to the six shift/scale/gate vectors, 6 x 3072.
        Workload("dit_modulation_w8a8_2x3072x18432", 2, 3072, 18432, "w8", "bf16"),
        # Small-batch GEMV with int4 weights.
        Workload("gemv_w4a8_m1_5120x13824", 1, 5120, 13824, "w4", "bf16"),
        Workload("gemv_w4a8_m4_5120x13824", 4, 5120, 13824, "w4", "bf16"),
        Workload("gemv_w4a8_m16_5120x13824", 16, 5120, 13824, "w4", "bf16"),
    ]
}

# The workload the headline throughput figure is quoted on: the largest
# single-GPU configuration (16384 tokens x 3072 -> 12288, int8 weights).
HEADLINE = "dit_4k_w8a8_16384x3072x12288"


def _streams(seed: int):
    ss = np.random.SeedSequence(seed).spawn(4)
    return [np.random.default_rng(s) for s in ss]


def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest even, via torch) and return the raw
    16-bit patterns as uint16."""
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def activations(w: Workload, seed: int = 0, rows: Optional[int] = None) -> np.ndarray:
    """bf16 bit patterns [rows or M, K] of the workload's activations.

    Drawing `rows` < M gives the first `rows` rows of the same full draw
    (the generator draws row by row in the same order)."""
    r_idx, r_x, _, _ = _streams(seed)
    m = w.M if rows is None else rows
    if w.x_dist == "normal":
        x = r_x.standard_normal((m, w.K), dtype=np.float32)
    elif w.x_dist == "student_t4":
        x = r_x.standard_t(4.0, size=(m, w.K)).astype(np.float32)
    else:
        raise ValueError(w.x_dist)
    if w.outliers:
        cols = r_idx.choice(w.K, size=w.outliers, replace=False)
        x[:, cols] *= np.float32(w.outlier_scale)
    return to_bf16_bits(x)


def weights(w: Workload, seed: int = 0) -> np.ndarray:
    """fp32 weights [N, K] ~ N(0, 0.02)."""
    _, _, r_w, _ = _streams(seed)
    return (r_w.standard_normal((w.N, w.K), dtype=np.float32) * np.float32(0.02))


def bias(w: Workload, seed: int = 0) -> np.ndarray:
    """fp32 bias [N] ~ N(0, 0.1)."""
    _, _, _, r_b = _streams(seed)
    return (r_b.standard_normal(w.N, dtype=np.float32) * np.float32(0.1))


def random_bf16(shape, seed: int, scale: float = 1.0, dist: str = "normal") -> np.ndarray:
    """Generic seeded bf16 activations for parity sweeps."""
    rng = np.random.default_rng(seed)
    if dist == "normal":
        x = rng.standard_normal(shape, dtype=np.float32)
    elif dist == "student_t4":
        x = rng.standard_t(4.0, size=shape).astype(np.float32)
    elif dist == "uniform":
        x = rng.uniform(-1.0, 1.0, size=shape).astype(np.float32)
    else:
        raise ValueError(dist)
    return to_bf16_bits(x * np.float32(scale))


def random_f32(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)


# ------------------------------------------------------------------ attention
# "qlip-mlx" README, "Quick start": the bare-tensor attention check runs 40
# heads x 14040 tokens at head dim 128 (q/k/v [B, heads, L, 128]); DiT
# attention is bidirectional.  The draws stand in for a DiT's q/k/v after
# its q/k normalization: q and v ~ N(0, 1); k ~ N(0, 1) plus a per-(head,
# channel) offset ~ N(0, key_bias^2) shared by all tokens, the channel bias
# of DiT keys that the SageAttention smoothing removes.  Recipe:
# SeedSequence(seed).spawn(4) -> streams for (q, k, key offsets, v), drawn
# in fp32 [B, H, L, 128] and cast to fp16 (nearest even); tokens-first
# layouts are the same draws transposed.
@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    name: str
    B: int
    H: int
    Lq: int
    Lk: int
    q_block: int = 128
    k_block: int = 64

    @property
    def ops(self) -> int:
        """Operations of the two products (QK^T in int8, P.V in fp16), a
        multiply-add counted as two."""
        return 4 * self.B * self.H * self.Lq * self.Lk * 128


ATTN_WORKLOADS = {
    w.name: w
    for w in [
        # The README's bare-tensor attention check: 40 heads x 14040 tokens.
        AttnWorkload("sage_attn_40x14040", 1, 40, 14040, 14040),
        # A 1024px DiT block: 24 heads x 4096 image tokens, batch 2.
        AttnWorkload("sage_attn_dit1024_2x24x4096", 2, 24, 4096, 4096),
    ]
}

ATTN_HEADLINE = "sage_attn_40x14040"


def attention_inputs(B: int, H: int, Lq: int, Lk: int, seed: int = 0, layout: str = "bhld",
                     key_bias: float = 3.0):
    """fp16 (q, k, v) numpy arrays, [B, H, L, 128] for layout "bhld" or
    [B, L, H, 128] for "blhd" (the same values)."""
    rq, rk, rb, rv = [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(4)]
    q = rq.standard_normal((B, H, Lq, 128), dtype=np.float32).astype(np.float16)
    k = rk.standard_normal((B, H, Lk, 128), dtype=np.float32)
    k += rb.standard_normal((B, H, 1, 128), dtype=np.float32) * np.float32(key_bias)
    k = k.astype(np.float16)
    v = rv.standard_normal((B, H, Lk, 128), dtype=np.float32).astype(np.float16)
    if layout == "blhd":
        q, k, v = (np.ascontiguousarray(t.transpose(0, 2, 1, 3)) for t in (q, k, v))
    elif layout != "bhld":
        raise ValueError(layout)
    return q, k, v
