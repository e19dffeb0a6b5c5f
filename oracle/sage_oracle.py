"""Plain numpy oracle of the INT8 attention (SageAttention-style) -- TEST
INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.

What it computes, and from where ("qlip-mlx" README):
  - sage_attention bullet: INT8 QK^T inside a flash-attention structure
    with exact online softmax;
  - "Key features", second bullet: quantization touches only QK^T, with
    per-token or per-block scales; softmax and P.V stay in floating point;
    fp16 rounding level;
  - "Key features", fourth bullet and "Quick start": head dim 128,
    bidirectional (mask-free) attention, q/k/v [B, heads, L, 128] or
    tokens-first, scale 128^-0.5, fp16 output in the same layout.
The name refers to the published SageAttention method (Zhang et al.,
"SageAttention: Accurate 8-bit attention for plug-and-play inference
acceleration"): K is smoothed by subtracting its mean over the tokens
(softmax is unchanged by it in exact arithmetic, since every score of a
query row moves by the same amount), then Q and the smoothed K are
quantized to int8 with one absmax scale per block of tokens, and the
scores are the dequantized int8 products.

Readings where the pages are silent (listed with their reasons in the
design notes):
  - inputs q, k, v are fp16; D = 128;
  - the K mean is taken per (batch, head, channel) over all Lk tokens,
    exactly: the fp16 values are summed as integers in units of 2^-24 (an
    fp16 value is a whole multiple of 2^-24, so the int64 sum is exact in
    any order), the sum is converted to fp64 (nearest even), scaled by
    2^-24, divided by Lk in fp64 and rounded to fp32 -- the same steps on
    both sides give the same bits;
  - smoothed K = fp32(k - mean), one fp32 subtraction;
  - a block of `block` consecutive tokens (the last one may be shorter)
    shares one scale: the linears' absmax rule over all block x D values
    (amax, inv = fp32(127/amax), codes = clamp(rint(fp32(v*inv)), +-127),
    scale = fp32(amax/127), scale 0 and codes 0 when 127/amax overflows);
    block 1 is per-token;
  - scores S[i,j] = scale * sq[i] * sk[j] * (qc[i] . kc[j]), the dot
    product an exact integer;
  - the result is the exact softmax(S) V for these operands, rounded once
    to fp16 (the GPU evaluates it in fp32 with P rounded to fp16 for the
    P.V product, so it is compared within a tolerance derived from those
    roundings).
"""
from __future__ import annotations

import numpy as np

from .kq_oracle import quantize_rows_absmax

D_HEAD = 128
_TWO24 = float(2 ** 24)


def k_mean_exact(k_f16: np.ndarray) -> np.ndarray:
    """Per-channel mean over the token axis of fp16 keys [..., L, D], as
    fp32 [..., D], by the exact fixed-point sum described above."""
    k = np.asarray(k_f16)
    if k.dtype != np.float16:
        raise ValueError("keys must be float16")
    L = k.shape[-2]
    if L < 1:
        raise ValueError("need at least one token")
    units = (k.astype(np.float64) * _TWO24).astype(np.int64)  # exact: |k| * 2^24 < 2^40
    s = units.sum(axis=-2, dtype=np.int64)
    mean64 = (s.astype(np.float64) / _TWO24) / np.float64(L)
    return mean64.astype(np.float32)


def smooth_k(k_f16: np.ndarray) -> np.ndarray:
    """fp32(k - mean) over the token axis: the smoothed keys."""
    mean = k_mean_exact(k_f16)
    return (np.asarray(k_f16).astype(np.float32) - mean[..., None, :]).astype(np.float32)


def quantize_token_blocks(x_f32: np.ndarray, block: int):
    """int8 codes [L, D] and per-token fp32 scales [L] for fp32 values
    [L, D], one absmax scale per block of `block` tokens (the last block
    may be shorter), replicated to each token of the block."""
    x = np.asarray(x_f32, dtype=np.float32)
    L, D = x.shape
    if block < 1:
        raise ValueError("block must be >= 1")
    codes = np.empty((L, D), np.int8)
    scales = np.empty((L,), np.float32)
    for t0 in range(0, L, block):
        t1 = min(L, t0 + block)
        c, s = quantize_rows_absmax(x[t0:t1].reshape(1, -1))
        codes[t0:t1] = c.reshape(t1 - t0, D)
        scales[t0:t1] = s[0]
    return codes, scales


def prepare(q_f16: np.ndarray, k_f16: np.ndarray, q_block: int, k_block: int):
    """Quantized operands of one (batch, head): q [Lq, D], k [Lk, D] fp16.
    Returns (qc int8 [Lq,D], sq fp32 [Lq], kc int8 [Lk,D], sk fp32 [Lk],
    k_mean fp32 [D])."""
    q32 = np.asarray(q_f16).astype(np.float32)
    mean = k_mean_exact(k_f16)
    ks = (np.asarray(k_f16).astype(np.float32) - mean[None, :]).astype(np.float32)
    qc, sq = quantize_token_blocks(q32, q_block)
    kc, sk = quantize_token_blocks(ks, k_block)
    return qc, sq, kc, sk, mean


def scores_exact(qc, sq, kc, sk, scale: float) -> np.ndarray:
    """S = scale * sq[i] * sk[j] * (qc[i] . kc[j]) in fp64 [Lq, Lk].  The
    integer dot products are exact (|qc . kc| <= 128 * 127^2 < 2^53)."""
    acc = np.asarray(qc, np.float64) @ np.asarray(kc, np.float64).T
    return float(scale) * np.asarray(sq, np.float64)[:, None] * np.asarray(sk, np.float64)[None, :] * acc


def softmax_rows(S: np.ndarray) -> np.ndarray:
    """Row softmax in fp64 (max subtracted first, which changes nothing
    mathematically)."""
    S = np.asarray(S, np.float64)
    e = np.exp(S - S.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def attention_from_codes(qc, sq, kc, sk, v_f16, scale: float):
    """(O fp64 [Lq, D], T fp64 [Lq, D]): O = softmax(S) V exactly, and the
    magnitude T = softmax(S) |V| that bounds the rounding error of an
    evaluation with rounded probabilities."""
    P = softmax_rows(scores_exact(qc, sq, kc, sk, scale))
    v = np.asarray(v_f16).astype(np.float64)
    return P @ v, P @ np.abs(v)


def attention_terms(qc, sq, kc, sk, v_f16, scale: float):
    """(T fp64 [Lq, D], U fp64 [Lq, D]): the two magnitudes against which an
    evaluation with fp16-rounded probabilities and fp32 accumulation is
    accurate.  T = softmax(S) |V|; U = sum_j |V_j| / l with l = sum_j
    exp(S_j - max_j S), the softmax normalizer relative to the row max
    (probabilities in the fp16 subnormal range lose absolute precision
    2^-25 each, relative to that normalizer)."""
    S = scores_exact(qc, sq, kc, sk, scale)
    e = np.exp(S - S.max(axis=1, keepdims=True))
    l = e.sum(axis=1)
    av = np.abs(np.asarray(v_f16).astype(np.float64))
    T = (e / l[:, None]) @ av
    U = av.sum(axis=0)[None, :] / l[:, None]
    return T, U


def sage_attention_head(q_f16, k_f16, v_f16, scale: float, q_block: int, k_block: int):
    """The whole method for one (batch, head): (O fp64 [Lq, D], T fp64
    [Lq, D]) as attention_from_codes."""
    qc, sq, kc, sk, _ = prepare(q_f16, k_f16, q_block, k_block)
    return attention_from_codes(qc, sq, kc, sk, v_f16, scale)


def attention_fp64(q, k, v, scale: float) -> np.ndarray:
    """Unquantized attention softmax(scale q k^T) v in fp64, one head."""
    S = float(scale) * (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T)
    return softmax_rows(S) @ np.asarray(v, np.float64)


def round_f16(y64) -> np.ndarray:
    """Round to fp16, nearest even (numpy's conversion from fp64 rounds
    once)."""
    return np.asarray(y64, np.float64).astype(np.float16)


def f16_ulp(h) -> np.ndarray:
    """Spacing of fp16 at |h| (the subnormal spacing 2^-24 near zero)."""
    a = np.abs(np.asarray(h, np.float16)).astype(np.float64)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
    return 2.0 ** (e - 10)
