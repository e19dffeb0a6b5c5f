"""Plain numpy oracle of the INT8 quantized linear (test infrastructure only).

What it computes, and from where:
  - Per-token activation quantization ("qlip-mlx" README, w8a8_linear feature
    bullet and "Quick start": per-token activation quantization inside the
    kernel, no calibration).  Symmetric absmax int8 with an fp32 scale.
  - Offline weight quantization ("qlip-mlx" README, "Quick start":
    quantize_weight_int8 maps [N,K] weights to int8 plus fp32 scales), the
    same rule per output channel; and affine 4-bit weights with a per-group
    scale and bias, group 64 (MLX pull request 4722, serving test "affine
    4-bit g64" and "Selector rules"; "qlip-mlx" README, w4a8_linear bullet:
    packed int4).
  - The linear: INT8xINT8->INT32 products, then dequantization and bias
    ("qlip-mlx" README, w8a8_linear bullet).  The result is the exact value
    of x_hat . w_hat^T + bias for the dequantized operands, rounded ONCE to
    the output type (mlx-kquant pull request 89 commit list: a route must
    not round beyond one weight and one output rounding; split partials are
    folded so the result rounds once).

Readings where the pages are silent (each is listed with its reason in the
design notes):
  - codes are symmetric in [-127, 127]; rounding is half-to-even (rint);
  - the code is rint(fp32(x * inv)) with inv = fp32(127 / amax) (one IEEE
    multiply per element), and the stored scale is fp32(amax / 127);
  - a row whose 127/amax overflows fp32 (all zero, or tiny) gets scale 0
    and codes 0;
  - int4: min-max affine per 64-group, scale = fp16(fp32((max-min)/15)),
    offset = fp16(min), codes rint(fp32(fp32(w - offset) * fp32(1/scale)))
    clamped to [0, 15], scale 0 -> codes 0; two codes per byte, low nibble
    = even k;
  - bf16 output = round-to-nearest-even of the fp32 output.

Arithmetic: the quantizers use numpy float32 operations (IEEE single,
round-to-nearest-even, subnormals kept), the linear uses float64.  Integer
accumulators are computed with float64 matrix products of integer-valued
operands: every partial sum is an integer below 2^53 in magnitude
(|sum| <= 65536 * 127 * 127 < 2^31), so the result is exact in any order.

Pins (CPU tests): exact-rational brute force of the quantizers on small
inputs, quantizer invariants (absmax code, error bound, sign symmetry,
power-of-two scaling, zero rows), pack/unpack round trips, integer
accumulators against Python-integer dot products, the integer-grid
reductions where dequantization is exact, one-hot rows, the quantization
error bound against an fp64 GEMM of the unquantized operands, and bf16
rounding against torch's conversion.
"""
from __future__ import annotations

import numpy as np

F32_MAX = np.float32(np.finfo(np.float32).max)
_F127 = np.float32(127.0)


# ---------------------------------------------------------------- quantizers
def quantize_rows_absmax(v: np.ndarray):
    """Symmetric per-row int8 quantization of fp32 values v [R, C].

    Returns (codes int8 [R, C], scale fp32 [R]).  Per row: amax = max |v|;
    inv = fp32(127 / amax); if inv is not finite the row quantizes to zero
    with scale 0; else codes = clamp(rint(fp32(v * inv)), -127, 127) and
    scale = fp32(amax / 127)."""
    v = np.asarray(v, dtype=np.float32)
    if v.ndim != 2 or v.shape[1] < 1:
        raise ValueError("need a 2-D array with at least one column")
    amax = np.max(np.abs(v), axis=1)
    with np.errstate(divide="ignore", over="ignore"):
        inv = _F127 / amax
    ok = inv <= F32_MAX
    inv = np.where(ok, inv, np.float32(0.0)).astype(np.float32)
    scale = np.where(ok, amax / _F127, np.float32(0.0)).astype(np.float32)
    t = v * inv[:, None]
    codes = np.clip(np.rint(t), -127, 127).astype(np.int8)
    return codes, scale


def quantize_act(x_bf16_bits: np.ndarray, with_group_sums: bool = True):
    """Per-token activation quantization of bf16 activations [M, K].

    Returns (a int8 [M,K], sx fp32 [M], A int32 [M, K/64] or None).
    A[m, g] is the sum of the codes of row m in the 64-wide K group g,
    produced only when K % 64 == 0 and requested."""
    x = bf16_bits_to_f32(x_bf16_bits)
    a, sx = quantize_rows_absmax(x)
    gsum = None
    if with_group_sums and x.shape[1] % 64 == 0:
        m, k = a.shape
        gsum = a.astype(np.int32).reshape(m, k // 64, 64).sum(axis=2, dtype=np.int32)
    return a, sx, gsum


def quantize_w8(w: np.ndarray):
    """int8 per-output-channel weights: the activation rule applied to each
    row of W [N, K].  Returns (q8 int8 [N,K], sw fp32 [N])."""
    return quantize_rows_absmax(np.asarray(w, dtype=np.float32))


def quantize_w4(w: np.ndarray):
    """Affine 4-bit weights, one fp16 scale and fp16 offset per 64-wide K group.

    Returns (packed uint8 [N, K/2], gs fp16 [N, K/64], gb fp16 [N, K/64],
    q uint8 [N, K] unpacked codes)."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if k % 64:
        raise ValueError("K must be a multiple of 64")
    blocks = w.reshape(n, k // 64, 64)
    lo = blocks.min(axis=2)
    hi = blocks.max(axis=2)
    gs = ((hi - lo) / np.float32(15.0)).astype(np.float16)
    gb = lo.astype(np.float16)
    gs32 = gs.astype(np.float32)
    gb32 = gb.astype(np.float32)
    nz = gs32 != 0
    with np.errstate(divide="ignore"):
        inv = np.where(nz, np.float32(1.0) / np.where(nz, gs32, np.float32(1.0)),
                       np.float32(0.0)).astype(np.float32)
    t = (blocks - gb32[:, :, None]) * inv[:, :, None]
    q = np.clip(np.rint(t), 0, 15).astype(np.uint8).reshape(n, k)
    return pack_w4(q), gs, gb, q


def pack_w4(q: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte: byte j of a row holds code 2j in the low
    nibble and code 2j+1 in the high nibble."""
    q = np.asarray(q, dtype=np.uint8)
    if np.any(q > 15):
        raise ValueError("codes must be in [0, 15]")
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def unpack_w4(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    n, kh = packed.shape
    q = np.empty((n, 2 * kh), dtype=np.uint8)
    q[:, 0::2] = packed & 0x0F
    q[:, 1::2] = packed >> 4
    return q


# --------------------------------------------------------- dequantization
def dequant_w8(q8, sw) -> np.ndarray:
    """w_hat[n,k] = sw[n] * q8[n,k], exact in float64."""
    return np.asarray(sw, np.float64)[:, None] * np.asarray(q8, np.float64)


def dequant_w4(q, gs, gb) -> np.ndarray:
    """w_hat[n,k] = gs[n,g] * q[n,k] + gb[n,g] with g = k // 64, in float64
    (exact for fp16 scale and offset within a few binades of each other)."""
    q = np.asarray(q, np.float64)
    n, k = q.shape
    g = np.arange(k) // 64
    s = np.asarray(gs, np.float64)[:, g]
    b = np.asarray(gb, np.float64)[:, g]
    return s * q + b


# ----------------------------------------------------- integer accumulators
def w8a8_acc(a, q8) -> np.ndarray:
    """acc[m,n] = sum_k a[m,k] * q8[n,k], exact, as int32."""
    acc = np.asarray(a, np.float64) @ np.asarray(q8, np.float64).T
    return acc.astype(np.int64).astype(np.int32)


def w4a8_group_acc(a, q) -> np.ndarray:
    """P[g,m,n] = sum_{k in group g} a[m,k] * q[n,k], exact, int32 [G,M,N]."""
    a = np.asarray(a, np.float64)
    q = np.asarray(q, np.float64)
    m, k = a.shape
    n = q.shape[0]
    out = np.empty((k // 64, m, n), dtype=np.int32)
    for g in range(k // 64):
        sl = slice(64 * g, 64 * g + 64)
        out[g] = (a[:, sl] @ q[:, sl].T).astype(np.int64).astype(np.int32)
    return out


# ------------------------------------------------------------------ linears
# y = x_hat . w_hat^T + bias for the dequantized operands.  The scales are
# factored out of the exact integer sums (the same algebra), so the float64
# result is within a few roundings (2^-52 relative) of the exact value; a
# float64 product of the dequantized operands would instead carry an error
# proportional to sum |x_hat||w_hat|, which need not vanish where the exact
# result is 0.
def w8a8_linear_exact(x_bf16_bits, q8, sw, bias=None) -> np.ndarray:
    """y[m,n] = sx[m] * sw[n] * acc[m,n] + bias[n] in float64, with
    acc = sum_k a*q8 exact (x_hat = sx*a, w_hat = sw*q8)."""
    a, sx, _ = quantize_act(x_bf16_bits, with_group_sums=False)
    acc = w8a8_acc(a, q8).astype(np.float64)
    s = np.asarray(sx, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :]  # exact
    y = s * acc
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    return y


def w4a8_linear_exact(x_bf16_bits, q, gs, gb, bias=None) -> np.ndarray:
    """y[m,n] = sx[m] * sum_g (gs[n,g]*P[g,m,n] + gb[n,g]*A[m,g]) + bias[n]
    in float64, with P and A exact integers (x_hat = sx*a, w_hat = gs*q + gb
    per 64-group: sum_k x_hat*w_hat = sx * sum_g (gs*P + gb*A)).  Each
    gs*P and gb*A is exact in float64."""
    a, sx, A = quantize_act(x_bf16_bits, with_group_sums=True)
    if A is None:
        raise ValueError("K must be a multiple of 64")
    a64 = a.astype(np.float64)
    q64 = np.asarray(q, np.float64)
    gs64 = np.asarray(gs, np.float64)
    gb64 = np.asarray(gb, np.float64)
    s = np.zeros((a.shape[0], q64.shape[0]))
    for g in range(a.shape[1] // 64):
        sl = slice(64 * g, 64 * g + 64)
        P = a64[:, sl] @ q64[:, sl].T                         # exact integers
        s += gs64[None, :, g] * P + gb64[None, :, g] * A[:, g, None].astype(np.float64)
    y = np.asarray(sx, np.float64)[:, None] * s
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    return y


def linear_dequantized_fp64(x_bf16_bits, w_hat, bias=None) -> np.ndarray:
    """The plain definition: float64 product of the dequantized operands,
    x_hat . w_hat^T + bias (used to cross-check the factored forms)."""
    a, sx, _ = quantize_act(x_bf16_bits, with_group_sums=False)
    xh = np.asarray(sx, np.float64)[:, None] * a.astype(np.float64)
    y = xh @ np.asarray(w_hat, np.float64).T
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    return y


def w8a8_magnitude(x_bf16_bits, q8, sw, bias=None) -> np.ndarray:
    """Term magnitude T[m,n] = |sx*sw*acc| + |bias|: the scale against which
    an fp32 evaluation of the int8 epilogue is accurate."""
    a, sx, _ = quantize_act(x_bf16_bits, with_group_sums=False)
    acc = w8a8_acc(a, q8).astype(np.float64)
    t = np.abs(np.asarray(sx, np.float64)[:, None] * np.asarray(sw, np.float64)[None, :] * acc)
    if bias is not None:
        t = t + np.abs(np.asarray(bias, np.float64))[None, :]
    return t


def w4a8_magnitude(x_bf16_bits, q, gs, gb, bias=None) -> np.ndarray:
    """T[m,n] = sx * sum_g (|gs*P| + |gb*A|) + |bias|: the scale against which
    an fp32 per-group evaluation of the int4 epilogue is accurate."""
    a, sx, A = quantize_act(x_bf16_bits, with_group_sums=True)
    a64 = a.astype(np.float64)
    q64 = np.asarray(q, np.float64)
    gs64 = np.asarray(gs, np.float64)
    gb64 = np.asarray(gb, np.float64)
    s = np.zeros((a.shape[0], q64.shape[0]))
    for g in range(a.shape[1] // 64):
        sl = slice(64 * g, 64 * g + 64)
        P = a64[:, sl] @ q64[:, sl].T
        s += np.abs(gs64[None, :, g] * P) + np.abs(gb64[None, :, g] * A[:, g, None].astype(np.float64))
    t = np.asarray(sx, np.float64)[:, None] * s
    if bias is not None:
        t = t + np.abs(np.asarray(bias, np.float64))[None, :]
    return t


# ------------------------------------------------- gated residual epilogue
# mlx-kquant pull request 89 commit list: a quantized matmul with a gated
# residual epilogue, its elements held within 2 ulp.  The pages give no
# formula; the reading is the DiT block's gated residual add: the block
# input plus a per-sample, per-channel gate times the linear's output, with
# one gate row shared by `gate_rows` consecutive token rows.
def gated_residual_exact(y64, residual_bf16_bits=None, gate=None, gate_rows=1) -> np.ndarray:
    """out[m,n] = r[m,n] + g[m // gate_rows, n] * y[m,n] in float64, for the
    linear's exact result y (float64 [M,N]); residual bf16 bits [M,N] or None
    (zero), gate fp32 [ceil(M/gate_rows), N] or None (one)."""
    y = np.asarray(y64, np.float64)
    if gate is not None:
        rows = np.arange(y.shape[0]) // int(gate_rows)
        y = np.asarray(gate, np.float64)[rows, :] * y
    if residual_bf16_bits is not None:
        y = y + bf16_bits_to_f32(residual_bf16_bits).astype(np.float64)
    return y


def gated_magnitude(T, residual_bf16_bits=None, gate=None, gate_rows=1) -> np.ndarray:
    """|r| + |g| * T for the linear's term magnitude T: the scale against
    which an fp32 evaluation of the gated epilogue is accurate."""
    t = np.asarray(T, np.float64)
    if gate is not None:
        rows = np.arange(t.shape[0]) // int(gate_rows)
        t = np.abs(np.asarray(gate, np.float64)[rows, :]) * t
    if residual_bf16_bits is not None:
        t = t + np.abs(bf16_bits_to_f32(residual_bf16_bits).astype(np.float64))
    return t


# ------------------------------------------------------------ output rounding
def round_f32(y64) -> np.ndarray:
    """Round float64 to fp32, nearest even."""
    return np.asarray(y64, np.float64).astype(np.float32)


def round_bf16_bits(y32) -> np.ndarray:
    """Round fp32 to bf16, nearest even, returning uint16 bit patterns.
    (Finite inputs: add 0x7FFF plus the lowest kept bit, then truncate.)"""
    u = np.asarray(y32, np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def bf16_ulp(bits) -> np.ndarray:
    """Spacing of bf16 numbers at each value (the gap to the next larger
    magnitude), as fp64."""
    b = np.asarray(bits, dtype=np.uint16)
    mag = b & 0x7FFF
    nxt = (mag + 1).astype(np.uint16)
    return (bf16_bits_to_f32(nxt).astype(np.float64)
            - bf16_bits_to_f32(mag).astype(np.float64))
