"""w8a8_gemm_dit_amd -- Python binding of libkq, the MI355X INT8 quantized
linear (W8A8 / W4A8 / small-M GEMV) and INT8 attention.

Argument marshalling only: every step of the computation runs in libkq's HIP
kernels.  The functions carry the C entry points' names, take torch tensors
on the GPU (torch provides device memory and the current stream) and raise
ValueError (invalid or unsupported arguments, workspace) or RuntimeError
(no device, launch failure) with libkq's "[op] message".  If libkq.so has
not been built, every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "KQ_W8_PER_CHANNEL", "KQ_W4_AFFINE_G64", "KQ_DTYPE_F32", "KQ_DTYPE_BF16",
    "KQ_DTYPE_I32", "KQ_MAX_K", "KQ_GEMV_MAX_M", "lib", "lib_path", "exported_symbols",
    "kq_is_available", "kq_last_error", "kq_workspace_bytes", "kq_route",
    "kq_quantize_weights", "kq_quantize_act", "kq_w8a8_linear", "kq_w4a8_linear",
    "kq_gemv_small_m", "kq_w8a8_gemm", "kq_w4a8_gemm", "kq_linear_gated", "KqError",
    "KQ_LAYOUT_BHLD", "KQ_LAYOUT_BLHD", "kq_sage_workspace_layout", "kq_sage_prepare",
    "kq_sage_attend", "kq_sage_attention", "kq_probe_read", "kq_probe_mfma_i8",
    "kq_w8a8_linear_noalloc", "KQ_NOALLOC_SCRATCH_BYTES", "KQ_CODES_NATURAL",
    "KQ_CODES_SPLIT8", "kq_quantize_act_ordered", "kq_w4a8_gemm_ordered",
]

KQ_SUCCESS, KQ_ERR_INVALID_VALUE, KQ_ERR_UNSUPPORTED = 0, 1, 2
KQ_ERR_NO_DEVICE, KQ_ERR_WORKSPACE, KQ_ERR_LAUNCH = 3, 4, 5
KQ_W8_PER_CHANNEL, KQ_W4_AFFINE_G64 = 0, 1
KQ_DTYPE_F32, KQ_DTYPE_BF16, KQ_DTYPE_I32 = 0, 1, 2
KQ_ROUTE_GEMM, KQ_ROUTE_GEMV, KQ_ROUTE_FUSED = 0, 1, 2
_ROUTE_NAMES = {KQ_ROUTE_GEMM: "gemm", KQ_ROUTE_GEMV: "gemv", KQ_ROUTE_FUSED: "fused"}
KQ_MAX_K = 65536
KQ_GEMV_MAX_M = 16
KQ_GEMV_MAX_K = 16384
KQ_LAYOUT_BHLD, KQ_LAYOUT_BLHD = 0, 1
KQ_NOALLOC_SCRATCH_BYTES = 64 << 20
KQ_CODES_NATURAL, KQ_CODES_SPLIT8 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkq.so")
_lib: Optional[ctypes.CDLL] = None

exported_symbols = (
    "kq_is_available", "kq_last_error", "kq_workspace_bytes", "kq_route",
    "kq_quantize_weights", "kq_quantize_act", "kq_w8a8_linear",
    "kq_w4a8_linear", "kq_gemv_small_m", "kq_w8a8_gemm", "kq_w4a8_gemm",
    "kq_linear_gated", "kq_sage_workspace_layout", "kq_sage_prepare", "kq_sage_attend",
    "kq_sage_attention", "kq_probe_read", "kq_probe_mfma_i8", "kq_w8a8_linear_noalloc",
    "kq_quantize_act_ordered", "kq_w4a8_gemm_ordered",
)


class KqError(RuntimeError):
    pass


class RouteInfo(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("tile_m", ctypes.c_int32),
                ("tile_n", ctypes.c_int32), ("threads", ctypes.c_int32),
                ("grid", ctypes.c_int64), ("splits", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class SageWorkspace(ctypes.Structure):
    _fields_ = [("lq_pad", ctypes.c_int64), ("lk_pad", ctypes.c_int64), ("chunks", ctypes.c_int64),
                ("qc", ctypes.c_size_t), ("sq", ctypes.c_size_t), ("kc", ctypes.c_size_t),
                ("sk", ctypes.c_size_t), ("vt", ctypes.c_size_t), ("kmean", ctypes.c_size_t),
                ("colsum", ctypes.c_size_t), ("meta", ctypes.c_size_t),
                ("total", ctypes.c_size_t)]


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libkq (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise KqError(f"libkq.so is not built ({_LIB_PATH}); run "
                      "`python -m w8a8_gemm_dit_amd.build` or __graft_entry__.build()")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    i32 = ctypes.c_int
    L.kq_is_available.restype = i32
    L.kq_is_available.argtypes = []
    L.kq_last_error.restype = ctypes.c_char_p
    L.kq_last_error.argtypes = []
    L.kq_workspace_bytes.restype = sz
    L.kq_workspace_bytes.argtypes = [i64, i64, i64, i32]
    L.kq_route.restype = i32
    L.kq_route.argtypes = [i64, i64, i64, i32, i32, ctypes.POINTER(RouteInfo)]
    L.kq_quantize_weights.restype = i32
    L.kq_quantize_weights.argtypes = [vp, i64, i64, i32, vp, vp, vp, vp]
    L.kq_quantize_act.restype = i32
    L.kq_quantize_act.argtypes = [vp, i64, i64, vp, vp, vp, vp]
    L.kq_w8a8_linear.restype = i32
    L.kq_w8a8_linear.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, i32, vp, sz, vp]
    L.kq_w4a8_linear.restype = i32
    L.kq_w4a8_linear.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    L.kq_w8a8_gemm.restype = i32
    L.kq_w8a8_gemm.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, i32, vp]
    L.kq_w4a8_gemm.restype = i32
    L.kq_w4a8_gemm.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, i32, vp]
    L.kq_quantize_act_ordered.restype = i32
    L.kq_quantize_act_ordered.argtypes = [vp, i64, i64, vp, vp, vp, i32, vp]
    L.kq_w4a8_gemm_ordered.restype = i32
    L.kq_w4a8_gemm_ordered.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, i32, i32, vp]
    L.kq_gemv_small_m.restype = i32
    L.kq_gemv_small_m.argtypes = [i32, vp, i64, i64, i64, vp, vp, vp, vp, vp, i32, vp, sz, vp]
    L.kq_sage_workspace_layout.restype = i32
    L.kq_sage_workspace_layout.argtypes = [i64, i64, i64, i64, ctypes.POINTER(SageWorkspace)]
    L.kq_sage_prepare.restype = i32
    L.kq_sage_prepare.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, i32, i64, i64, vp, sz, vp]
    L.kq_sage_attend.restype = i32
    L.kq_sage_attend.argtypes = [vp, sz, vp, i64, i64, i64, i64, i64, i32, ctypes.c_float, i64,
                                 vp]
    L.kq_sage_attention.restype = i32
    L.kq_sage_attention.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, ctypes.c_float,
                                    i64, i64, vp, sz, vp]
    L.kq_linear_gated.restype = i32
    L.kq_linear_gated.argtypes = [i32, vp, i64, i64, i64, vp, vp, vp, vp, vp, vp, i64, vp, i32,
                                  vp, sz, vp]
    L.kq_w8a8_linear_noalloc.restype = i32
    L.kq_w8a8_linear_noalloc.argtypes = [vp, i64, i64, i64, vp, vp, vp, vp, i32, vp]
    L.kq_probe_read.restype = i32
    L.kq_probe_read.argtypes = [vp, i64, i64, ctypes.c_int32, vp, vp]
    L.kq_probe_mfma_i8.restype = i32
    L.kq_probe_mfma_i8.argtypes = [i64, i64, vp, vp]
    _lib = L
    return L


def _check(status: int) -> None:
    if status == KQ_SUCCESS:
        return
    msg = lib().kq_last_error().decode()
    if status in (KQ_ERR_INVALID_VALUE, KQ_ERR_UNSUPPORTED, KQ_ERR_WORKSPACE):
        raise ValueError(msg)
    raise KqError(msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_OUT = {torch.float32: KQ_DTYPE_F32, torch.bfloat16: KQ_DTYPE_BF16, torch.int32: KQ_DTYPE_I32}


# ------------------------------------------------------------------ queries
def kq_is_available() -> bool:
    return bool(lib().kq_is_available())


def kq_last_error() -> str:
    return lib().kq_last_error().decode()


def kq_workspace_bytes(M: int, N: int, K: int, fmt: int) -> int:
    return int(lib().kq_workspace_bytes(M, N, K, fmt))


def kq_route(M: int, N: int, K: int, fmt: int, out_dtype: int = KQ_DTYPE_BF16) -> dict:
    info = RouteInfo()
    _check(lib().kq_route(M, N, K, fmt, out_dtype, ctypes.byref(info)))
    return {"kind": _ROUTE_NAMES.get(info.kind, "?"), "tile_m": info.tile_m,
            "tile_n": info.tile_n, "threads": info.threads, "grid": info.grid,
            "splits": info.splits}


# ------------------------------------------------------------- quantizers
def kq_quantize_weights(w: torch.Tensor, fmt: int):
    """fp32 [N,K] -> (wq, scale, gbias): int8 [N,K], fp32 [N], None for
    KQ_W8_PER_CHANNEL; uint8 [N,K/2], fp16 [N,K/64], fp16 [N,K/64] for
    KQ_W4_AFFINE_G64."""
    _need(w, "w", torch.float32, 2)
    N, K = w.shape
    dev = w.device
    if fmt == KQ_W8_PER_CHANNEL:
        wq = torch.empty((N, K), dtype=torch.int8, device=dev)
        sc = torch.empty((N,), dtype=torch.float32, device=dev)
        gb = None
    elif fmt == KQ_W4_AFFINE_G64:
        if K % 64:
            raise ValueError(f"[kq_quantize_weights] K={K} must be a multiple of 64 for int4 weights")
        wq = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
        sc = torch.empty((N, K // 64), dtype=torch.float16, device=dev)
        gb = torch.empty((N, K // 64), dtype=torch.float16, device=dev)
    else:
        raise ValueError(f"unknown weight format {fmt}")
    _check(lib().kq_quantize_weights(_ptr(w), N, K, fmt, _ptr(wq), _ptr(sc), _ptr(gb), _stream()))
    return wq, sc, gb


def kq_quantize_act(x: torch.Tensor, group_sums: bool = False, out=None):
    """bf16 [M,K] -> (codes int8 [M,K], scales fp32 [M], group sums int32
    [M,K/64] or None).  out: optional (codes, scales, group sums or None)
    tensors to write into."""
    return _quantize_act(x, None, group_sums, out)


def kq_quantize_act_ordered(x: torch.Tensor, order: int, group_sums: bool = False, out=None):
    """kq_quantize_act with the codes of each row in `order` (KQ_CODES_*)."""
    return _quantize_act(x, int(order), group_sums, out)


def _quantize_act(x, order, group_sums, out):
    # order None: kq_quantize_act, else kq_quantize_act_ordered
    _need(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    if out is None:
        a = torch.empty((M, K), dtype=torch.int8, device=x.device)
        sx = torch.empty((M,), dtype=torch.float32, device=x.device)
        gs = torch.empty((M, K // 64), dtype=torch.int32, device=x.device) if group_sums else None
    else:
        a, sx, gs = out
        _need(a, "codes", torch.int8, 2)
        _need(sx, "scales", torch.float32, 1)
        if tuple(a.shape) != (M, K) or tuple(sx.shape) != (M,):
            raise ValueError("out codes / scales have the wrong shape")
        if group_sums:
            _need(gs, "group sums", torch.int32, 2)
            if tuple(gs.shape) != (M, K // 64):
                raise ValueError("out group sums have the wrong shape")
        else:
            gs = None
    if order is None:
        _check(lib().kq_quantize_act(_ptr(x), M, K, _ptr(a), _ptr(sx), _ptr(gs), _stream()))
    else:
        _check(lib().kq_quantize_act_ordered(_ptr(x), M, K, _ptr(a), _ptr(sx), _ptr(gs), order,
                                             _stream()))
    return a, sx, gs


# ----------------------------------------------------------------- linears
def _prep_out(out, shape, out_dtype, dev):
    if out is None:
        return torch.empty(shape, dtype=out_dtype, device=dev)
    if tuple(out.shape) != tuple(shape) or out.dtype != out_dtype or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous {out_dtype} tensor of shape {tuple(shape)}")
    return out


def _prep_ws(workspace, M, N, K, fmt, dev):
    need = kq_workspace_bytes(M, N, K, fmt)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    return workspace, workspace.numel() * workspace.element_size()


def _out_shape(M, N, K, out_dtype, per_group):
    if out_dtype == torch.int32 and per_group:
        return (K // 64, M, N)
    return (M, N)


def kq_w8a8_linear(x, wq, sw, bias=None, out_dtype=torch.bfloat16, out=None, workspace=None):
    """y = dequant(int8 per-token x) . dequant(int8 per-channel W)^T + bias."""
    _need(x, "x", torch.bfloat16, 2)
    _need(wq, "wq", torch.int8, 2)
    _need(sw, "sw", torch.float32, 1)
    if bias is not None:
        _need(bias, "bias", torch.float32, 1)
    M, K = x.shape
    N = wq.shape[0]
    if wq.shape[1] != K or sw.shape[0] != N or (bias is not None and bias.shape[0] != N):
        raise ValueError("[kq_w8a8_linear] operand shapes disagree")
    y = _prep_out(out, _out_shape(M, N, K, out_dtype, False), out_dtype, x.device)
    ws, wsb = _prep_ws(workspace, M, N, K, KQ_W8_PER_CHANNEL, x.device)
    _check(lib().kq_w8a8_linear(_ptr(x), M, K, N, _ptr(wq), _ptr(sw), _ptr(bias), _ptr(y),
                                _OUT[out_dtype], _ptr(ws), wsb, _stream()))
    return y


def kq_w4a8_linear(x, wq4, gscale, gbias, bias=None, out_dtype=torch.bfloat16, out=None,
                   workspace=None):
    """y = dequant(int8 per-token x) . dequant(int4 affine g64 W)^T + bias.
    out_dtype=torch.int32 returns the per-group products [K/64, M, N]."""
    _need(x, "x", torch.bfloat16, 2)
    _need(wq4, "wq4", torch.uint8, 2)
    _need(gscale, "gscale", torch.float16, 2)
    _need(gbias, "gbias", torch.float16, 2)
    if bias is not None:
        _need(bias, "bias", torch.float32, 1)
    M, K = x.shape
    N = wq4.shape[0]
    if (wq4.shape[1] * 2 != K or tuple(gscale.shape) != (N, K // 64)
            or tuple(gbias.shape) != (N, K // 64) or (bias is not None and bias.shape[0] != N)):
        raise ValueError("[kq_w4a8_linear] operand shapes disagree")
    y = _prep_out(out, _out_shape(M, N, K, out_dtype, True), out_dtype, x.device)
    ws, wsb = _prep_ws(workspace, M, N, K, KQ_W4_AFFINE_G64, x.device)
    _check(lib().kq_w4a8_linear(_ptr(x), M, K, N, _ptr(wq4), _ptr(gscale), _ptr(gbias), _ptr(bias),
                                _ptr(y), _OUT[out_dtype], _ptr(ws), wsb, _stream()))
    return y


def kq_gemv_small_m(fmt, x, wq, scale, gbias=None, bias=None, out_dtype=torch.bfloat16, out=None,
                    workspace=None):
    """The M <= 16 register-dequant GEMV, for either weight format."""
    _need(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    N = wq.shape[0]
    if fmt == KQ_W4_AFFINE_G64:
        _need(wq, "wq", torch.uint8, 2)
        _need(scale, "scale", torch.float16, 2)
        _need(gbias, "gbias", torch.float16, 2)
    elif fmt == KQ_W8_PER_CHANNEL:
        _need(wq, "wq", torch.int8, 2)
        _need(scale, "scale", torch.float32, 1)
    else:
        raise ValueError(f"unknown weight format {fmt}")
    if bias is not None:
        _need(bias, "bias", torch.float32, 1)
    y = _prep_out(out, _out_shape(M, N, K, out_dtype, fmt == KQ_W4_AFFINE_G64), out_dtype, x.device)
    ws, wsb = _prep_ws(workspace, M, N, K, fmt, x.device)
    _check(lib().kq_gemv_small_m(fmt, _ptr(x), M, K, N, _ptr(wq), _ptr(scale), _ptr(gbias),
                                 _ptr(bias), _ptr(y), _OUT[out_dtype], _ptr(ws), wsb, _stream()))
    return y


def kq_linear_gated(fmt, x, wq, scale, gbias=None, bias=None, residual=None, gate=None,
                    gate_rows=1, out_dtype=torch.bfloat16, out=None, workspace=None):
    """out = residual + gate[m // gate_rows] * linear(x), in the linear's
    epilogue.  residual: bf16 [M,N] or None (may be `out` itself for a bf16
    output); gate: fp32 [ceil(M/gate_rows), N] or None."""
    _need(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    N = wq.shape[0]
    if fmt == KQ_W4_AFFINE_G64:
        _need(wq, "wq", torch.uint8, 2)
        _need(scale, "scale", torch.float16, 2)
        _need(gbias, "gbias", torch.float16, 2)
    elif fmt == KQ_W8_PER_CHANNEL:
        _need(wq, "wq", torch.int8, 2)
        _need(scale, "scale", torch.float32, 1)
    else:
        raise ValueError(f"unknown weight format {fmt}")
    if bias is not None:
        _need(bias, "bias", torch.float32, 1)
    if residual is not None:
        _need(residual, "residual", torch.bfloat16, 2)
        if tuple(residual.shape) != (M, N):
            raise ValueError(f"[kq_linear_gated] residual must be [{M}, {N}]")
    if gate is not None:
        _need(gate, "gate", torch.float32, 2)
        if gate_rows < 1 or tuple(gate.shape) != (-(-M // gate_rows), N):
            raise ValueError("[kq_linear_gated] gate must be [ceil(M/gate_rows), N]")
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("[kq_linear_gated] out_dtype must be float32 or bfloat16")
    y = _prep_out(out, (M, N), out_dtype, x.device)
    ws, wsb = _prep_ws(workspace, M, N, K, fmt, x.device)
    _check(lib().kq_linear_gated(fmt, _ptr(x), M, K, N, _ptr(wq), _ptr(scale), _ptr(gbias),
                                 _ptr(bias), _ptr(residual), _ptr(gate), gate_rows, _ptr(y),
                                 _OUT[out_dtype], _ptr(ws), wsb, _stream()))
    return y


def kq_w8a8_gemm(a, sx, wq, sw, bias=None, out_dtype=torch.bfloat16, out=None):
    """kq_w8a8_linear on codes/scales from kq_quantize_act."""
    _need(a, "a", torch.int8, 2)
    _need(sx, "sx", torch.float32, 1)
    _need(wq, "wq", torch.int8, 2)
    _need(sw, "sw", torch.float32, 1)
    M, K = a.shape
    N = wq.shape[0]
    y = _prep_out(out, _out_shape(M, N, K, out_dtype, False), out_dtype, a.device)
    _check(lib().kq_w8a8_gemm(_ptr(a), _ptr(sx), M, K, N, _ptr(wq), _ptr(sw), _ptr(bias), _ptr(y),
                              _OUT[out_dtype], _stream()))
    return y


def kq_w4a8_gemm(a, sx, gsum, wq4, gscale, gbias, bias=None, out_dtype=torch.bfloat16, out=None):
    """kq_w4a8_linear on codes/scales/group sums from kq_quantize_act."""
    return _w4a8_gemm(a, sx, gsum, wq4, gscale, gbias, None, bias, out_dtype, out)


def kq_w4a8_gemm_ordered(a, sx, gsum, wq4, gscale, gbias, order, bias=None,
                         out_dtype=torch.bfloat16, out=None):
    """kq_w4a8_gemm on codes in `order` (KQ_CODES_*), e.g. from
    kq_quantize_act_ordered."""
    return _w4a8_gemm(a, sx, gsum, wq4, gscale, gbias, int(order), bias, out_dtype, out)


def _w4a8_gemm(a, sx, gsum, wq4, gscale, gbias, order, bias, out_dtype, out):
    # order None: kq_w4a8_gemm, else kq_w4a8_gemm_ordered
    _need(a, "a", torch.int8, 2)
    _need(sx, "sx", torch.float32, 1)
    _need(gsum, "gsum", torch.int32, 2)
    _need(wq4, "wq4", torch.uint8, 2)
    M, K = a.shape
    N = wq4.shape[0]
    y = _prep_out(out, _out_shape(M, N, K, out_dtype, True), out_dtype, a.device)
    args = (_ptr(a), _ptr(sx), _ptr(gsum), M, K, N, _ptr(wq4), _ptr(gscale), _ptr(gbias),
            _ptr(bias), _ptr(y), _OUT[out_dtype])
    if order is None:
        _check(lib().kq_w4a8_gemm(*args, _stream()))
    else:
        _check(lib().kq_w4a8_gemm_ordered(*args, order, _stream()))
    return y


# ---------------------------------------------------------------- attention
_LAYOUTS = {"bhld": KQ_LAYOUT_BHLD, "blhd": KQ_LAYOUT_BLHD}


def kq_sage_workspace_layout(B: int, H: int, Lq: int, Lk: int) -> dict:
    """Byte offsets of the attention workspace's regions and its total size."""
    out = SageWorkspace()
    _check(lib().kq_sage_workspace_layout(B, H, Lq, Lk, ctypes.byref(out)))
    return {name: getattr(out, name) for name, _ in SageWorkspace._fields_}


def _sage_dims(q, k, v, layout):
    if layout not in _LAYOUTS:
        raise ValueError(f"layout must be 'bhld' or 'blhd', got {layout!r}")
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, name, torch.float16, 4)
    if layout == "bhld":
        B, H, Lq, D = q.shape
        Lk = k.shape[2]
        kshape = (B, H, Lk, D)
    else:
        B, Lq, H, D = q.shape
        Lk = k.shape[1]
        kshape = (B, Lk, H, D)
    if tuple(k.shape) != kshape or tuple(v.shape) != kshape:
        raise ValueError("[kq_sage_attention] q, k and v shapes disagree")
    return B, H, Lq, Lk, D


def _sage_ws(workspace, B, H, Lq, Lk, dev):
    need = kq_sage_workspace_layout(B, H, Lq, Lk)["total"]
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    return workspace, workspace.numel() * workspace.element_size()


def kq_sage_prepare(q, k, v, q_block=128, k_block=64, layout="bhld", workspace=None):
    """The preparation pass: returns the workspace holding the key means,
    the query/key codes and scales and the transposed values."""
    B, H, Lq, Lk, D = _sage_dims(q, k, v, layout)
    ws, wsb = _sage_ws(workspace, B, H, Lq, Lk, q.device)
    _check(lib().kq_sage_prepare(_ptr(q), _ptr(k), _ptr(v), B, H, Lq, Lk, D, _LAYOUTS[layout],
                                 q_block, k_block, _ptr(ws), wsb, _stream()))
    return ws


def kq_sage_attend(workspace, B, H, Lq, Lk, scale=None, layout="bhld", out=None, device=None,
                   k_block=64):
    """The attention on a workspace kq_sage_prepare filled (with the same
    shape and k_block); returns out (fp16)."""
    if layout not in _LAYOUTS:
        raise ValueError(f"layout must be 'bhld' or 'blhd', got {layout!r}")
    shape = (B, H, Lq, 128) if layout == "bhld" else (B, Lq, H, 128)
    y = _prep_out(out, shape, torch.float16, device or workspace.device)
    scale = 128 ** -0.5 if scale is None else float(scale)
    _check(lib().kq_sage_attend(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                _ptr(y), B, H, Lq, Lk, 128, _LAYOUTS[layout], scale, k_block,
                                _stream()))
    return y


def kq_sage_attention(q, k, v, scale=None, q_block=128, k_block=64, layout="bhld", out=None,
                      workspace=None):
    """INT8 attention: softmax(scale * dequant(Qc) dequant(Kc)^T) V with K
    smoothed by its token mean, fp16 in and out.  layout 'bhld' takes
    [B, H, L, 128] tensors, 'blhd' [B, L, H, 128]."""
    B, H, Lq, Lk, D = _sage_dims(q, k, v, layout)
    y = _prep_out(out, tuple(q.shape), torch.float16, q.device)
    ws, wsb = _sage_ws(workspace, B, H, Lq, Lk, q.device)
    scale = D ** -0.5 if scale is None else float(scale)
    _check(lib().kq_sage_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(y), B, H, Lq, Lk, D,
                                   _LAYOUTS[layout], scale, q_block, k_block, _ptr(ws), wsb,
                                   _stream()))
    return y


def kq_w8a8_linear_noalloc(x: torch.Tensor, wq: torch.Tensor, sw: torch.Tensor,
                           bias: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16,
                           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """kq_w8a8_linear on the library's own device scratch (no workspace;
    the C call allocates nothing).  Shapes whose workspace would exceed
    KQ_NOALLOC_SCRATCH_BYTES raise ValueError; calls that may overlap on
    one GPU race on the shared scratch."""
    _need(x, "x", torch.bfloat16, 2)
    _need(wq, "wq", torch.int8, 2)
    _need(sw, "sw", torch.float32, 1)
    if bias is not None:
        _need(bias, "bias", torch.float32, 1)
    M, K = x.shape
    N = wq.shape[0]
    if wq.shape[1] != K or sw.shape[0] != N or (bias is not None and bias.shape[0] != N):
        raise ValueError("[kq_w8a8_linear_noalloc] operand shapes disagree")
    if out_dtype not in _OUT:
        raise ValueError(f"unsupported out_dtype {out_dtype}")
    y = _prep_out(out, (M, N), out_dtype, x.device)
    _check(lib().kq_w8a8_linear_noalloc(_ptr(x), M, K, N, _ptr(wq), _ptr(sw), _ptr(bias), _ptr(y),
                                        _OUT[out_dtype], _stream()))
    return y


# --------------------------------------------------------- measurement probes
def kq_probe_read(src: torch.Tensor, grid: int, threads: int = 512,
                  sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Streaming read of all of `src` (any dtype, contiguous, a multiple of
    16 bytes) over `grid` workgroups; returns the (untouched) sink."""
    if not src.is_cuda or not src.is_contiguous():
        raise ValueError("src must be a contiguous GPU tensor")
    if sink is None:
        sink = torch.zeros((grid,), dtype=torch.int32, device=src.device)
    _check(lib().kq_probe_read(_ptr(src), src.numel() * src.element_size(), grid, threads,
                               _ptr(sink), _stream()))
    return sink


def kq_probe_mfma_i8(iters: int, grid: int, sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """iters x 8 int8 MFMAs per wavefront, 8 wavefronts x `grid` workgroups
    (2^21 * iters * grid integer operations)."""
    if sink is None:
        sink = torch.zeros((grid,), dtype=torch.int32, device="cuda")
    _check(lib().kq_probe_mfma_i8(iters, grid, _ptr(sink), _stream()))
    return sink
