"""CPU tests of the C ABI: the library loads, exports every symbol the header
declares, and its host logic (validation, routing, workspace sizing, error
messages) behaves as documented.  No call here reaches the device: each one
fails validation, or is a no-op, before any device access."""
import ctypes
import os
import re

import pytest

import w8a8_gemm_dit_amd as kq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kq.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:int|kq_status|size_t|const char\*)\s+(kq_\w+)\s*\(",
                                 src, flags=re.M)))


def test_library_exports_every_declared_function():
    L = kq.lib()
    declared = _declared_functions()
    assert len(declared) == 21, declared
    assert sorted(kq.exported_symbols) == declared
    for name in declared:
        assert hasattr(L, name), name


def test_is_available_false_without_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("GPU present")
    assert kq.kq_is_available() is False


def test_workspace_layout():
    al = lambda v: (v + 255) // 256 * 256
    M, K = 4096, 3072
    N = 3072
    assert kq.kq_workspace_bytes(M, N, K, kq.KQ_W8_PER_CHANNEL) == al(M * K) + al(4 * M)
    assert kq.kq_workspace_bytes(M, N, K, kq.KQ_W4_AFFINE_G64) == al(M * K) + al(4 * M) + al(4 * M * K // 64)
    assert kq.kq_workspace_bytes(0, N, K, kq.KQ_W8_PER_CHANNEL) == 0
    assert kq.kq_workspace_bytes(M, 0, K, kq.KQ_W8_PER_CHANNEL) == 0
    # codes for rows rounded up to 16 (the GEMV's fragment order covers
    # whole 16-row blocks)
    assert kq.kq_workspace_bytes(3, N, 64, kq.KQ_W8_PER_CHANNEL) == 1024 + 256
    # the fused routes use only the scales, but the size covers the
    # two-kernel route of the same shape
    assert kq.kq_route(2048, 48, 5120, kq.KQ_W8_PER_CHANNEL)["kind"] == "fused"
    assert kq.kq_workspace_bytes(2048, 48, 5120, kq.KQ_W8_PER_CHANNEL) == al(2048 * 5120) + al(4 * 2048)
    assert kq.kq_workspace_bytes(2048, 48, 5120, kq.KQ_W4_AFFINE_G64) == \
        al(2048 * 5120) + al(4 * 2048) + al(4 * 2048 * 80)
    # a split GEMM adds its int32 partial sums
    r = kq.kq_route(128, 3072, 12288, kq.KQ_W8_PER_CHANNEL)
    assert r["splits"] > 1
    assert kq.kq_workspace_bytes(128, 3072, 12288, kq.KQ_W8_PER_CHANNEL) == \
        al(128 * 12288) + al(4 * 128) + al(4 * r["splits"] * 128 * 3072)


@pytest.mark.parametrize("M,N,K,fmt,kind,tile,grid", [
    (1, 13824, 5120, kq.KQ_W4_AFFINE_G64, "fused", (2, 32), 432),   # lane GEMV quantizing x itself
    (2, 13824, 5120, kq.KQ_W4_AFFINE_G64, "fused", (2, 32), 432),
    (3, 13824, 5120, kq.KQ_W4_AFFINE_G64, "fused", (4, 32), 432),   # MFMA GEMV quantizing x itself
    (1, 13824, 6208, kq.KQ_W4_AFFINE_G64, "gemv", (16, 32), 432),   # past the lane kernel's K limit
    (4, 18432, 3072, kq.KQ_W8_PER_CHANNEL, "fused", (4, 16), 1152),  # int8: 16 columns
    (4, 512, 6208, kq.KQ_W8_PER_CHANNEL, "gemv", (16, 16), 32),      # past its K limit
    (5, 13824, 5120, kq.KQ_W4_AFFINE_G64, "gemv", (16, 32), 432),
    (16, 13824, 5120, kq.KQ_W4_AFFINE_G64, "gemv", (16, 32), 432),
    (4, 512, 16384, kq.KQ_W8_PER_CHANNEL, "gemv", (16, 16), 32),
    (4, 512, 16448, kq.KQ_W8_PER_CHANNEL, "gemm", None, None),
    (17, 13824, 5120, kq.KQ_W4_AFFINE_G64, "gemv", (16, 32), 432 * 2),  # two row blocks
    (32, 13824, 5120, kq.KQ_W8_PER_CHANNEL, "gemv", (16, 16), 864 * 2),
    (33, 13824, 5120, kq.KQ_W4_AFFINE_G64, "gemm", None, None),
    (4096, 3072, 3072, kq.KQ_W8_PER_CHANNEL, "gemm", (256, 192), 256),
    (16384, 12288, 3072, kq.KQ_W8_PER_CHANNEL, "gemm", (256, 256), 3072),  # 8-wave 256x256
    (2048, 12288, 4096, kq.KQ_W4_AFFINE_G64, "gemm", (128, 128), 1536),
    (2048, 4096, 12288, kq.KQ_W4_AFFINE_G64, "gemm", (128, 128), 512),
    (100, 640, 256, kq.KQ_W4_AFFINE_G64, "gemm", (64, 128), 10),
    (2048, 48, 5120, kq.KQ_W8_PER_CHANNEL, "fused", (8, 48), 256),   # thin N: one kernel
    (300, 64, 640, kq.KQ_W4_AFFINE_G64, "fused", (8, 64), 38),
    (17, 48, 5120, kq.KQ_W4_AFFINE_G64, "fused", (8, 48), 3),
    (16, 48, 5120, kq.KQ_W4_AFFINE_G64, "gemv", (16, 32), 2),         # one row block: GEMV
    (2048, 33, 6144, kq.KQ_W8_PER_CHANNEL, "fused", (8, 48), 256),
    (2048, 48, 6208, kq.KQ_W8_PER_CHANNEL, "gemv", (16, 16), 3 * 128),  # past the fused K limit
    (300, 65, 640, kq.KQ_W8_PER_CHANNEL, "gemm", (64, 64), 5 * 2),
    (2048, 48, 16448, kq.KQ_W8_PER_CHANNEL, "gemm", (64, 64), 32 * 8),  # 8 K slices
    (16 * 65535, 48, 6208, kq.KQ_W8_PER_CHANNEL, "gemv", (16, 16), 3 * 65535),
    (16 * 65535 + 1, 48, 6208, kq.KQ_W8_PER_CHANNEL, "gemm", None, None),  # grid y limit
    (16 * 65535 + 1, 32, 128, kq.KQ_W8_PER_CHANNEL, "fused", (8, 32), 131071),  # N <= 32: any M
    (8192, 64, 3072, kq.KQ_W8_PER_CHANNEL, "fused", (8, 64), 1024),   # M*N = 2^19
    (8193, 64, 3072, kq.KQ_W8_PER_CHANNEL, "gemv", (16, 16), 4 * 513),  # past it: two kernels
])
def test_route_decisions(M, N, K, fmt, kind, tile, grid, kq_env):
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_FUSE=None)
    r = kq.kq_route(M, N, K, fmt)
    assert r["kind"] == kind
    if tile is not None:
        assert (r["tile_m"], r["tile_n"]) == tile
        assert r["grid"] == grid


@pytest.mark.parametrize("M,N,K,tile,splits", [
    (128, 3072, 12288, (128, 128), 8),      # small-M prefill, long K
    (200, 1000, 65536, (128, 128), 16),
    (4, 512, 16448, (64, 64), 13),          # past the GEMV's K limit
    (4096, 3072, 3072, (256, 192), 1),      # a full grid never splits
    (16384, 12288, 3072, (256, 256), 1),
    (512, 3072, 3072, (64, 64), 1),         # short K: the partials would cost more
])
def test_split_k_decisions(M, N, K, tile, splits, kq_env):
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_SPLIT=None)
    r = kq.kq_route(M, N, K, kq.KQ_W8_PER_CHANNEL)
    assert (r["tile_m"], r["tile_n"]) == tile and r["splits"] == splits
    assert r["grid"] == ((M + tile[0] - 1) // tile[0]) * ((N + tile[1] - 1) // tile[1]) * splits


@pytest.mark.parametrize("M,N,K,tile,splits", [
    (128, 3072, 12288, (128, 128), 6),      # int4 slices are whole 16-group chunks
    (64, 4096, 4096, (64, 128), 4),
    (300, 640, 2112, (64, 128), 3),         # a one-group last slice
    (2048, 4096, 12288, (128, 128), 1),
])
def test_split_k_decisions_int4(M, N, K, tile, splits, kq_env):
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_SPLIT=None)
    r = kq.kq_route(M, N, K, kq.KQ_W4_AFFINE_G64)
    assert (r["tile_m"], r["tile_n"]) == tile and r["splits"] == splits


def test_split_k_lever(kq_env):
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_SPLIT="1")
    assert kq.kq_route(128, 3072, 12288, kq.KQ_W8_PER_CHANNEL)["splits"] == 1
    kq_env(KQ_SPLIT="4")
    r = kq.kq_route(4096, 3072, 3072, kq.KQ_W8_PER_CHANNEL)
    tiles = (4096 // r["tile_m"]) * (3072 // r["tile_n"])
    assert r["splits"] == 4 and r["grid"] == tiles * 4
    kq_env(KQ_SPLIT="16")
    assert kq.kq_route(64, 256, 320, kq.KQ_W8_PER_CHANNEL)["splits"] == 2  # 5 steps: slices of 4
    assert kq.kq_route(64, 256, 3200, kq.KQ_W4_AFFINE_G64)["splits"] == 4  # 50 groups: 16, 16, 16, 2
    kq_env(KQ_SPLIT="7")
    # 48 steps in slices of ceil(48/7) = 7 -> 8 steps: 6 slices
    assert kq.kq_route(4096, 3072, 3072, kq.KQ_W8_PER_CHANNEL)["splits"] == 6


def test_gemv_lane_lever(kq_env):
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_FUSE=None, KQ_GEMV_LANE="0")
    r = kq.kq_route(1, 13824, 5120, kq.KQ_W4_AFFINE_G64)
    assert (r["kind"], r["tile_m"], r["tile_n"], r["grid"]) == ("fused", 4, 32, 432)
    kq_env(KQ_GEMV_LANE=None, KQ_FORCE_ROUTE="gemv")
    r = kq.kq_route(2, 13824, 5120, kq.KQ_W4_AFFINE_G64)
    assert (r["kind"], r["tile_m"], r["tile_n"], r["grid"]) == ("gemv", 2, 32, 432)
    # int8 weights take it too (the int8 lane kernel)
    r = kq.kq_route(1, 13824, 5120, kq.KQ_W8_PER_CHANNEL)
    assert (r["kind"], r["tile_m"], r["tile_n"]) == ("gemv", 2, 32)
    r = kq.kq_route(3, 13824, 5120, kq.KQ_W8_PER_CHANNEL)
    assert (r["kind"], r["tile_m"], r["tile_n"]) == ("gemv", 16, 16)
    r = kq.kq_route(3, 13824, 5120, kq.KQ_W4_AFFINE_G64)
    assert (r["kind"], r["tile_m"], r["tile_n"]) == ("gemv", 16, 32)


def test_fused_route_lever(kq_env):
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE=None, KQ_FUSE="0")
    r = kq.kq_route(2048, 48, 5120, kq.KQ_W8_PER_CHANNEL)
    assert (r["kind"], r["grid"]) == ("gemv", 3 * 128)
    assert kq.kq_route(1, 13824, 5120, kq.KQ_W4_AFFINE_G64)["kind"] == "gemv"
    assert kq.kq_workspace_bytes(3, 3072, 64, kq.KQ_W8_PER_CHANNEL) == 1024 + 256
    kq_env(KQ_FUSE=None, KQ_FORCE_ROUTE="gemm")
    assert kq.kq_route(2048, 48, 5120, kq.KQ_W8_PER_CHANNEL)["kind"] == "gemm"


def test_route_levers(kq_env):
    kq_env(KQ_FORCE_ROUTE="gemm")
    assert kq.kq_route(4, 512, 512, kq.KQ_W4_AFFINE_G64)["kind"] == "gemm"
    kq_env(KQ_FORCE_ROUTE="gemv")
    assert kq.kq_route(4, 512, 512, kq.KQ_W8_PER_CHANNEL)["kind"] == "gemv"
    with pytest.raises(ValueError, match=r"\[kq_route\] M=32 exceeds the GEMV limit 16"):
        kq.kq_route(32, 512, 512, kq.KQ_W8_PER_CHANNEL)
    with pytest.raises(ValueError, match=r"\[kq_route\] K=16448 exceeds the GEMV limit 16384"):
        kq.kq_route(4, 512, 16448, kq.KQ_W8_PER_CHANNEL)
    kq_env(KQ_FORCE_ROUTE=None, KQ_TILE="128x128")
    r = kq.kq_route(4096, 3072, 3072, kq.KQ_W8_PER_CHANNEL)
    assert (r["tile_m"], r["tile_n"], r["grid"]) == (128, 128, 32 * 24)
    kq_env(KQ_TILE="256x256")
    r = kq.kq_route(4096, 3072, 3072, kq.KQ_W4_AFFINE_G64)
    assert (r["tile_m"], r["tile_n"]) == (128, 256)     # int4: nearest tile it has
    kq_env(KQ_TILE="64x64")
    r = kq.kq_route(4096, 3072, 3072, kq.KQ_W4_AFFINE_G64)
    assert (r["tile_m"], r["tile_n"], r["threads"]) == (64, 128, 256)
    kq_env(KQ_TILE="128x256")
    r = kq.kq_route(4096, 3072, 3072, kq.KQ_W8_PER_CHANNEL)
    assert (r["tile_m"], r["tile_n"]) == (256, 128)     # int8: same area
    # a tile the kernel has is taken as named, also where another tile has
    # the same area (the 4- and 8-wavefront 256x256 tiles)
    kq_env(KQ_TILE="256x256w8")
    r = kq.kq_route(1024, 1536, 1024, kq.KQ_W8_PER_CHANNEL)
    assert (r["tile_m"], r["tile_n"], r["threads"], r["grid"]) == (256, 256, 512, 24)
    kq_env(KQ_TILE="256x256")
    r = kq.kq_route(1024, 1536, 1024, kq.KQ_W8_PER_CHANNEL)
    assert (r["tile_m"], r["tile_n"], r["threads"]) == (256, 256, 256)


@pytest.mark.parametrize("K,msg", [
    (100, r"\[kq_route\] K=100 must be a positive multiple of 64"),
    (0, r"K=0 must be a positive multiple of 64"),
    (65536 + 64, r"K=65600 exceeds 65536"),
])
def test_route_rejects_unsupported_k(K, msg):
    with pytest.raises(ValueError, match=msg):
        kq.kq_route(64, 64, K, kq.KQ_W8_PER_CHANNEL)


def test_route_rejects_bad_enums_and_sizes():
    with pytest.raises(ValueError, match="unknown weight format 7"):
        kq.kq_route(64, 64, 64, 7)
    with pytest.raises(ValueError, match="unknown output dtype 9"):
        kq.kq_route(64, 64, 64, kq.KQ_W8_PER_CHANNEL, 9)
    with pytest.raises(ValueError, match="negative size"):
        kq.kq_route(-1, 64, 64, kq.KQ_W8_PER_CHANNEL)


# Raw C-ABI calls with fake (never dereferenced) device addresses.
P = ctypes.c_void_p


def _w8(M, K, N, x=16, w=32, sw=48, y=64, ws=80, wsb=1 << 30, dtype=kq.KQ_DTYPE_BF16):
    return kq.lib().kq_w8a8_linear(P(x), M, K, N, P(w), P(sw), None, P(y), dtype, P(ws), wsb, None)


def test_linear_validation_without_device():
    L = kq.lib()
    assert _w8(64, 100, 64) == kq.KQ_ERR_UNSUPPORTED
    assert "[kq_w8a8_linear] K=100 must be a positive multiple of 64" in kq.kq_last_error()
    assert _w8(0, 128, 64) == kq.KQ_SUCCESS          # empty: nothing enqueued
    assert _w8(64, 128, 0) == kq.KQ_SUCCESS
    assert _w8(64, 128, 64, x=0) == kq.KQ_ERR_INVALID_VALUE
    assert "null tensor pointer" in kq.kq_last_error()
    assert _w8(64, 128, 64, x=17) == kq.KQ_ERR_INVALID_VALUE
    assert "16-byte aligned" in kq.kq_last_error()
    assert _w8(64, 128, 64, wsb=100) == kq.KQ_ERR_WORKSPACE
    assert "smaller than the" in kq.kq_last_error()
    assert _w8(64, 128, 64, dtype=5) == kq.KQ_ERR_INVALID_VALUE
    # int4 needs the group offsets
    st = L.kq_w4a8_linear(P(16), 64, 128, 64, P(32), P(48), None, None, P(64),
                          kq.KQ_DTYPE_BF16, P(80), 1 << 30, None)
    assert st == kq.KQ_ERR_INVALID_VALUE and "group offsets" in kq.kq_last_error()
    # GEMV limit
    st = L.kq_gemv_small_m(kq.KQ_W4_AFFINE_G64, P(16), 17, 128, 64, P(32), P(48), P(64), None,
                           P(80), kq.KQ_DTYPE_BF16, P(96), 1 << 30, None)
    assert st == kq.KQ_ERR_UNSUPPORTED and "exceeds the GEMV limit 16" in kq.kq_last_error()
    st = L.kq_gemv_small_m(kq.KQ_W8_PER_CHANNEL, P(16), 4, 128, 64, P(32), P(48), P(64), None,
                           P(80), kq.KQ_DTYPE_BF16, P(96), 1 << 30, None)
    assert st == kq.KQ_ERR_INVALID_VALUE and "gbias must be NULL" in kq.kq_last_error()


def test_code_order_validation_without_device(monkeypatch):
    L = kq.lib()
    st = L.kq_quantize_act_ordered(P(16), 4, 128, P(32), P(48), None, 7, None)
    assert st == kq.KQ_ERR_INVALID_VALUE and "unknown code order 7" in kq.kq_last_error()
    st = L.kq_quantize_act_ordered(P(16), 4, 100, P(32), P(48), None, kq.KQ_CODES_SPLIT8, None)
    assert st == kq.KQ_ERR_UNSUPPORTED and "needs K % 8 == 0" in kq.kq_last_error()
    st = L.kq_quantize_act_ordered(P(16), 0, 104, P(32), P(48), None, kq.KQ_CODES_SPLIT8, None)
    assert st == kq.KQ_SUCCESS  # empty: nothing enqueued
    args = (P(16), P(32), P(48), 4, 128, 64, P(64), P(80), P(96), None, P(112), kq.KQ_DTYPE_BF16)
    assert L.kq_w4a8_gemm_ordered(*args, 9, None) == kq.KQ_ERR_INVALID_VALUE
    assert "unknown code order 9" in kq.kq_last_error()
    monkeypatch.setenv("KQ_FORCE_ROUTE", "gemv")
    assert L.kq_w4a8_gemm_ordered(*args, kq.KQ_CODES_SPLIT8, None) == kq.KQ_ERR_UNSUPPORTED
    assert "natural-order codes" in kq.kq_last_error()


def _gated(fmt=kq.KQ_W8_PER_CHANNEL, M=64, K=128, N=64, gbias=None, residual=None, gate=None,
           gate_rows=1, y=1 << 20, dtype=kq.KQ_DTYPE_BF16, wsb=1 << 30):
    return kq.lib().kq_linear_gated(fmt, P(16), M, K, N, P(32), P(48), P(gbias) if gbias else None,
                                    None, P(residual) if residual else None,
                                    P(gate) if gate else None, gate_rows, P(y), dtype, P(1 << 24),
                                    wsb, None)


def test_gated_linear_validation_without_device():
    assert _gated(dtype=kq.KQ_DTYPE_I32) == kq.KQ_ERR_UNSUPPORTED
    assert "writes f32 or bf16, not i32" in kq.kq_last_error()
    assert _gated(gate_rows=0, gate=64) == kq.KQ_ERR_INVALID_VALUE
    assert "gate_rows=0" in kq.kq_last_error()
    assert _gated(residual=(1 << 21) + 8) == kq.KQ_ERR_INVALID_VALUE
    assert "residual must be 16-byte aligned" in kq.kq_last_error()
    assert _gated(gate=(1 << 21) + 2) == kq.KQ_ERR_INVALID_VALUE
    assert "gate must be 4-byte aligned" in kq.kq_last_error()
    assert _gated(fmt=2) == kq.KQ_ERR_INVALID_VALUE
    assert _gated(gbias=64) == kq.KQ_ERR_INVALID_VALUE and "gbias must be NULL" in kq.kq_last_error()
    # a residual that overlaps y without being y (bf16 y of 64*64*2 bytes)
    assert _gated(residual=(1 << 20) + 4096) == kq.KQ_ERR_INVALID_VALUE
    assert "overlaps y" in kq.kq_last_error()
    assert _gated(residual=(1 << 20) - 4096) == kq.KQ_ERR_INVALID_VALUE
    # in place needs a bf16 output; a disjoint or in-place residual passes
    # the overlap checks and stops at the (too small) workspace instead
    assert _gated(residual=1 << 20, dtype=kq.KQ_DTYPE_F32) == kq.KQ_ERR_INVALID_VALUE
    assert "in-place residual needs a bf16 output" in kq.kq_last_error()
    for r in ((1 << 20) + 64 * 64 * 2, (1 << 20) - 64 * 64 * 2, 1 << 20):
        assert _gated(residual=r, wsb=100) == kq.KQ_ERR_WORKSPACE, r
    # the plain linears' checks still apply
    assert _gated(K=100) == kq.KQ_ERR_UNSUPPORTED
    assert _gated(fmt=kq.KQ_W4_AFFINE_G64) == kq.KQ_ERR_INVALID_VALUE
    assert "group offsets" in kq.kq_last_error()
    assert _gated(wsb=100) == kq.KQ_ERR_WORKSPACE
    assert _gated(M=0) == kq.KQ_SUCCESS


def test_sage_workspace_layout():
    lay = kq.kq_sage_workspace_layout(2, 3, 300, 777)
    assert lay["lq_pad"] == 384 and lay["lk_pad"] == 896 and lay["chunks"] == 4
    order = ["qc", "sq", "kc", "sk", "vt", "kmean", "colsum", "meta"]
    sizes = {"qc": 6 * 384 * 128, "sq": 6 * 384 * 4, "kc": 6 * 896 * 128, "sk": 6 * 896 * 4,
             "vt": 6 * 896 * 128 * 2, "kmean": 6 * 128 * 4, "colsum": 6 * 4 * 128 * 8,
             "meta": 16}
    for a, b in zip(order, order[1:] + ["total"]):
        assert lay[a] % 256 == 0 and lay[b] - lay[a] >= sizes[a] and lay[b] - lay[a] < sizes[a] + 256
    with pytest.raises(ValueError):
        kq.kq_sage_workspace_layout(1, 70000, 10, 10)


def _sage(B=1, H=2, Lq=64, Lk=64, D=128, layout=0, scale=0.1, qb=128, kb=64, q=16, k=32, v=48,
          out=64, ws=1 << 20, wsb=1 << 40):
    return kq.lib().kq_sage_attention(P(q), P(k), P(v), P(out), B, H, Lq, Lk, D, layout, scale, qb, kb,
                                      P(ws), wsb, None)


def test_sage_validation_without_device():
    L = kq.lib()
    assert _sage(D=64) == kq.KQ_ERR_UNSUPPORTED and "only 128" in kq.kq_last_error()
    assert _sage(layout=2) == kq.KQ_ERR_INVALID_VALUE and "unknown layout" in kq.kq_last_error()
    assert _sage(qb=3) == kq.KQ_ERR_UNSUPPORTED and "powers of two" in kq.kq_last_error()
    assert _sage(kb=256) == kq.KQ_ERR_UNSUPPORTED
    assert _sage(scale=0.0) == kq.KQ_ERR_INVALID_VALUE and "scale" in kq.kq_last_error()
    assert _sage(scale=-1.0) == kq.KQ_ERR_INVALID_VALUE
    assert _sage(scale=float("inf")) == kq.KQ_ERR_INVALID_VALUE
    assert _sage(Lk=0) == kq.KQ_ERR_INVALID_VALUE and "no keys" in kq.kq_last_error()
    assert _sage(B=0) == kq.KQ_SUCCESS and _sage(Lq=0) == kq.KQ_SUCCESS and _sage(H=0) == kq.KQ_SUCCESS
    assert _sage(Lq=-1) == kq.KQ_ERR_INVALID_VALUE
    assert _sage(B=300, H=300) == kq.KQ_ERR_UNSUPPORTED
    assert _sage(Lk=(1 << 22) + 1) == kq.KQ_ERR_UNSUPPORTED
    assert _sage(q=0) == kq.KQ_ERR_INVALID_VALUE and "null" in kq.kq_last_error()
    assert _sage(v=40) == kq.KQ_ERR_INVALID_VALUE and "aligned" in kq.kq_last_error()
    assert _sage(out=72) == kq.KQ_ERR_INVALID_VALUE and "aligned" in kq.kq_last_error()
    assert _sage(wsb=100) == kq.KQ_ERR_WORKSPACE and "smaller than" in kq.kq_last_error()
    assert _sage(ws=0) == kq.KQ_ERR_WORKSPACE
    st = L.kq_sage_attend(P(16), 1 << 40, P(32), 1, 2, 64, 64, 128, 0, 0.0, 64, None)
    assert st == kq.KQ_ERR_INVALID_VALUE and "[kq_sage_attend] scale" in kq.kq_last_error()
    st = L.kq_sage_attend(P(16), 1 << 40, P(32), 1, 2, 64, 64, 128, 0, 0.1, 96, None)
    assert st == kq.KQ_ERR_UNSUPPORTED and "k_block=96" in kq.kq_last_error()
    st = L.kq_sage_prepare(P(16), P(32), P(48), 1, 2, 64, 64, 128, 0, 5, 64, P(64), 1 << 40, None)
    assert st == kq.KQ_ERR_UNSUPPORTED and "[kq_sage_prepare]" in kq.kq_last_error()
    st = L.kq_sage_prepare(P(16), P(32), P(48), 1, 2, 64, 64, 128, 0, 8, 64, P(64), 10, None)
    assert st == kq.KQ_ERR_WORKSPACE


def test_quantizer_validation_without_device():
    L = kq.lib()
    assert L.kq_quantize_act(P(16), 4, 0, P(32), P(48), None, None) == kq.KQ_ERR_UNSUPPORTED
    assert L.kq_quantize_act(P(16), 4, 100, P(32), P(48), P(64), None) == kq.KQ_ERR_UNSUPPORTED
    assert "group sums need K % 64 == 0" in kq.kq_last_error()
    assert L.kq_quantize_act(P(16), 0, 100, P(32), P(48), None, None) == kq.KQ_SUCCESS
    assert L.kq_quantize_act(None, 4, 64, P(32), P(48), None, None) == kq.KQ_ERR_INVALID_VALUE
    assert L.kq_quantize_weights(P(16), 4, 100, kq.KQ_W4_AFFINE_G64, P(32), P(48), P(64),
                                 None) == kq.KQ_ERR_UNSUPPORTED
    assert L.kq_quantize_weights(P(16), 4, 64, kq.KQ_W8_PER_CHANNEL, P(32), P(48), P(64),
                                 None) == kq.KQ_ERR_INVALID_VALUE
    assert L.kq_quantize_weights(P(16), 4, 64, 3, P(32), P(48), None, None) == kq.KQ_ERR_INVALID_VALUE
    assert L.kq_quantize_weights(P(16), 0, 64, kq.KQ_W8_PER_CHANNEL, P(32), P(48), None,
                                 None) == kq.KQ_SUCCESS


def test_last_error_is_per_thread():
    import threading
    _w8(64, 100, 64)
    seen = {}

    def other():
        seen["msg"] = kq.kq_last_error()
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "K=100" in kq.kq_last_error()


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(kq, "_lib", None)
    monkeypatch.setattr(kq, "_LIB_PATH", "/nonexistent/libkq.so")
    with pytest.raises(kq.KqError, match="not built"):
        kq.lib()
