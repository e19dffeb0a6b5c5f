"""GPU test: every route of the linears, the gated residual linear, the
allocation-free entry point and the INT8 attention, captured once in a HIP
graph and replayed several times, each replay checked bit for bit against
the eager call (the benchmark times such replays).  Between replays the
program runs its own eager work: the outputs are overwritten with a poison
pattern, in-place operands are restored, and other calls run on other
buffers; the host synchronizes around every replay."""
import numpy as np
import pytest
import torch

import synth
import w8a8_gemm_dit_amd as kq

pytestmark = pytest.mark.gpu

REPLAYS = 3

# (fmt, M, K, N, out, tile): one case per route kind -- the tiled GEMM on
# every tile the benchmarks take (pinned with KQ_TILE where the route would
# pick another at this size), split K (also on the 4-buffer ring: 128x128
# tiles, eight slices of 24 K steps, one workgroup per CU), the GEMV, the
# GEMV quantizing in its prologue, the lane GEMVs and fused thin N, for both
# weight formats
LINEAR_CASES = [
    ("w8", 1000, 1024, 768, "bf16", None),
    ("w8", 1024, 1024, 1536, "bf16", "256x256w8"),
    ("w8", 1024, 1024, 1536, "f32", "256x192"),
    ("w8", 128, 12288, 384, "bf16", None),
    ("w8", 128, 12288, 3072, "bf16", None),
    ("w8", 10, 2048, 1000, "f32", None),
    ("w8", 3, 1024, 4096, "bf16", None),
    ("w8", 2, 3072, 2048, "bf16", None),
    ("w8", 200, 1024, 48, "f32", None),
    ("w4", 512, 1024, 1024, "bf16", None),
    ("w4", 512, 1024, 1024, "bf16", "128x128"),
    ("w4", 512, 1024, 1024, "f32", "128x256"),
    ("w4", 128, 3072, 2048, "f32", None),
    ("w4", 16, 1024, 2048, "bf16", None),
    ("w4", 4, 1024, 2048, "f32", None),
    ("w4", 1, 2048, 1024, "bf16", None),
    ("w4", 300, 1024, 64, "bf16", None),
]

_DT = {"bf16": torch.bfloat16, "f32": torch.float32}
_FMT = {"w8": kq.KQ_W8_PER_CHANNEL, "w4": kq.KQ_W4_AFFINE_G64}


def _bits(t):
    return t.view(torch.int16) if t.dtype in (torch.bfloat16, torch.float16) else t.view(torch.int32)


def _poison(t):
    # a pattern no kernel writes: all bits set (a NaN in every float type)
    _bits(t).fill_(-1)


def _replay_and_check(call, outs, restore=None, other=None, tag=""):
    """Eager call -> reference; capture `call` once; REPLAYS replays, each
    after eager poisoning (and `restore`, `other`), each compared bitwise."""
    if restore:
        restore()
    call()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        if restore:
            restore()
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        for o in outs:
            _poison(o)
        if restore:
            restore()
        if other:
            other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, rf) in enumerate(zip(outs, ref)):
            same = torch.equal(_bits(o), _bits(rf))
            assert same, f"{tag}: replay {r} output {i} differs from the eager call"
    del g
    # the eager call still gives the same result after the replays
    for o in outs:
        _poison(o)
    if restore:
        restore()
    call()
    torch.cuda.synchronize()
    for o, rf in zip(outs, ref):
        assert torch.equal(_bits(o), _bits(rf)), f"{tag}: eager call after the replays differs"


def _linear_operands(fmt, M, K, N, seed):
    xb = synth.random_bf16((M, K), seed=seed, dist="student_t4")
    w = synth.random_f32((N, K), seed=seed + 1, scale=0.02)
    b = synth.random_f32((N,), seed=seed + 2, scale=0.1)
    x = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    wq, sc, gb = kq.kq_quantize_weights(torch.from_numpy(w).cuda(), _FMT[fmt])
    return x, wq, sc, gb, torch.from_numpy(b).cuda()


def _linear(fmt, x, wq, sc, gb, b, dt, y, ws):
    if fmt == "w8":
        return kq.kq_w8a8_linear(x, wq, sc, b, out_dtype=dt, out=y, workspace=ws)
    return kq.kq_w4a8_linear(x, wq, sc, gb, b, out_dtype=dt, out=y, workspace=ws)


@pytest.mark.parametrize("fmt,M,K,N,out,tile", LINEAR_CASES)
def test_linear_graph_replays_match_eager(fmt, M, K, N, out, tile, kq_env):
    kq_env(KQ_TILE=tile)
    route = kq.kq_route(M, N, K, _FMT[fmt])
    tag = (f"{fmt} {M}x{K}->{N} {out} route={route['kind']} tile={route['tile_m']}x"
           f"{route['tile_n']}/{route['threads']} splits={route['splits']}")
    print(f"[graph] {tag}", flush=True)
    x, wq, sc, gb, b = _linear_operands(fmt, M, K, N, 4100 + M + N)
    dt = _DT[out]
    y = torch.empty((M, N), dtype=dt, device="cuda")
    ws = torch.empty((max(1, kq.kq_workspace_bytes(M, N, K, _FMT[fmt])),), dtype=torch.uint8,
                     device="cuda")
    # eager work between replays: the same linear on other inputs and buffers
    x2 = torch.flip(x, dims=[0]).contiguous()
    y2 = torch.empty_like(y)
    ws2 = torch.empty_like(ws)
    _replay_and_check(lambda: _linear(fmt, x, wq, sc, gb, b, dt, y, ws), [y],
                      other=lambda: _linear(fmt, x2, wq, sc, gb, b, dt, y2, ws2), tag=tag)


@pytest.mark.parametrize("fmt,M,K,N", [("w8", 512, 1024, 768), ("w4", 256, 1024, 512),
                                       ("w8", 8, 2048, 1024)])
def test_gated_in_place_graph_replays_match_eager(fmt, M, K, N):
    """out = residual + gate * linear(x) in place: the residual is restored
    eagerly before every replay."""
    tag = f"gated {fmt} {M}x{K}->{N}"
    print(f"[graph] {tag}", flush=True)
    x, wq, sc, gb, b = _linear_operands(fmt, M, K, N, 5200 + M)
    L = 64
    res0 = torch.from_numpy(synth.random_bf16((M, N), seed=5300 + M).view(np.int16)).cuda().view(
        torch.bfloat16)
    gate = torch.from_numpy(synth.random_f32((-(-M // L), N), seed=5400 + M, scale=0.5)).cuda()
    res = res0.clone()
    ws = torch.empty((max(1, kq.kq_workspace_bytes(M, N, K, _FMT[fmt])),), dtype=torch.uint8,
                     device="cuda")

    def call():
        kq.kq_linear_gated(_FMT[fmt], x, wq, sc, gb if fmt == "w4" else None, b, residual=res,
                           gate=gate, gate_rows=L, out_dtype=torch.bfloat16, out=res, workspace=ws)

    _replay_and_check(call, [res], restore=lambda: res.copy_(res0), tag=tag)


def test_noalloc_graph_replays_match_eager():
    """The allocation-free W8A8 linear (the library's own scratch) under
    capture, on a GEMM shape and on a split-K shape."""
    for i, (M, K, N) in enumerate([(1000, 1024, 768), (128, 12288, 384)]):
        tag = f"noalloc {M}x{K}->{N}"
        print(f"[graph] {tag}", flush=True)
        x, wq, sc, _, b = _linear_operands("w8", M, K, N, 6100 + i)
        y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        _replay_and_check(lambda: kq.kq_w8a8_linear_noalloc(x, wq, sc, b, out=y), [y], tag=tag)


@pytest.mark.parametrize("k_block", [64, 1])
def test_attention_graph_replays_match_eager(k_block):
    tag = f"attention 1x2x300 k_block={k_block}"
    print(f"[graph] {tag}", flush=True)
    rng = np.random.default_rng(7100 + k_block)
    q, k, v = (torch.from_numpy(rng.standard_normal((1, 2, 300, 128)).astype(np.float16)).cuda()
               for _ in range(3))
    out = torch.empty_like(q)
    ws = kq.kq_sage_prepare(q, k, v, 128, k_block)
    q2 = torch.flip(q, dims=[2]).contiguous()
    out2 = torch.empty_like(q)
    ws2 = torch.empty_like(ws)
    _replay_and_check(
        lambda: kq.kq_sage_attention(q, k, v, k_block=k_block, out=out, workspace=ws), [out],
        other=lambda: kq.kq_sage_attention(q2, k, v, k_block=k_block, out=out2, workspace=ws2),
        tag=tag)
