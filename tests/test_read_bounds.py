"""CPU model of the GEMM kernels' buffer-descriptor reads.

The tiled GEMMs move operand rows global -> LDS through buffer descriptors
rebased on the tile's first row and the K slice's first code; a read at an
offset at or past the descriptor's num_records returns zero instead of
touching memory.  This models the descriptor arithmetic of gemm_w8a8.hip
and gemm_w4a8.hip for every tile and forced slice count, and checks that
(1) every byte fetched from memory lies inside the operand buffer, and
(2) every byte the products use lies below num_records (nothing needed is
zeroed).  Pure host arithmetic, no GPU.
"""
import pytest

# (BM, BN) of the int8 tiles and of the int4 tiles
W8_TILES = [(256, 256), (256, 192), (256, 128), (128, 128), (64, 64)]
W4_TILES = [(128, 256), (128, 128), (64, 128)]


def split_chunk(K, want, unit):
    """Slices of `chunk` codes, a multiple of `unit` (kq_route.cpp)."""
    units = -(-K // unit)
    if want < 2 or units < 2:
        return 1, K
    per = -(-units // want)
    chunk = per * unit
    return -(-K // chunk), chunk


def _check(rows_total, stride, row0, rows_valid, base_shift, num_records, reads, used):
    """reads / used: iterables of (row, byte offset within the slice's row)."""
    size = rows_total * stride
    base = row0 * stride + base_shift
    for r, off in reads:
        rel = r * stride + off
        if rel < num_records:               # fetched from memory
            a = base + rel
            assert 0 <= a < size, (r, off, a, size)
    for r, off in used:
        assert r < rows_valid
        assert r * stride + off < num_records, (r, off, num_records)


def _w8_case(M, N, K, BM, BN, splits):
    sp, kchunk = split_chunk(K, splits, 256)
    for y in range(sp):
        k0 = y * kchunk
        KT = min(kchunk, K - k0) // 64
        last = max(0, (KT - 1) >> 1) * 128   # pairs past the end re-load the last pair
        for rows_total, B, t in ((M, BM, "a"), (N, BN, "w")):
            for t0 in range(0, rows_total, B):
                rows = min(B, rows_total - t0)
                nrec = rows * K - k0
                # every pair buffer load reads 128 bytes of each of the tile's
                # rows at ks = 0, 128, ..., last (the odd tail's second half
                # included); rows past the edge lie past num_records
                ends = [(r, last + 127) for r in range(B)] + [(r, last) for r in range(B)]
                used = [(r, KT * 64 - 1) for r in range(rows)] + [(r, 0) for r in range(rows)]
                _check(rows_total, K, t0, rows, k0, nrec, ends, used)


def _w4_case(M, N, K, BM, BN, splits):
    sp, chunk = split_chunk(K, splits, 1024)
    gchunk = chunk // 64
    G_all = K // 64
    for y in range(sp):
        g0 = y * gchunk
        G = min(gchunk, G_all - g0)
        for rows_total, B, stride, per_group in ((M, BM, K, 64), (N, BN, K // 2, 32)):
            for t0 in range(0, rows_total, B):
                rows = min(B, rows_total - t0)
                nrec = rows * stride - g0 * per_group
                # steps past the slice re-load its last group
                ends = [(r, G * per_group - 1) for r in range(B)]
                used = [(r, G * per_group - 1) for r in range(rows)] + [(r, 0) for r in range(rows)]
                _check(rows_total, stride, t0, rows, g0 * per_group, nrec, ends, used)


SHAPES = [(1, 64, 64), (70, 130, 1088), (300, 200, 1344), (256, 192, 4096), (129, 257, 12288),
          (64, 48, 5120), (17, 1000, 2112)]


@pytest.mark.parametrize("tile", W8_TILES)
@pytest.mark.parametrize("splits", [1, 2, 3, 4, 7, 16])
def test_w8a8_reads_stay_in_the_operands(tile, splits):
    for M, N, K in SHAPES:
        _w8_case(M, N, K, *tile, splits)


@pytest.mark.parametrize("tile", W4_TILES)
@pytest.mark.parametrize("splits", [1, 2, 3, 5, 12])
def test_w4a8_reads_stay_in_the_operands(tile, splits):
    for M, N, K in SHAPES:
        _w4_case(M, N, K, *tile, splits)


def test_unfixed_descriptor_is_caught():
    # the descriptor before the fix (num_records = rows*K with the base moved
    # by k0) lets the dead half of an odd last slice fetch past the buffer
    M, N, K, BM, BN = 64, 64, 1088, 64, 64
    sp, kchunk = split_chunk(K, 2, 256)
    k0 = (sp - 1) * kchunk
    KT = (K - k0) // 64
    assert KT % 2 == 1
    last = ((KT - 1) >> 1) * 128
    with pytest.raises(AssertionError):
        _check(N, K, 0, N, k0, N * K, [(N - 1, last + 127)], [])


# Lane-per-column GEMVs (gemv.hip, M <= 2, int4 or int8 weights): wavefront w of a
# workgroup takes the 8 columns nw = 32*block + 8*(w % 4) .. +8 and K slice
# w / 4 of each row's 128-byte lines.  Its descriptor starts at row
# min(nw, N-1) with num_records = max(0, min(8, N - nw)) * row bytes (K/2 or
# K); lane (c, p) reads 16 bytes at c*rowbytes + 128*(l0 + i) + 16p for i < its line count, and
# lines past its share get an offset past num_records.
def _lane_gemv_case(N, K, slices=2, w8=False):
    G = K // 64
    QB = K if w8 else K // 2   # bytes per weight row
    nl = -(-QB // 128)
    nlh = -(-nl // slices)
    for blk in range(-(-N // 32)):
        for w in range(4 * slices):
            cw, kh = w % 4, w // 4
            nw = 32 * blk + 8 * cw
            row0 = min(nw, N - 1)
            nrec = max(0, min(8, N - nw)) * QB
            l0 = kh * nlh
            nlw = max(0, min(nlh, nl - l0))
            reads, used = [], []
            for c in range(8):
                for p in range(8):
                    for i in range(nlw):
                        off = c * QB + 128 * (l0 + i) + 16 * p
                        reads += [(0, off), (0, off + 15)]
                        byte = 128 * (l0 + i) + 16 * p  # first byte of the piece in the row
                        if nw + c < N and byte < QB:
                            used.append((c, byte + 15))
            _check(N, QB, row0, 8, 0, nrec, reads, [])
            for c, off in used:  # every byte a used group needs lies below num_records
                assert c * QB + off < nrec, (N, K, blk, w, c, off)
                assert (row0 + c) * QB + off < N * QB


@pytest.mark.parametrize("N,K", [(1, 64), (16, 128), (33, 320), (200, 1088), (100, 6144),
                                 (13824, 5120), (40, 4160), (8, 2112)])
@pytest.mark.parametrize("w8", [False, True])
def test_lane_gemv_reads_stay_in_the_weights(N, K, w8):
    _lane_gemv_case(N, K, w8=w8)


# int4 MFMA GEMV (gemv.hip, M >= 3 or K > 6144): a workgroup owns 32 columns
# (two blocks of 16) and 8 wavefronts split the K groups into slices of
# `per` groups (rounded to the 2-group load unit for int4).  Weights: the
# descriptor starts at column n0 with num_records = cols * RB; lane (q, c)
# of unit u reads 16 bytes at c*RB + UB*g0 + 16q + 16*b*RB + UB*GU*u for
# column block b, units past the wavefront's share at an offset past
# num_records.  Activation codes in fragment order: the descriptor starts at
# the 16-row block (G KB each) with num_records = G*1024; lane l of group g
# reads 16 bytes at 1024*g + 16*l.
def _reg_gemv_case(M, N, K, w4):
    G = K // 64
    RB = K // 2 if w4 else K
    UB, GU = (32, 2) if w4 else (64, 1)
    per = (-(-G // 8) + GU - 1) // GU * GU
    for blk in range(-(-N // 32)):
        n0 = 32 * blk
        cols = min(32, N - n0)
        nrec = cols * RB
        for w in range(8):
            g0 = min(w * per, G)
            gn = min(per, G - g0)
            nu = -(-gn // GU)
            for u in range(nu):
                for lane in range(64):
                    q, c = lane >> 4, lane & 15
                    for b in range(2):
                        off = c * RB + UB * g0 + 16 * q + 16 * b * RB + UB * GU * u
                        if off < nrec:  # fetched: inside the weight buffer
                            assert 0 <= n0 * RB + off and n0 * RB + off + 15 < N * RB
                        col = 16 * b + c
                        byte = UB * (g0 + GU * u) + 16 * q  # first byte in the column's row
                        g = (g0 + GU * u) + (16 * q) // UB   # the group those bytes hold
                        if col < cols and g < G and g - g0 < gn:  # used: the right column's row
                            assert byte + 15 < RB and col * RB + byte + 15 < nrec
        for mb in range(-(-M // 16)):
            for g in range(G):
                for lane in range(64):
                    off = 1024 * g + 16 * lane
                    assert off + 15 < G * 1024
                    assert mb * G * 1024 + off + 15 < (-(-M // 16) * 16) * K


@pytest.mark.parametrize("M,N,K", [(3, 13824, 5120), (16, 48, 5120), (17, 40, 6208), (5, 33, 64),
                                   (32, 100, 16384), (4, 64, 1088)])
def test_mfma_gemv_reads_stay_in_the_operands(M, N, K):
    _reg_gemv_case(M, N, K, True)
