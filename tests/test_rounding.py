"""The int8 code identity the quantizing kernels use, checked exhaustively on
the CPU in IEEE fp32 (numpy: every multiply and add rounds once, as in the
kernels, which compile these two operations without contraction).

With inv = fp32(127 / amax), for every finite bf16 x with |x| <= amax:
the low byte of the fp32 sum fp32(x * inv) + 1.5 * 2^23 is the two's
complement of clamp(rint(fp32(x * inv)), -127, 127), the quantizer's rule:
the sum is exact at spacing 1 and rounds half to even, and |x * inv| stays
below 127.5, so the clamp never binds.  Also: the max of |x| taken on the
bf16 magnitude bits (x & 0x7FFF) is the max of |x| as floats."""
import numpy as np

SHIFT = np.float32(12582912.0)  # 1.5 * 2^23


def _all_finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32)
    exp = (bits >> 7) & 0xFF
    bits = bits[exp != 0xFF]                      # drop inf / nan
    return bits, (bits << 16).view(np.float32)


def _rule(x, inv):
    with np.errstate(over="ignore", invalid="ignore"):
        p = (x * inv).astype(np.float32)
    return np.clip(np.rint(p), -127, 127).astype(np.int32)


def _shift_codes(x, inv):
    with np.errstate(over="ignore", invalid="ignore"):
        p = (x * inv).astype(np.float32)
        t = (p + SHIFT).astype(np.float32)
    return (t.view(np.uint32) & 0xFF).astype(np.uint8).view(np.int8).astype(np.int32)


def test_shift_rounding_matches_the_rule_for_every_bf16_value():
    bits, x = _all_finite_bf16()
    ax = np.abs(x)
    rng = np.random.default_rng(0)
    # amax values: every power of two in range, random bf16 magnitudes
    # (normal and subnormal), the largest finite bf16, and values whose
    # 127/amax rounds up or down
    amaxes = [np.float32(2.0) ** e for e in range(-133, 128)]
    pick = rng.choice(np.flatnonzero(ax > 0), size=300, replace=False)
    amaxes += list(ax[pick])
    amaxes += [ax.max(), np.float32(127.0), np.float32(1.0) / np.float32(3.0)]
    checked = 0
    for amax in amaxes:
        amax = np.float32(amax)
        with np.errstate(over="ignore", divide="ignore"):
            inv = np.float32(np.float32(127.0) / amax)
        if not np.isfinite(inv):
            inv = np.float32(0.0)              # the rule's zero row
        sel = ax <= amax
        xs = x[sel]
        got = _shift_codes(xs, inv)
        want = _rule(xs, inv)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (f"amax {amax!r} inv {inv!r}: x {xs[bad[0]]!r} "
                               f"gives {got[bad[0]]} instead of {want[bad[0]]}")
        # the clamp never binds within |x| <= amax
        with np.errstate(over="ignore", invalid="ignore"):
            assert np.all(np.abs(np.rint((xs * inv).astype(np.float32))) <= 127)
        checked += xs.size
    assert checked > 10_000_000


def test_ties_round_to_even():
    # x * inv landing exactly on k + 1/2 rounds to the even neighbour
    inv = np.float32(1.0)
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, -126.5], np.float32)
    assert _shift_codes(x, inv).tolist() == [0, 2, 2, 0, -2, -2, 126, -126]


def test_magnitude_bits_order_as_abs():
    bits, x = _all_finite_bf16()
    mag = bits & 0x7FFF
    order_bits = np.argsort(mag, kind="stable")
    a = np.abs(x)[order_bits]
    assert np.all(np.diff(a) >= 0)             # nondecreasing along the bit order
    # and the max of the bits is the bits of the max (signed zeros included)
    rng = np.random.default_rng(1)
    for _ in range(200):
        idx = rng.choice(bits.size, size=64)
        m = mag[idx].max()
        assert (np.uint32(m) << 16).view(np.float32) == np.abs(x[idx]).max()
