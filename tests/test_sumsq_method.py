"""Host checks of the RMSNorm mean square: the fast exact sum of squares
(quant.hip: sq_add, round128).  The kernel adds every x^2 as an integer
relative to the row's largest exponent bin, in 128 bits, cutting the bits of
very small terms below the unit and flagging the cut; it then rounds to
binary64 unless the cut could carry into the rounding position, in which
case the kernel falls back to its exponent-bin sum.

The method is restated here with explicit 64-bit arithmetic and checked
against the exact rational sum (fractions.Fraction; float(Fraction) is
correctly rounded) on random rows, rows spanning the whole exponent range,
subnormal rows, and on the rounding step itself with the extreme values the
cut part can take."""
import struct
from fractions import Fraction

import numpy as np
import pytest

M64 = (1 << 64) - 1


def bin_of(x):
    u = struct.unpack("<I", struct.pack("<f", float(x)))[0] & 0x7FFFFFFF
    e, f = u >> 23, u & 0x7FFFFF
    if e == 255:
        return 254, 0
    return (e if e else 1), ((f | 0x800000) if e else f)


def sq_add(x, bmax, acc):
    lo, hi, cut = acc
    b, m = bin_of(x)
    if not m:
        return acc
    sq = m * m
    s = 2 * (b - bmax) + 62
    add_lo = add_hi = 0
    if s >= 0:
        add_lo = (sq << s) & M64
        add_hi = (sq >> (64 - s)) if s > 16 else 0
    elif s > -48:
        add_lo = sq >> (-s)
        cut = cut or (sq & ((1 << (-s)) - 1)) != 0
    else:
        cut = True
    lo = (lo + add_lo) & M64
    hi = (hi + add_hi + (1 if lo < add_lo else 0)) & M64
    return lo, hi, cut


def shr128(lo, hi, k):
    return (((hi << 64) | lo) >> k) & M64


def round128(lo, hi, cut, L):
    """(ok, value) as the kernel computes them."""
    if hi == 0 and lo == 0:
        return (not cut), 0.0
    a = (hi << 64) | lo
    P = a.bit_length() - 1
    if P <= 52:
        return (not cut), float(Fraction(a) * Fraction(2) ** L)
    rp = P - 53
    if cut:
        if rp <= 16:
            return False, None
        mid = shr128(lo, hi, 16) & ((1 << (rp - 16)) - 1)
        if mid == (1 << (rp - 16)) - 1:
            return False, None
    mant = shr128(lo, hi, rp + 1) & ((1 << 53) - 1)
    rnd = (shr128(lo, hi, rp) & 1) != 0
    below = cut
    if rp >= 64:
        below = below or lo != 0 or (hi & ((1 << (rp - 64)) - 1)) != 0
    elif rp > 0:
        below = below or (lo & ((1 << rp) - 1)) != 0
    e = rp + 1 + L
    if rnd and (below or (mant & 1)):
        mant += 1
        if mant == 1 << 53:
            mant >>= 1
            e += 1
    return True, float(Fraction(mant) * Fraction(2) ** e)


def fast_sumsq(row):
    bmax = 0
    for x in row:
        b, m = bin_of(x)
        if m:
            bmax = max(bmax, b)
    acc = (0, 0, False)
    for x in row:
        acc = sq_add(x, bmax, acc)
    return round128(acc[0], acc[1], acc[2], 2 * (bmax - 150) - 62)


def exact_sumsq(row):
    return float(sum(Fraction(float(x)) ** 2 for x in row))


def rows():
    rng = np.random.default_rng(7)
    yield rng.standard_normal(2560).astype(np.float32)
    yield (rng.standard_normal(6912) * 20).astype(np.float32)
    # every binade of the format, one row
    e = rng.integers(-149, 128, size=4096)
    yield (rng.uniform(1, 2, size=4096) * np.exp2(e.astype(np.float64))).astype(np.float32)
    # a few huge values among many tiny ones (terms cut below the unit)
    r = (rng.standard_normal(3000) * 1e-30).astype(np.float32)
    r[::700] = 3e18
    yield r
    # subnormals only
    yield (rng.uniform(-1, 1, size=1000) * 1e-39).astype(np.float32)
    yield np.zeros(64, np.float32)
    yield np.array([np.float32(2.0 ** -149)] * 5 + [np.float32(1.0)], np.float32)


@pytest.mark.parametrize("i", range(7))
def test_fast_sum_of_squares_is_the_rounded_exact_sum(i):
    row = list(rows())[i]
    ok, v = fast_sumsq(row)
    assert ok
    assert v == exact_sumsq(row)


def test_rounding_step_is_safe_for_every_cut_value():
    """Whenever round128 decides, the result equals the rounding of
    (A + R) * 2^L for the smallest and largest R the cut terms can add."""
    rng = np.random.default_rng(11)
    L = -300
    decided = undecided = 0
    for t in range(4000):
        top = int(rng.integers(108, 126))
        a = (1 << top) | int(rng.integers(0, 1 << 62)) << max(0, top - 62) | int(rng.integers(0, 1 << 40))
        if t % 4 == 0:  # force a run of ones above bit 16 (the carry-prone case)
            rp = top - 53
            a |= ((1 << rp) - 1) & ~((1 << 16) - 1)
        a &= (1 << 127) - 1
        lo, hi = a & M64, a >> 64
        ok, v = round128(lo, hi, True, L)
        if not ok:
            undecided += 1
            continue
        decided += 1
        for r in (1, (1 << 16) - 1):
            assert v == float(Fraction(a + r) * Fraction(2) ** L)
    assert decided > 2000 and undecided > 500


# ---------------------------------------------------------------------------
# The RMSNorm mean square (bl_device.h, block_meansq): a binary64 sum of the
# squares decides ms = binary32(binary64(S) / D) directly unless S / D lies
# within 2^-35 of a binary32 rounding midpoint; then the exact sum decides.

def meansq_fast(row, rng):
    """(decided, value) as the kernel's fast path computes them, with the
    binary64 additions in a random order (the kernel's order differs)."""
    sq = np.asarray(row, np.float64) ** 2
    a = 0.0
    for v in sq[rng.permutation(len(sq))]:
        a += float(v)
    D = len(row)
    qa = a * (1.0 / D)  # the kernel multiplies by the binary64 reciprocal
    with np.errstate(over="ignore"):
        c = np.float32(qa)
    cb = int(c.view(np.uint32))
    if not np.isfinite(c) or cb == 0 or cb >= 0x7F7FFFFF:
        return False, None
    lo = 0.5 * (float(c) + float(np.uint32(cb - 1).view(np.float32)))
    hi = 0.5 * (float(c) + float(np.uint32(cb + 1).view(np.float32)))
    tol = qa * 2.0 ** -35
    if qa - lo > tol and hi - qa > tol:
        return True, float(c)
    return False, None


def meansq_exact(row):
    s = float(sum(Fraction(float(x)) ** 2 for x in row))  # RN64 of the exact sum
    return float(np.float32(s / len(row)))  # RN64 of the quotient, then RN32


def near_midpoint_rows(rng, count, D=2560):
    """Rows whose exact mean square is pushed onto a binary32 midpoint, or to
    a few times the tolerance on either side of it, by re-solving the largest
    and then a small element: the fast path must not decide them wrongly."""
    offsets = [0, 0, 2.0 ** -34, -(2.0 ** -34), 2.0 ** -33, -(2.0 ** -33), 2.0 ** -30, -(2.0 ** -30)]
    for t in range(count):
        row = rng.standard_normal(D).astype(np.float32)
        S = sum(Fraction(float(x)) ** 2 for x in row)
        q = S / D
        c = np.float32(float(q))
        cb = int(c.view(np.uint32))
        mid = (Fraction(float(c)) + Fraction(float(np.uint32(cb + 1).view(np.float32)))) / 2
        mid *= 1 + Fraction(offsets[t % len(offsets)])
        # coarse: the largest element; fine: a small one (finer binary32 steps)
        for i in (int(np.argmax(np.abs(row))), int(np.argmin(np.abs(row) + (np.abs(row) < 1e-3)))):
            S = sum(Fraction(float(x)) ** 2 for x in row)
            want = Fraction(float(row[i])) ** 2 + (mid * D - S)
            row[i] = np.float32(np.sqrt(float(max(want, Fraction(0)))))
        yield row


def test_mean_square_fast_path_never_decides_wrongly():
    rng = np.random.default_rng(5)
    decided = undecided = 0
    cases = list(near_midpoint_rows(rng, 60)) + [r for r in rows() if np.any(r)]
    for row in cases:
        ok, v = meansq_fast(row, rng)
        if ok:
            decided += 1
            assert v == meansq_exact(row)
        else:
            undecided += 1
    assert decided >= 20 and undecided >= 15
