"""The device encoder's coding step for a renormalised state x (x < 2^20 f,
1 <= f <= 4096; any 32-bit x for f = 4096) is x' = floor(x / f) 2^12 +
(x mod f) + c. It finds q = floor(x / f) with fp32 and 24-bit integer
operations only:

    z     = RN32(RN32(x) * rcp - 1/4)     one fused multiply-add
    rcp   = RN32(RN64(1 / f))
    q_est = trunc(z)                      claimed: q - 1 or q (0 when q = 0)
    r     = x - q_est f  (mod 2^32)       in [0, 2f) by the claim
    x'    = q_est (4096 - f) + x + c + (r >= f ? 4096 - f : 0)

These tests check that claim and the whole step on the CPU, in exact integer
arithmetic: every fp32 value involved is a dyadic rational, so the fused
multiply-add is an exact integer rounded once to 24 significant bits (ties to
even). The rounding helper is itself checked against numpy's float32 cast and
against a nearest-neighbour search in exact rationals."""
from fractions import Fraction

import numpy as np

PROB_BITS = 12
PROB_SCALE = 1 << PROB_BITS
MASK32 = (1 << 32) - 1


def bit_length(a):
    """Bit length of each positive int64 in a (exact, though computed through
    float64: a value rounded up to a power of two is caught and fixed)."""
    e = np.frexp(a.astype(np.float64))[1].astype(np.int64)
    return e - (a < (np.int64(1) << (e - 1)))


def rn24(n):
    """Round each int64 in n to the nearest value with 24 significant bits,
    ties to even. Returns (sign, keep, shift) with value = sign keep 2^shift
    and 0 <= keep <= 2^24."""
    n = np.asarray(n, dtype=np.int64)
    sign = np.where(n < 0, -1, 1).astype(np.int64)
    a = np.abs(n)
    shift = np.zeros_like(a)
    nz = a > 0
    shift[nz] = np.maximum(bit_length(a[nz]) - 24, 0)
    keep = a >> shift
    rem = a - (keep << shift)
    half = np.where(shift > 0, np.int64(1) << np.maximum(shift - 1, 0), 0)
    up = (shift > 0) & ((rem > half) | ((rem == half) & ((keep & 1) == 1)))
    return sign, keep + up, shift


def fp32_int(x):
    """RN32 of non-negative integers below 2^32, as integers."""
    _, keep, shift = rn24(x)
    return keep << shift


def rcp_parts(f):
    """rcp = RN32(RN64(1/f)) = m 2^-k with integer m, for each f."""
    rcp = np.float32(np.float64(1.0) / np.asarray(f, dtype=np.float64))
    mant, e = np.frexp(rcp.astype(np.float64))
    m = (mant * (1 << 24)).astype(np.int64)
    assert np.all(m.astype(np.float64) == mant * (1 << 24))
    return m, (24 - e).astype(np.int64)


def q_estimate(x, f):
    """trunc(RN32(RN32(x) rcp - 1/4)) in exact integer arithmetic."""
    x = np.asarray(x, dtype=np.int64)
    m, k = rcp_parts(f)
    # RN32(x) m 2^-k - 2^-2 = n 2^-k; |n| < 2^57
    n = fp32_int(x) * m - (np.int64(1) << (k - 2))
    sign, keep, shift = rn24(n)
    # z = sign keep 2^(shift - k); shift - k < 0 here as |z| < 2^21 needs
    # no more than 24 bits above 2^-3
    assert np.all(shift < k)
    mag = (keep << shift) >> k          # floor(|z|)
    return np.where(sign < 0, -mag, mag)


def mul24(a, b):
    """Low 32 bits of the product of the sign-extended low 24 bits of a, b."""
    def sx(v):
        v = np.asarray(v, dtype=np.int64) & 0xFFFFFF
        return np.where(v >= 1 << 23, v - (1 << 24), v)
    return (sx(a) * sx(b)) & MASK32


def code_step(x, f, c):
    """The device encoder's step, emulated with its operand widths."""
    x = np.asarray(x, dtype=np.int64)
    f = np.asarray(f, dtype=np.int64)
    g = PROB_SCALE - f
    q = q_estimate(x, f)
    assert np.all(q >= 0)               # trunc(z) of z > -1
    r = (x + mul24(q, -f)) & MASK32
    fix = np.where(r >= f, g, 0)
    return (mul24(q, g) + x + c + fix) & MASK32, q


def check(x, f, c=None):
    x = np.asarray(x, dtype=np.int64)
    f = np.broadcast_to(np.asarray(f, dtype=np.int64), x.shape)
    if c is None:
        c = PROB_SCALE - f              # the largest cumulative start
    top = np.where(f < PROB_SCALE, (f << 20) - 1, MASK32)
    assert np.all((x >= 0) & (x <= top))
    got, q_est = code_step(x, f, c)
    q = x // f
    assert np.all((q_est == q) | (q_est == q - 1)), "estimate off by more than one"
    assert np.all(q_est[q == 0] == 0)
    want = np.where(f < PROB_SCALE, (q << PROB_BITS) + x % f + c, x)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (int(x[bad[0]]), int(f[bad[0]]))


def test_rounding_helper_matches_numpy_on_integers():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.integers(0, 1 << 32, 200_000, dtype=np.int64),
                        np.arange(0, 1 << 16, dtype=np.int64),
                        (np.int64(1) << np.arange(24, 33)) - 1,
                        (np.int64(1) << np.arange(24, 32)) + 1])
    want = np.float32(x.astype(np.float64)).astype(np.float64)
    assert np.array_equal(fp32_int(x).astype(np.float64), want)


def nearest_fp32(v: Fraction) -> Fraction:
    """RN32 of an exact rational: the nearest of the fp32 neighbours of a
    first guess, ties to the even significand."""
    guess = np.float32(float(v))
    cands = {np.nextafter(guess, np.float32(-np.inf)), guess,
             np.nextafter(guess, np.float32(np.inf))}
    best = sorted(cands, key=lambda c: (abs(Fraction(float(c)) - v),
                                        int(np.frexp(c)[0] * (1 << 24)) & 1))
    return Fraction(float(best[0]))


def test_fma_rounding_matches_exact_rationals():
    rng = np.random.default_rng(5)
    f = rng.integers(1, PROB_SCALE + 1, 3000, dtype=np.int64)
    x = (rng.random(3000) * (f << 20).astype(np.float64)).astype(np.int64)
    x[:64] = f[:64] * rng.integers(0, 1 << 20, 64)     # exact multiples
    x[64:128] = 0
    m, k = rcp_parts(f)
    n = fp32_int(x) * m - (np.int64(1) << (k - 2))
    sign, keep, shift = rn24(n)
    for i in range(x.size):
        rcp = Fraction(float(np.float32(1.0 / float(f[i]))))
        exact = Fraction(float(np.float32(float(x[i])))) * rcp - Fraction(1, 4)
        got = Fraction(int(sign[i]) * int(keep[i]) << int(shift[i]), 1 << int(k[i]))
        assert got == nearest_fp32(exact), (int(x[i]), int(f[i]))


def test_step_exhaustive_small_frequencies():
    for f in (1, 2, 3, 5):
        check(np.arange(0, f << 20, dtype=np.int64), f)


def test_step_at_bucket_edges_for_every_frequency():
    """Every f, the buckets where the estimate's error is largest (q near
    2^20) and smallest, each at r = 0, 1, f - 2, f - 1."""
    rng = np.random.default_rng(11)
    qs = np.concatenate([np.arange(0, 64), np.arange((1 << 20) - 1024, 1 << 20),
                         rng.integers(64, (1 << 20) - 1024, 128)]).astype(np.int64)
    for f0 in range(1, PROB_SCALE, 256):
        f = np.arange(f0, min(f0 + 256, PROB_SCALE), dtype=np.int64)
        ff, qq, oo = np.meshgrid(f, qs, np.arange(4), indexing="ij")
        off = np.choose(oo, [np.zeros_like(ff), np.ones_like(ff), ff - 2, ff - 1])
        x = (qq * ff + off).ravel()
        ok = (off.ravel() >= 0) & (off.ravel() < ff.ravel())
        check(x[ok], ff.ravel()[ok])


def test_step_random_states():
    rng = np.random.default_rng(13)
    f = rng.integers(1, PROB_SCALE, 2_000_000, dtype=np.int64)
    x = (rng.random(f.size) * (f << 20).astype(np.float64)).astype(np.int64)
    x = np.minimum(x, (f << 20) - 1)
    check(x, f, c=rng.integers(0, PROB_SCALE - f + 1))


def test_single_symbol_table_keeps_the_state():
    rng = np.random.default_rng(17)
    x = np.concatenate([rng.integers(0, 1 << 32, 100_000, dtype=np.int64),
                        np.array([0, 1, 4095, 4096, MASK32 - 1, MASK32], dtype=np.int64)])
    check(x, PROB_SCALE, c=0)
