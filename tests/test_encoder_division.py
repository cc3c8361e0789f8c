"""The device encoder computes q = floor(x / f) for a renormalised state
(x < 2^20 f, 1 <= f <= 4096) as the truncation of one fp64 fused
multiply-add, fl64(x * fl64(1/f) + 2^-13). This checks that claim on the
CPU with exact rational arithmetic (a correctly rounded fma is the exact
value rounded once to the nearest double): for every f, at the states where
a truncation error would show first -- just below and at multiples of f,
and the largest renormalised state."""
from fractions import Fraction

import numpy as np

BIAS = Fraction(1, 8192)


def fma_trunc(x: int, rcp: float) -> int:
    return int(float(Fraction(x) * Fraction(rcp) + BIAS))


def test_fp64_quotient_is_exact_at_every_frequency():
    rng = np.random.default_rng(11)
    for f in range(1, 4097):
        rcp = 1.0 / f                     # round-to-nearest double, as on the device
        top = (1 << 20) * f - 1 if f < 4096 else (1 << 32) - 1
        qs = set(int(v) for v in rng.integers(0, top // f + 1, 6))
        qs |= {0, 1, top // f, top // f - 1}
        for q in qs:
            for x in (q * f, q * f + 1, q * f + f - 1, q * f - 1):
                if 0 <= x <= top:
                    assert fma_trunc(x, rcp) == x // f, (f, x)
        assert fma_trunc(top, rcp) == top // f, f
