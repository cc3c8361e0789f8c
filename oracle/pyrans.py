"""A second, independent statement of the interleaved rANS coder, in pure
Python, for small inputs only.

TEST INFRASTRUCTURE (part of the oracle). It exists so that oracle.c can be
cross-checked against code written separately from the same definition:
range ANS (Duda, "Asymmetric numeral systems", 2013) with K interleaved
states (Giesen, "Interleaved entropy coders", 2014), probability scale
M = 2^12, states in [2^16, 2^32), 16-bit renormalisation words, symbol i on
lane i mod K. The pages this library follows name ANS for the weight
bitstream (EntQuant, "Float8@2bits ...", technical summary §2 "Codificación
de Pesos") but give no coder, so the parameters are the library's format.

Written in terms of the state's arithmetic meaning rather than as a copy of
oracle.c: a symbol s with frequency f and cumulative c maps state x to
    C(s, x) = M * (x // f) + c + (x % f)
and back with
    D(x) = (s, f * (x // M) + (x % M) - c)  where c <= x % M < c + f.
"""
from __future__ import annotations

import bisect

M = 4096
L = 1 << 16
B = 1 << 16  # word base


def _cum(freq):
    c = [0]
    for f in freq:
        c.append(c[-1] + int(f))
    return c


def encode(symbols, K, freq):
    """Returns (states list[K], words list) -- the decoder reads words front
    to back."""
    cum = _cum(freq)
    assert cum[-1] == M, "frequencies must sum to M"
    x = [L] * K
    out_rev = []
    for i in range(len(symbols) - 1, -1, -1):
        j = i % K
        s = symbols[i]
        f = int(freq[s])
        assert f > 0
        # the largest state that still codes s without leaving [L, 2^32) is
        # below (L // M) * B * f; states at or above it first shed 16 bits
        if x[j] >= (L // M) * B * f:
            out_rev.append(x[j] % B)
            x[j] //= B
        x[j] = M * (x[j] // f) + cum[s] + (x[j] % f)
        assert L <= x[j] < (1 << 32)
    return x, out_rev[::-1]


def decode(states, words, n, K, freq):
    """Returns (symbols, ok) where ok means every lane ended at L and every
    word was used exactly once."""
    cum = _cum(freq)
    x = list(states)
    p = 0
    out = []
    ok = True
    for i in range(n):
        j = i % K
        r = x[j] % M
        # the owner of r is the s with cum[s] <= r < cum[s + 1]; such an s
        # always has a nonzero frequency
        s = bisect.bisect_right(cum, r) - 1
        out.append(s)
        x[j] = int(freq[s]) * (x[j] // M) + r - cum[s]
        if x[j] < L:
            if p >= len(words):
                ok = False
                continue
            x[j] = x[j] * B + words[p]
            p += 1
    ok = ok and p == len(words) and all(v == L for v in x)
    return out, ok
