"""The device table builder applies the table rule's trimming step in one
pass instead of one unit at a time: taking one from the largest frequency
(smallest byte on ties) K times leaves every frequency at most L, where L is
the smallest level with D(L) = sum over s of max(0, q_s - L) <= K, and the
remaining K - D(L) units come off the smallest-index bytes whose frequency
reached L. This checks that reading against the oracle's rule on the CPU."""
import numpy as np

import oracle

M = 4096


def levels_rule(counts: np.ndarray) -> np.ndarray:
    c = counts.astype(np.int64)
    n = int(c.sum())
    present = c > 0
    f = np.zeros(256, np.int64)
    if present.sum() == 0:
        return f.astype(np.uint16)
    if present.sum() == 1:
        f[present] = M
        return f.astype(np.uint16)
    q = (2 * c * M + n) // (2 * n)
    q = np.where(present, np.maximum(q, 1), 0)
    total = int(q.sum())
    if total > M:
        k = total - M
        lo, hi = 1, M                       # smallest L with D(L) <= k
        while lo < hi:
            mid = (lo + hi) // 2
            if int(np.maximum(q - mid, 0).sum()) <= k:
                hi = mid
            else:
                lo = mid + 1
        L = lo
        r = k - int(np.maximum(q - L, 0).sum())
        at = q >= L
        q = np.minimum(q, L)
        rank = np.cumsum(at) - 1            # index among the bytes at level L
        q = np.where(at & (rank < r), q - 1, q)
    elif total < M:
        q[int(np.argmax(c))] += M - total   # first maximum: smallest byte
    return q.astype(np.uint16)


def test_levels_equal_the_oracle_rule():
    rng = np.random.default_rng(12)
    cases = [np.full(256, 7), np.eye(256, dtype=np.int64)[3] * 99, np.arange(256)]
    for i in range(3000):
        c = rng.integers(0, [2, 50, 5000, 1 << 20][i % 4], 256)
        c[rng.random(256) < rng.random()] = 0
        if i % 3 == 0:                      # one dominant byte and many rare ones
            c[int(rng.integers(0, 256))] += int(rng.integers(1, 1 << 30))
        cases.append(c)
    trims = 0
    for c in cases:
        c = np.asarray(c, np.uint64)
        want = oracle.quantize_freqs(c) if c.sum() else np.zeros(256, np.uint16)
        got = levels_rule(c)
        np.testing.assert_array_equal(got, want)
        q = np.where(c > 0, np.maximum((2 * c.astype(np.int64) * M + int(c.sum())) //
                                       (2 * max(int(c.sum()), 1)), 1), 0)
        trims += int(q.sum() > M)
    assert trims > 300                      # the trimming step is exercised
