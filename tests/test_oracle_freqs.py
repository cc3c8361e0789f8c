"""Pins of the oracle's frequency quantiser by its invariants.

The pages fix no quantisation rule (they only say the weights are entropy
coded, EntQuant summary "Float8@2bits ...", technical part §2); the table is
a decoder input, so any table that sums to M and gives every present symbol
a nonzero frequency decodes exactly. What is pinned here is that contract
plus closeness to the counts. The exact tie-breaking rule is "parity
unpinned" (it moves only the compressed size, never a decoded value)."""
import numpy as np

import oracle


def _check_contract(counts, f):
    assert f.dtype == np.uint16
    present = counts > 0
    if not present.any():
        assert not f.any()
        return
    assert int(f.sum()) == oracle.M
    assert np.all(f[present] >= 1)
    assert np.all(f[~present] == 0)


def test_random_count_vectors():
    rng = np.random.default_rng(0)
    for trial in range(300):
        k = int(rng.integers(1, 257))
        counts = np.zeros(256, np.uint64)
        idx = rng.choice(256, size=k, replace=False)
        scale = 10 ** rng.uniform(0, 9)
        counts[idx] = np.maximum(1, rng.exponential(scale, size=k)).astype(np.uint64)
        f = oracle.quantize_freqs(counts)
        _check_contract(counts, f)
        # every frequency is within the rounding slack of its exact share,
        # except where the floor of 1 or the final correction moved it
        exact = counts.astype(np.float64) * oracle.M / counts.sum()
        err = np.abs(f.astype(np.float64) - exact)
        assert np.all(err[counts > 0] <= 1.0 + 256)


def test_single_symbol_gets_everything():
    for s in (0, 17, 255):
        counts = np.zeros(256, np.uint64)
        counts[s] = 12345
        f = oracle.quantize_freqs(counts)
        assert f[s] == oracle.M and f.sum() == oracle.M


def test_empty_is_all_zero():
    f = oracle.quantize_freqs(np.zeros(256, np.uint64))
    assert not f.any()


def test_all_256_symbols_equal_counts_are_uniform():
    f = oracle.quantize_freqs(np.full(256, 1000, np.uint64))
    assert np.all(f == 16)


def test_rare_symbols_are_floored_to_one_and_sum_is_restored():
    counts = np.zeros(256, np.uint64)
    counts[0] = 10**9
    counts[1:200] = 1
    f = oracle.quantize_freqs(counts)
    _check_contract(counts, f)
    assert np.all(f[1:200] == 1)
    assert f[0] == oracle.M - 199


def test_deterministic():
    rng = np.random.default_rng(5)
    counts = rng.integers(0, 10**6, size=256).astype(np.uint64)
    a = oracle.quantize_freqs(counts)
    b = oracle.quantize_freqs(counts.copy())
    np.testing.assert_array_equal(a, b)


def test_proportional_counts_are_exact():
    # counts that are an exact multiple of a valid table map back to it
    rng = np.random.default_rng(6)
    for _ in range(50):
        f0 = np.zeros(256, np.uint64)
        cuts = np.sort(rng.choice(np.arange(1, oracle.M), size=30, replace=False))
        parts = np.diff(np.concatenate([[0], cuts, [oracle.M]]))
        f0[rng.choice(256, size=parts.size, replace=False)] = parts
        f = oracle.quantize_freqs(f0 * np.uint64(777))
        np.testing.assert_array_equal(f, f0.astype(np.uint16))
