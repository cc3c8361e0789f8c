"""Pins of the oracle's frequency quantiser by its invariants.

The pages fix no quantisation rule (they only say the weights are entropy
coded, EntQuant summary "Float8@2bits ...", technical part §2); the table is
a decoder input, so any table that sums to M and gives every present symbol
a nonzero frequency decodes exactly. What is pinned here is that contract,
closeness to the counts, and the table rule's own choices -- halves round
up, the excess comes off the largest frequency (smallest byte on a tie),
the shortfall goes to the largest count (smallest byte on a tie) -- by
worked cases derived by hand, each of which a plausible slip in one of
those choices fails."""
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


def _table(pairs):
    f = np.zeros(256, np.uint16)
    for sym, v in pairs.items():
        f[sym] = v
    return f


def test_worked_case_halves_round_up():
    # counts 5 and 8187 (N = 8192): exact shares 4096 * c / N = 2.5 and 4093.5.
    # Halves up: 3 + 4094 = 4097, one over M, taken from the largest (byte 8):
    # {7: 3, 8: 4093}. (Halves to even would give 2 + 4094 = 4096 unchanged.)
    counts = np.zeros(256, np.uint64)
    counts[7], counts[8] = 5, 8187
    np.testing.assert_array_equal(oracle.quantize_freqs(counts), _table({7: 3, 8: 4093}))


def test_worked_case_excess_alternates_between_tied_largest():
    # bytes 0 and 1 count 500,000 each, bytes 2..254 count 1 each (253 bytes);
    # N = 1,000,253. Shares: 2047.48 -> 2047 for the two large bytes,
    # 0.0041 -> 0 -> floored to 1 for each rare byte. Sum 2 * 2047 + 253 =
    # 4347, so 251 units come off. Each unit goes to the largest frequency,
    # the smaller byte on a tie: byte 0, byte 1, byte 0, ... -- byte 0 loses
    # 126, byte 1 loses 125: {0: 1921, 1: 1922}, the rare bytes stay at 1.
    counts = np.zeros(256, np.uint64)
    counts[0] = counts[1] = 500_000
    counts[2:255] = 1
    want = _table({0: 1921, 1: 1922})
    want[2:255] = 1
    np.testing.assert_array_equal(oracle.quantize_freqs(counts), want)


def test_worked_case_shortfall_goes_to_largest_count():
    # byte 1 count 216, byte 2 count 217, bytes 3..21 count 206 each; N = 4347.
    # Shares: 203.53 -> 204, 204.47 -> 204, 194.11 -> 194. Sum 204 + 204 +
    # 19 * 194 = 4094: two units short. They go to the largest count, byte 2
    # (217), not to byte 1, which ties it on frequency and is the smaller byte:
    # {1: 204, 2: 206, 3..21: 194}.
    counts = np.zeros(256, np.uint64)
    counts[1], counts[2] = 216, 217
    counts[3:22] = 206
    want = _table({1: 204, 2: 206})
    want[3:22] = 194
    np.testing.assert_array_equal(oracle.quantize_freqs(counts), want)


def test_worked_case_shortfall_tie_on_count_goes_to_smaller_byte():
    # counts {1: 1, 2: 2, 3: 3, 4: 3}, N = 9. Shares 455.1, 910.2, 1365.3,
    # 1365.3 -> 455 + 910 + 1365 + 1365 = 4095: one unit short, given to the
    # largest count; bytes 3 and 4 tie on it and byte 3 is the smaller.
    counts = np.zeros(256, np.uint64)
    counts[1:5] = [1, 2, 3, 3]
    np.testing.assert_array_equal(oracle.quantize_freqs(counts),
                                  _table({1: 455, 2: 910, 3: 1366, 4: 1365}))


def test_worked_case_three_equal_counts():
    # three equal counts: 4096 / 3 = 1365.33 -> 1365 each, 4095 in all; the
    # unit goes to the smallest of the three tied bytes.
    counts = np.zeros(256, np.uint64)
    counts[[5, 9, 200]] = 1
    np.testing.assert_array_equal(oracle.quantize_freqs(counts),
                                  _table({5: 1366, 9: 1365, 200: 1365}))
