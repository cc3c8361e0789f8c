"""A CPU model of how the per-chunk-table decode builds a chunk's slot ->
symbol map in LDS (the kernel's steps restated lane by lane), checked against
the definition of the map -- slots cum[s] .. cum[s] + f[s] - 1 belong to
symbol s -- on tables with runs of absent symbols, an absent symbol 0,
single-symbol tables, all 256 symbols present, frequency-1 symbols and starts
that fall exactly on a lane's first slot.

The build: each lane l holds the frequencies of symbols 4l .. 4l+3; a scan
over the lanes gives their starts; the map is cleared; every present symbol
writes its byte at its start; each lane finds the symbol of its first slot
64 l by a binary search over the starts and replaces its 64 map bytes by the
running maximum of the marks, starting from that symbol."""
import numpy as np
import pytest

import oracle

M = 4096


def definition(freq):
    f = freq.astype(np.int64)
    return np.repeat(np.arange(256), f).astype(np.uint8)


def first_symbol(cb, j0):
    """The kernel's binary search: the last symbol whose start is at or below j0."""
    s = 0
    for step in (128, 64, 32, 16, 8, 4, 2, 1):
        assert s + step <= 255
        if cb[s + step] <= j0:
            s += step
    return s


def model_build(freq, map_base=0, first=first_symbol):
    f = freq.astype(np.int64)
    assert f.sum() == M
    cum = np.concatenate([[0], np.cumsum(f)[:-1]])
    cb = cum + map_base                      # the entry's high half
    sym_map = np.zeros(M, np.int64)          # cleared by the lanes
    for s in range(256):                     # marks (distinct slots: f >= 1)
        if f[s]:
            sym_map[cum[s]] = s
    out = np.empty(M, np.uint8)
    for lane in range(64):
        m = first(cb, 64 * lane + map_base)
        for j in range(64 * lane, 64 * lane + 64):
            m = max(m, sym_map[j])
            out[j] = m
    return out


def _tables():
    rng = np.random.default_rng(71)
    t = []
    one = np.zeros(256, np.uint16)
    for s in (0, 77, 255):
        u = one.copy()
        u[s] = M
        t.append(u)
    t.append(np.full(256, 16, np.uint16))                  # all present, uniform
    u = np.ones(256, np.uint16)
    u[0] = M - 255                                         # 255 frequency-1 symbols
    t.append(u)
    u = np.ones(256, np.uint16)
    u[255] = M - 255
    t.append(u)
    u = np.zeros(256, np.uint16)
    u[[1, 2, 200]] = [64, 64 * 3, M - 256]                 # symbol 0 absent, starts on lanes
    t.append(u)
    u = np.zeros(256, np.uint16)
    u[[5, 6, 7, 250]] = [1, 63, 64, M - 128]               # a start at slot 1, one at 64
    t.append(u)
    for i in range(300):
        counts = rng.integers(0, [3, 40, 5000][i % 3], 256).astype(np.uint64)
        counts[rng.random(256) < rng.random()] = 0
        if counts.sum() == 0:
            counts[int(rng.integers(0, 256))] = 1
        t.append(oracle.quantize_freqs(counts))
    for sigma in (0.6, 1.0, 3.0):                          # int8 codes of a normal spread
        x = np.clip(np.rint(rng.normal(0, sigma, 65536)), -127, 127).astype(np.int8)
        t.append(oracle.quantize_freqs(oracle.count_symbols(x.view(np.uint8))))
    return t


@pytest.mark.parametrize("map_base", [0, 4096 * 6, 57344])
def test_branch_free_build_equals_the_slot_map(map_base):
    for freq in _tables():
        assert int(freq.astype(np.int64).sum()) == M
        np.testing.assert_array_equal(model_build(freq, map_base), definition(freq))


def test_planted_mistakes_are_caught():
    """The check can fail: a first-slot search that takes the first present
    symbol starting at or after the lane's first slot, or one that ignores
    the map base, differs from the definition on these tables."""
    freq = np.zeros(256, np.uint16)
    freq[[3, 9]] = [100, M - 100]   # symbol 3 runs across lane 1's first slot (64)

    def first_at_or_after(cb, j0):
        return next(s for s in range(256) if cb[s] >= j0 and (s == 255 or cb[s + 1] > cb[s]))

    def base_ignored(cb, j0):
        return first_symbol(cb - cb[0] + 4096, j0)

    assert not np.array_equal(model_build(freq, 0, first_at_or_after), definition(freq))
    assert not np.array_equal(model_build(freq, 8192, base_ignored), definition(freq))
    np.testing.assert_array_equal(model_build(freq, 8192), definition(freq))
