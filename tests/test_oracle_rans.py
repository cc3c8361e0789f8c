"""Pins of the oracle's interleaved rANS chunk coder.

The pages name the coder (ANS: EntQuant summary "Float8@2bits ...",
technical part §2 "Codificación de Pesos"; rANS in the discussion under the
DFloat11 write-up) but print none of it, so the coder is pinned by what the
mathematics fixes:
  * brute force over every short sequence on tiny alphabets with extreme
    tables: decode(encode(x)) = x, the encoding is injective, at most one
    word per symbol per lane, every lane ends back at L;
  * closed forms: a one-symbol table (f = M) codes nothing; with the uniform
    table f = 16 each symbol is exactly one byte of the state, so states and
    words can be written down by hand (this fixes lane assignment, word
    order and the reversal of the emission list);
  * an independent pure-Python statement of the same definition
    (oracle/pyrans.py) gives byte-identical states and words;
  * K = 1 is textbook single-state rANS (Duda 2013): its size is within the
    known bound of the information content.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
from oracle import pyrans

M = oracle.M
L = oracle.L


def table(fs):
    f = np.zeros(256, np.uint16)
    for s, v in fs.items():
        f[s] = v
    assert f.sum() == M
    return f


EXTREME_TABLES = [
    {0: M},                                   # one symbol
    {0: 1, 1: M - 1},                         # rarest vs almost certain
    {0: M - 1, 1: 1},
    {0: 2048, 1: 2048},                       # one bit each
    {0: 1, 1: 1, 2: M - 2},
    {0: 1, 1: 2, 2: 3, 3: M - 6},
    {3: 1, 7: 4094, 200: 1},                  # sparse byte values
    {0: 1365, 1: 1365, 2: 1366},
]


def _seqs(alphabet, max_len):
    for n in range(0, max_len + 1):
        yield from itertools.product(alphabet, repeat=n)


@pytest.mark.parametrize("fs", EXTREME_TABLES)
@pytest.mark.parametrize("K", [1, 2, 3, 64])
def test_bruteforce_round_trip_and_injective(fs, K):
    f = table(fs)
    alphabet = sorted(fs)
    max_len = {1: 12, 2: 10, 3: 7, 4: 6}[len(alphabet)] if len(alphabet) <= 4 else 5
    if K == 64:
        max_len = min(max_len, 8)
    seen = {}
    for seq in _seqs(alphabet, max_len):
        sym = np.array(seq, np.uint8)
        states, words = oracle.encode_chunk(sym, K, f)
        # at most one word per symbol per lane
        assert words.size <= sym.size
        assert np.all(states >= L) and np.all(states.astype(np.uint64) < (1 << 32))
        out, st = oracle.decode_chunk(states, words, sym.size, K, f)
        assert st == oracle.STATUS_OK
        assert out.tolist() == list(seq)
        key = (sym.size, states.tobytes(), words.tobytes())
        assert key not in seen, f"encodings of {seen.get(key)} and {seq} collide"
        seen[key] = seq


def test_words_per_lane_at_most_one_per_symbol():
    rng = np.random.default_rng(0)
    f = table({0: 1, 1: 1, 2: M - 2})
    # the rarest symbols cost 12 bits each: a lane full of them emits on
    # roughly every other symbol but never twice for one symbol
    sym = np.zeros(64 * 50, np.uint8)
    sym[rng.random(sym.size) < 0.5] = 1
    states, words = oracle.encode_chunk(sym, 64, f)
    assert words.size <= sym.size
    out, st = oracle.decode_chunk(states, words, sym.size, 64, f)
    assert st == 0 and np.array_equal(out, sym)


def test_one_symbol_table_codes_nothing():
    f = table({42: M})
    for n in (0, 1, 63, 64, 65, 4096, 5000):
        sym = np.full(n, 42, np.uint8)
        states, words = oracle.encode_chunk(sym, 64, f)
        assert words.size == 0
        assert np.all(states == L)
        out, st = oracle.decode_chunk(states, words, n, 64, f)
        assert st == 0 and np.all(out == 42)


UNIFORM = np.full(256, 16, np.uint16)


def test_uniform_table_two_symbols_per_lane_closed_form():
    # f = 16 for every byte: coding a byte multiplies the state by exactly
    # 2^8 and stores the byte in bits 4..11. From x = L, a lane's last symbol
    # b gives 2^24 + 16 b; its first symbol a then forces one word (the low
    # 16 bits, 16 b) out and leaves 2^16 + 16 a.
    rng = np.random.default_rng(1)
    sym = rng.integers(0, 256, size=128).astype(np.uint8)
    states, words = oracle.encode_chunk(sym, 64, UNIFORM)
    np.testing.assert_array_equal(states, (1 << 16) + 16 * sym[:64].astype(np.uint32))
    # lane k's word is 16 * (its second symbol), in ascending lane order
    np.testing.assert_array_equal(words, (16 * sym[64:].astype(np.uint32)).astype(np.uint16))


def test_uniform_table_three_symbols_per_lane_closed_form():
    rng = np.random.default_rng(2)
    sym = rng.integers(0, 256, size=192).astype(np.uint32)
    states, words = oracle.encode_chunk(sym.astype(np.uint8), 64, UNIFORM)
    a, b, c = sym[:64], sym[64:128], sym[128:]
    np.testing.assert_array_equal(states, (1 << 24) + (b << 12) + (a << 4))
    np.testing.assert_array_equal(words, (16 * c).astype(np.uint16))


def test_uniform_table_word_count_is_half_the_symbols_per_lane():
    rng = np.random.default_rng(3)
    for n in (1, 63, 64, 65, 200, 1000, 4096, 4095):
        sym = rng.integers(0, 256, size=n).astype(np.uint8)
        states, words = oracle.encode_chunk(sym, 64, UNIFORM)
        per_lane = [len(range(j, n, 64)) for j in range(64)]
        assert words.size == sum(m // 2 for m in per_lane)
        out, st = oracle.decode_chunk(states, words, n, 64, UNIFORM)
        assert st == 0 and np.array_equal(out, sym)


def _random_table(rng, k):
    syms = rng.choice(256, size=k, replace=False)
    if k == 1:
        return table({int(syms[0]): M})
    cuts = np.sort(rng.choice(np.arange(1, M), size=k - 1, replace=False))
    parts = np.diff(np.concatenate([[0], cuts, [M]]))
    return table({int(s): int(p) for s, p in zip(syms, parts)})


@pytest.mark.parametrize("K", [1, 2, 3, 7, 64])
def test_c_and_python_statements_agree_byte_for_byte(K):
    rng = np.random.default_rng(10 + K)
    for trial in range(40):
        k = int(rng.integers(1, 40))
        f = _random_table(rng, k)
        present = np.nonzero(f)[0]
        p = f[present].astype(np.float64) / M
        n = int(rng.integers(0, 700))
        sym = rng.choice(present, size=n, p=p).astype(np.uint8)
        st_c, w_c = oracle.encode_chunk(sym, K, f)
        st_p, w_p = pyrans.encode(sym.tolist(), K, f.tolist())
        assert st_c.tolist() == st_p
        assert w_c.tolist() == w_p
        out_p, ok = pyrans.decode(st_p, w_p, n, K, f.tolist())
        assert ok and out_p == sym.tolist()


def test_single_state_size_is_within_the_rans_bound():
    # K = 1: the coded size in bits (16 per word + 32 for the final state)
    # is at least the information content sum(log2(M / f_s)) and exceeds it
    # by at most the state's 32 bits plus a small per-symbol loss from
    # truncating the state to 16-bit words (below 1e-3 bit/symbol here).
    rng = np.random.default_rng(4)
    for _ in range(20):
        f = _random_table(rng, int(rng.integers(2, 60)))
        present = np.nonzero(f)[0]
        sym = rng.choice(present, size=20000, p=f[present] / M).astype(np.uint8)
        states, words = oracle.encode_chunk(sym, 1, f)
        info = float(np.sum(np.log2(M / f[sym].astype(np.float64))))
        bits = 16 * words.size + 32
        assert bits >= info - 16  # the final state's unused bits are at most 16
        assert bits <= info + 32 + 1e-3 * sym.size + 16


def test_corruption_is_detected():
    rng = np.random.default_rng(7)
    f = _random_table(rng, 20)
    present = np.nonzero(f)[0]
    sym = rng.choice(present, size=4096, p=f[present] / M).astype(np.uint8)
    states, words = oracle.encode_chunk(sym, 64, f)
    assert words.size > 10
    # dropping the last word: the stream runs out
    _, st = oracle.decode_chunk(states, words[:-1], sym.size, 64, f)
    assert st == oracle.STATUS_BAD_WORDS
    # an extra word: not used up
    _, st = oracle.decode_chunk(states, np.append(words, 7).astype(np.uint16), sym.size, 64, f)
    assert st == oracle.STATUS_BAD_WORDS
    # a wrong initial state with the right word count: detected or decoded
    # differently (here: detected)
    bad = states.copy()
    bad[5] ^= 1
    out, st = oracle.decode_chunk(bad, words, sym.size, 64, f)
    assert st != oracle.STATUS_OK or not np.array_equal(out, sym)
    flagged = 0
    for i in range(50):
        w = words.copy()
        w[int(rng.integers(0, w.size))] ^= np.uint16(1 << int(rng.integers(0, 16)))
        out, st = oracle.decode_chunk(states, w, sym.size, 64, f)
        assert st != oracle.STATUS_OK or not np.array_equal(out, sym) or np.array_equal(w, words)
        flagged += st != oracle.STATUS_OK
    assert flagged >= 40  # a single bit flip almost always breaks the end-state check


def test_invalid_tables_rejected():
    f = np.zeros(256, np.uint16)
    f[0] = 4095
    with pytest.raises(ValueError):
        oracle.encode_chunk(np.zeros(10, np.uint8), 64, f)
    f = table({0: M})
    with pytest.raises(ValueError):
        oracle.encode_chunk(np.ones(10, np.uint8), 64, f)  # symbol with f = 0
