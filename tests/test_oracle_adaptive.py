"""Pins of the oracle's per-chunk-table (adaptive) container. The reading:
each chunk is coded with the C2 table of its own counts, stored at the head
of its region (u16 freq[256], then the 64 states and the words)."""
import numpy as np

import oracle
import synth


def test_layout_of_a_single_symbol_chunk():
    # 64 copies of byte 5: the chunk's table is f[5] = 4096, the coder emits
    # no words and every state stays 2^16 (closed form, C5 with f = 4096)
    sp = dict(kind=0, rows=1, cols=64, chunk_symbols=64, symbols=np.full(64, 5, np.uint8))
    c = oracle.encode_container_adaptive([sp])
    want = np.zeros(768, np.uint8)
    want[10:12] = [0x00, 0x10]                   # freq[5] = 4096, little-endian
    for j in range(64):
        want[512 + 4 * j:516 + 4 * j] = [0x00, 0x00, 0x01, 0x00]  # 2^16
    assert c.blob.size == 768 and np.array_equal(c.blob, want)
    assert c.chunks.tolist() == [[0, 64, 0, 0, 0]]


def test_one_chunk_tensor_matches_the_shared_table_container():
    # one chunk: its own table is the tensor's table, so after the 512-byte
    # table the region equals the shared-table container's region
    for seed, (r, cl) in enumerate([(8, 512), (3, 64), (16, 4096)]):
        sp = synth.random_int8_tensor(r, cl, 1.2 + seed, 60 + seed, r * cl)
        a = oracle.encode_container_adaptive([sp])
        s = oracle.encode_container([sp])
        assert a.n_chunks == s.n_chunks == 1
        assert np.array_equal(a.blob[512:], s.blob)
        assert np.array_equal(a.blob[:512].view("<u2"), s.tensors[0]["freq"])


def test_tables_follow_rule_c2_per_chunk():
    sp = synth.banded_int8_tensor(64, 1024, 8, 1, 4096)
    c = oracle.encode_container_adaptive([sp])
    sym = sp["symbols"]
    for t, n, nw, off, e0 in c.chunks.astype(np.int64):
        freq = c.blob[off:off + 512].view("<u2")
        counts = np.bincount(sym[e0:e0 + n], minlength=256)
        assert int(freq.sum()) == 4096
        assert ((freq > 0) == (counts > 0)).all()
        assert np.array_equal(freq, oracle.quantize_freqs(counts.astype(np.uint64)))


def test_round_trip_ragged_and_degenerate():
    specs = [synth.random_int8_tensor(r, cl, 0.7 + 0.5 * i, 80 + i, C)
             for i, (r, cl, C) in enumerate([(3, 7, 64), (17, 129, 4096), (5, 4097, 4096),
                                             (33, 1000, 65536), (1, 65, 64)])]
    one = synth.random_int8_tensor(16, 64, 1.0, 90, 64)
    one["symbols"] = np.full(one["symbols"].shape, 200, np.uint8)
    allb = synth.random_int8_tensor(64, 512, 1.0, 91, 4096)
    allb["symbols"] = synth.random_bytes(64 * 512, 91).view(np.uint8)
    specs += [one, allb, synth.banded_int8_tensor(40, 2816, 3, 2, 2816 * 2)]
    c = oracle.encode_container_adaptive(specs)
    outs, st = oracle.decode_container_adaptive_symbols(c)
    assert (st == oracle.STATUS_OK).all()
    for sp, o in zip(specs, outs):
        assert np.array_equal(o, np.ascontiguousarray(sp["symbols"]).view(np.uint8).ravel())


def test_bad_table_is_reported():
    sp = synth.random_int8_tensor(16, 512, 1.5, 92, 4096)
    c = oracle.encode_container_adaptive([sp])
    off = int(c.chunks[1, 3])
    blob = c.blob.copy()
    blob[off] ^= 1                                 # table of chunk 1 no longer sums to 4096
    bad = oracle.Container(blob, c.tensors, c.chunks)
    _, st = oracle.decode_container_adaptive_symbols(bad)
    assert st.tolist() == [0, oracle.STATUS_BAD_TABLE]


def test_adaptive_tables_pay_on_banded_codes():
    # bands of different spread: the per-chunk words shrink; on identically
    # distributed codes they cannot beat the shared table by more than the
    # table quantisation (and the 512-byte tables are pure overhead)
    banded = synth.banded_int8_tensor(256, 4096, 16, 3, 65536)
    a = oracle.encode_container_adaptive([banded])
    s = oracle.encode_container([banded])
    words_a, words_s = int(a.chunks[:, 2].sum()), int(s.chunks[:, 2].sum())
    assert words_a < 0.98 * words_s and a.blob.size < s.blob.size
    iid = synth.random_int8_tensor(256, 4096, 2.0, 93, 65536)
    a = oracle.encode_container_adaptive([iid])
    s = oracle.encode_container([iid])
    words_a, words_s = int(a.chunks[:, 2].sum()), int(s.chunks[:, 2].sum())
    assert abs(words_a - words_s) <= 0.005 * words_s
    assert a.blob.size > s.blob.size


def test_exponent_streams_round_trip_with_per_chunk_tables():
    """BF16 weights split into exponent and sign+mantissa bytes, the exponent
    stream coded with per-chunk tables: the merge of the decoded exponents
    gives back every original bit pattern, ragged tails included."""
    a = synth.bf16_weights(64, 1024, sigma=0.02)[0]["bf16"]
    b = synth.bf16_weights(64, 1024, sigma=2.0)[0]["bf16"]
    w = np.concatenate([a, b, a[:70_001]])           # two regimes, then a ragged tail
    e, sm = oracle.bf16_split(w)
    spec = dict(kind=oracle.KIND_BF16EXP, rows=1, cols=w.size, symbols=e, chunk_symbols=16384)
    c = oracle.encode_container_adaptive([spec])
    got, st = oracle.decode_container_adaptive_split(c, sm)
    assert (st == oracle.STATUS_OK).all()
    np.testing.assert_array_equal(got, w)
    # the chunks of the two regimes carry different tables
    tabs = {bytes(c.blob[int(off):int(off) + 512]) for off in c.chunks[:, 3]}
    assert len(tabs) >= 2
