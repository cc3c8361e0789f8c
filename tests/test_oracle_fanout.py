"""The thread fan-out of the oracle (oracle/fanout.py) adds no arithmetic:
its output equals the single-threaded oracle's container decode and
dequantisation element for element, for shared and per-chunk tables, chunk
sizes that do and do not divide the row length, ragged tails and any
thread count; its comparison mode counts exactly the planted differences."""
import numpy as np
import pytest

import oracle
import synth
from oracle import fanout


def _specs():
    return [synth.random_int8_tensor(24, 1792, 2.0, 41, 4096),    # chunks cross rows
            synth.random_int8_tensor(33, 512, 0.9, 42, 2048),     # 8 rows per chunk, ragged tail
            synth.e4m3_matrix(rows=20, cols=768)[0] | {"chunk_symbols": 1024},
            synth.random_int8_tensor(3, 64, 5.0, 43, 64)]


def _chunks(c, t):
    sel = c.chunks[:, 0] == t
    return c.chunks[sel][:, 1:5]


@pytest.mark.parametrize("threads", [1, 3, 8])
def test_shared_tables_equal_the_single_threaded_oracle(threads):
    specs = _specs()
    c = oracle.encode_container(specs)
    scales = np.concatenate([s["scales"] for s in specs])
    want, st = oracle.decode_container_bf16(c, scales)
    assert (st == 0).all()
    for t, (sp, td) in enumerate(zip(specs, c.tensors)):
        o = td["out_elem_offset"]
        out, res = fanout.tensor_bf16(c.blob, _chunks(c, t), td["freq"], td["kind"], td["rows"],
                                      td["cols"], sp["scales"], n_threads=threads,
                                      codes_compare=sp["symbols"])
        np.testing.assert_array_equal(out, want[o:o + td["n_symbols"]])
        assert res.bad_chunks == 0 and res.code_mismatches == 0


def test_per_chunk_tables_equal_the_single_threaded_oracle():
    specs = _specs()
    c = oracle.encode_container_adaptive(specs)
    scales = np.concatenate([s["scales"] for s in specs])
    want, st = oracle.decode_container_adaptive_bf16(c, scales)
    assert (st == 0).all()
    for t, (sp, td) in enumerate(zip(specs, c.tensors)):
        o = td["out_elem_offset"]
        out, res = fanout.tensor_bf16(c.blob, _chunks(c, t), None, td["kind"], td["rows"],
                                      td["cols"], sp["scales"], n_threads=5, adaptive=True)
        np.testing.assert_array_equal(out, want[o:o + td["n_symbols"]])
        assert res.bad_chunks == 0


def test_compare_mode_counts_planted_differences():
    sp = synth.random_int8_tensor(24, 1792, 2.0, 44, 4096)
    c = oracle.encode_container([sp])
    td = c.tensors[0]
    want, _ = oracle.decode_container_bf16(c, sp["scales"])
    other = want.copy()
    other[[5, 4096 * 3 + 1, want.size - 1]] ^= np.uint16(1)
    _, res = fanout.tensor_bf16(c.blob, _chunks(c, 0), td["freq"], td["kind"], td["rows"],
                                td["cols"], sp["scales"], n_threads=4, compare=want)
    assert res.mismatches == 0 and res.first_mismatch == -1
    _, res = fanout.tensor_bf16(c.blob, _chunks(c, 0), td["freq"], td["kind"], td["rows"],
                                td["cols"], sp["scales"], n_threads=4, compare=other)
    assert res.mismatches == 3 and res.first_mismatch == 5
    # a corrupted word stream is reported as a bad chunk
    blob = c.blob.copy()
    k = 2
    off, nw = int(c.chunks[k, 3]), int(c.chunks[k, 2])
    blob[off + 256 + nw] ^= 0xFF
    _, res = fanout.tensor_bf16(blob, _chunks(c, 0), td["freq"], td["kind"], td["rows"],
                                td["cols"], sp["scales"], n_threads=2, compare=want)
    assert res.bad_chunks >= 1
