"""CPU checks of the library's per-chunk-table (adaptive) host encoder and
plan: containers byte-identical to the oracle's adaptive container, and the
plan's validation of what the adaptive decoder needs (failures happen before
any HIP call, against a dummy workspace address)."""
import ctypes
import os

import numpy as np
import pytest

import oracle
import synth

FAKE_WS = 1 << 20


@pytest.fixture(scope="module")
def E():
    import entropy_coded_weight_amd as E
    if not os.path.exists(E.LIB_PATH):
        from entropy_coded_weight_amd import build
        build.build()
    return E


def _specs():
    specs = [synth.random_int8_tensor(r, c, 0.6 + 0.4 * i, 120 + i, C)
             for i, (r, c, C) in enumerate([(3, 256, 256), (17, 512, 4096), (5, 4352, 4096),
                                            (33, 1024, 65536)])]
    one = synth.random_int8_tensor(16, 256, 1.0, 130, 1024)
    one["symbols"] = np.full(one["symbols"].shape, 77, np.uint8)
    allb = synth.random_int8_tensor(64, 512, 1.0, 131, 4096)
    allb["symbols"] = synth.random_bytes(64 * 512, 131).view(np.uint8)
    specs += [one, allb, synth.banded_int8_tensor(48, 2816, 4, 5, 2816 * 4)]
    return specs


@pytest.mark.parametrize("threads", [1, 3, 8])
def test_adaptive_batch_matches_oracle_byte_for_byte(E, threads):
    specs = _specs()
    c = oracle.encode_container_adaptive(specs)
    b = E.encode_batch_adaptive(specs, n_threads=threads)
    np.testing.assert_array_equal(b.blob, c.blob)
    got = np.stack([b.chunks["tensor"], b.chunks["n_symbols"], b.chunks["n_words"],
                    b.chunks["byte_offset"], b.chunks["elem_offset"]], axis=1).astype(np.uint64)
    np.testing.assert_array_equal(got, c.chunks)
    assert b.freq is None


def _try_plan(E, tensors, chunks, blob_bytes):
    h = ctypes.c_void_p()
    tensors = np.ascontiguousarray(tensors, E.TENSOR_DESC)
    chunks = np.ascontiguousarray(chunks, E.CHUNK_DESC)
    st = E.lib().entq_plan_adaptive(tensors.ctypes.data, tensors.size,
                                    chunks.ctypes.data if chunks.size else None, chunks.size,
                                    blob_bytes, FAKE_WS, 1 << 24, None, ctypes.byref(h))
    assert not h.value
    return st


def test_adaptive_plan_rejects_what_the_decoder_cannot_take(E):
    b = E.encode_batch_adaptive([synth.random_int8_tensor(8, 512, 1.5, 7, 1024)], n_threads=1)
    bb = b.blob.size
    # the regions include their tables: one byte short of the last one fails
    assert _try_plan(E, b.tensors, b.chunks, bb - 16) == -3
    # chunk size not a multiple of 256 symbols
    t = b.tensors.copy()
    t[0]["chunk_symbols"] = 1024 + 64
    assert _try_plan(E, t, b.chunks, bb) == -1
    # row length not a multiple of 256
    sp = synth.random_int8_tensor(8, 320, 1.5, 8, 1280)
    b2 = E.encode_batch_adaptive([sp], n_threads=1)
    assert _try_plan(E, b2.tensors, b2.chunks, b2.blob.size) == -1
    # exponent streams need whole blocks too (their rows need not be)
    t = b.tensors.copy()
    t[0]["kind"] = oracle.KIND_BF16EXP
    t[0]["chunk_symbols"] = 1024 + 64
    assert _try_plan(E, t, b.chunks, bb) == -1
    # output offset not a multiple of 16
    t = b.tensors.copy()
    t[0]["out_elem_offset"] = 8
    assert _try_plan(E, t, b.chunks, bb) == -1


def test_build_freq_chunks_equals_the_oracle_rule(E):
    rng = np.random.default_rng(44)
    rows = [np.zeros(256, np.uint32)]                                  # an empty chunk
    one = np.zeros(256, np.uint32); one[200] = 65536; rows.append(one)  # one symbol
    rows.append(np.full(256, 256, np.uint32))                          # uniform
    for i in range(300):
        c = rng.integers(0, 2000, 256).astype(np.uint32)
        c[rng.random(256) < 0.5 + 0.4 * (i % 2)] = 0
        c[int(rng.integers(0, 256))] += int(rng.integers(0, 1 << 20))
        rows.append(c)
    counts = np.stack(rows)
    for threads in (1, 5):
        got = E.build_freq_chunks(counts, n_threads=threads)
        for r, g in zip(counts, got):
            want = np.zeros(256, np.uint16) if r.sum() == 0 else oracle.quantize_freqs(r.astype(np.uint64))
            np.testing.assert_array_equal(g, want)
