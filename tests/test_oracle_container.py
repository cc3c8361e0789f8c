"""Pins of the oracle's container and of its compressed sizes on the
synthetic workloads.

Sizes: the pages report what entropy coding reaches on trained weights --
about 2 bits/parameter for EntQuant Int8 codes and about 6.5 bits for
entropy-coded Float8 (EntQuant summary "Float8@2bits ...", technical part §2
and Figure 4's caption on the sciencestack page), and about 2.6 bits for the
BF16 exponent (DFloat11 write-up, "Margen de compresión restante en el
exponente de BFloat16"). The synthetic inputs have closed-form entropies
(computed here from their distributions), and the coder must land within a
stated overhead of the table's cross-entropy plus the fixed state cost."""
import math

import numpy as np
import pytest

import oracle
import synth


def entropy_bits(sym):
    c = np.bincount(sym, minlength=256).astype(np.float64)
    p = c[c > 0] / c.sum()
    return float(-(p * np.log2(p)).sum())


def cross_entropy_bits(sym, freq):
    c = np.bincount(sym, minlength=256).astype(np.float64)
    nz = c > 0
    return float((c[nz] * np.log2(oracle.M / freq[nz].astype(np.float64))).sum())


def closed_form_entropy(pmf):
    p = pmf[pmf > 0]
    return float(-(p * np.log2(p)).sum())


def check_size(sym, C, blob, desc, freq):
    """payload bits <= (1 + 1%) * cross-entropy; plus 64 x 32 state bits and
    < 16 bytes of padding per chunk."""
    n_chunks = desc.shape[0]
    words = int(desc[:, 1].sum())
    assert blob.size == sum(-(-(256 + 2 * int(w)) // 16) * 16 for w in desc[:, 1])
    payload_bits = 16 * words
    ce = cross_entropy_bits(sym, freq)
    assert payload_bits <= 1.01 * ce + 16 * n_chunks * 64  # (at most 16 unused bits per lane)
    assert payload_bits >= ce - 16 * 64 * n_chunks  # the states hold at most 16 bits each above L
    return payload_bits, ce


def test_tiny_laplace_round_trip_and_entropy():
    t = synth.tiny_int8_laplace()[0]
    sym = t["symbols"]
    exact = closed_form_entropy(synth.rounded_pmf(lambda x: synth.laplace_cdf(x, 2.0)))
    assert abs(exact - 3.4552) < 1e-3
    assert abs(entropy_bits(sym) - exact) < 0.02  # 65,536 samples
    freq = oracle.quantize_freqs(oracle.count_symbols(sym))
    blob, desc = oracle.encode_tensor(sym, 4096, freq)
    assert desc.shape == (16, 4)
    assert np.all(desc[:, 2] % 16 == 0)
    out, st = oracle.decode_tensor(blob, desc, freq, sym.size)
    assert np.all(st == 0) and np.array_equal(out, sym)
    check_size(sym, 4096, blob, desc, freq)


def test_e4m3_matrix_round_trip_and_entropy():
    t = synth.e4m3_matrix()[0]
    sym = t["symbols"]
    h = entropy_bits(sym)
    assert 6.3 < h < 6.6  # the pages: entropy-coded Float8 ~6.5 bits
    freq = oracle.quantize_freqs(oracle.count_symbols(sym))
    blob, desc = oracle.encode_tensor(sym, 65536, freq)
    assert desc.shape[0] == 256
    out, st = oracle.decode_tensor(blob, desc, freq, sym.size)
    assert np.all(st == 0) and np.array_equal(out, sym)
    bits, ce = check_size(sym, 65536, blob, desc, freq)
    # quantising 254 probabilities to twelve bits costs under 0.5% of the rate
    assert (ce / sym.size - h) / h < 0.005


def test_bf16_exponent_stream_round_trip_bit_exact():
    t = synth.bf16_weights(2048, 2048)[0]
    w = t["bf16"]
    e, sm = oracle.bf16_split(w)
    h = entropy_bits(e)
    assert 2.4 < h < 2.7  # the pages: ~2.6 bits for the exponent
    assert entropy_bits(sm) > 7.9  # sign+mantissa close to incompressible
    freq = oracle.quantize_freqs(oracle.count_symbols(e))
    blob, desc = oracle.encode_tensor(e, 65536, freq)
    e2, st = oracle.decode_tensor(blob, desc, freq, e.size)
    assert np.all(st == 0)
    np.testing.assert_array_equal(oracle.bf16_merge(e2, sm), w)
    check_size(e, 65536, blob, desc, freq)


@pytest.mark.parametrize("sigma,expect", [(1.0, 2.1048), (0.8, 1.813), (3.0, 3.639)])
def test_normal_int8_entropy_closed_form(sigma, expect):
    exact = closed_form_entropy(synth.rounded_pmf(lambda x: synth.normal_cdf(x, sigma)))
    assert abs(exact - expect) < 2e-3
    sym = synth.int8_codes(lambda x: synth.normal_cdf(x, sigma), 2_000_000,
                           synth.key(77, int(sigma * 10), 0, 0)).view(np.uint8)
    assert abs(entropy_bits(sym) - exact) < 0.005


def test_13b_block_tensor_round_trip_and_rate():
    blk = synth.llama2_13b_block(shapes=[("k", 5120, 5120)])[0]
    sym = blk["symbols"]
    freq = oracle.quantize_freqs(oracle.count_symbols(sym))
    blob, desc = oracle.encode_tensor(sym, 65536, freq)
    assert desc.shape[0] == 400
    out, st = oracle.decode_tensor(blob, desc, freq, sym.size)
    assert np.all(st == 0) and np.array_equal(out, sym)
    bits, ce = check_size(sym, 65536, blob, desc, freq)
    rate = 8.0 * blob.size / sym.size
    assert 2.1 < rate < 2.2  # ~2.1 bits/parameter including the states


def test_70b_layer_sampled_tensor_round_trip():
    L0 = synth.llama2_70b_layer(0, shapes=[("q", 8192, 8192), ("k", 1024, 8192)])
    for t in L0[1:]:
        sym = t["symbols"]
        sigma = t["dist"][1]
        assert 0.8 <= sigma <= 3.0
        freq = oracle.quantize_freqs(oracle.count_symbols(sym))
        blob, desc = oracle.encode_tensor(sym, 65536, freq)
        out, st = oracle.decode_tensor(blob, desc, freq, sym.size)
        assert np.all(st == 0) and np.array_equal(out, sym)
        check_size(sym, 65536, blob, desc, freq)


@pytest.mark.parametrize("n,C", [(0, 4096), (1, 4096), (63, 4096), (64, 4096), (65, 64),
                                 (4095, 4096), (4097, 4096), (10000, 640), (70000, 65536)])
def test_ragged_and_edge_sizes(n, C):
    rng = np.random.default_rng(n)
    sym = rng.integers(0, 256, size=n).astype(np.uint8) if n else np.zeros(0, np.uint8)
    if n:
        freq = oracle.quantize_freqs(oracle.count_symbols(sym))
    else:
        freq = np.zeros(256, np.uint16)
        freq[0] = oracle.M
    blob, desc = oracle.encode_tensor(sym, C, freq)
    assert desc.shape[0] == -(-n // C)
    if n:
        assert int(desc[-1, 0]) == n - C * (desc.shape[0] - 1)
    out, st = oracle.decode_tensor(blob if blob.size else np.zeros(16, np.uint8), desc, freq, n)
    assert np.all(st == 0) and np.array_equal(out, sym)


def test_multi_tensor_container_layout():
    specs = [synth.random_int8_tensor(64, 192, 1.5, s, 4096) for s in range(3)]
    specs.append(dict(kind=0, rows=3, cols=5, symbols=np.full(15, 9, np.uint8),
                      chunk_symbols=64))
    c = oracle.encode_container(specs)
    assert c.n_chunks == 3 + 3 + 3 + 1
    # regions are contiguous, 16-byte aligned, in tensor then chunk order
    offs = c.chunks[:, 3].astype(np.int64)
    assert np.all(offs % 16 == 0) and np.all(np.diff(offs) > 0)
    syms, status = oracle.decode_container_symbols(c)
    assert np.all(status == 0)
    for sp, s in zip(specs, syms):
        np.testing.assert_array_equal(s, sp["symbols"])
    # a one-symbol tensor codes no words
    assert int(c.chunks[-1, 2]) == 0
