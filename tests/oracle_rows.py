"""Helpers for GPU tests at full size: the oracle's bf16 weights of a whole
tensor (decoded and dequantised chunk range by chunk range on all host
threads, oracle/fanout.py), and the fp64 check of a product against them."""
import numpy as np

from oracle import fanout


def desc_of(chunks):
    """(n_symbols, n_words, byte_offset, elem_offset) rows of one tensor's
    CHUNK_DESC records, in element order."""
    ch = chunks[np.argsort(chunks["elem_offset"])]
    return np.stack([ch["n_symbols"], ch["n_words"], ch["byte_offset"], ch["elem_offset"]],
                    axis=1).astype(np.uint64)


def tensor_from_oracle(blob, chunks, freq, spec, adaptive=False):
    """bf16 bits (uint16 [rows, cols]) of one tensor, every element decoded
    and dequantised by the oracle from the container's bytes (chunks: that
    tensor's CHUNK_DESC rows)."""
    out, res = fanout.tensor_bf16(blob, desc_of(chunks), freq, spec["kind"], spec["rows"],
                                  spec["cols"], spec["scales"], adaptive=adaptive)
    assert res.bad_chunks == 0
    return out.reshape(spec["rows"], spec["cols"])


def _f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def check_product(y, x, w_bits, block_rows=2048):
    """Every y[:, r] against the fp64 product x . w[r] of the bf16 weights
    w_bits [rows, cols]: |y - ref| <= cols * 2^-24 * sum |x w| (products of
    two bf16 are exact in fp32; each of at most cols additions rounds once).
    Returns the number of rows checked."""
    rows, cols = w_bits.shape
    xd = np.asarray(x, np.float64)
    ax = np.abs(xd)
    for r0 in range(0, rows, block_rows):
        w = _f64(w_bits[r0:r0 + block_rows])
        ref = xd @ w.T
        bound = cols * 2.0 ** -24 * (ax @ np.abs(w).T)
        got = y[:, r0:r0 + w.shape[0]]
        ok = np.abs(got - ref) <= bound
        assert ok.all(), (r0 + int(np.argmin(ok.all(axis=0))), float(np.abs(got - ref).max()))
    return rows
