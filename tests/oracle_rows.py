"""Helpers for GPU tests at full size: expected values for a few weight rows
or chunks, each decoded by the oracle from the one chunk that holds it (the
oracle decoding whole 70B-sized tensors would take too long)."""
import numpy as np

import oracle


def chunk_symbols_from_oracle(blob, chunks, freq, elem_offset):
    """The code bytes of the chunk of one tensor starting at elem_offset
    (chunks: that tensor's CHUNK_DESC rows)."""
    c = chunks[chunks["elem_offset"] == elem_offset][0]
    off, n, nw = int(c["byte_offset"]), int(c["n_symbols"]), int(c["n_words"])
    states = blob[off:off + 256].view(np.uint32)
    words = blob[off + 256:off + 256 + 2 * nw].view(np.uint16)
    sym, st = oracle.decode_chunk(states, words, n, 64, freq)
    assert st == 0
    return sym


def rows_from_oracle(blob, chunks, freq, spec, rows):
    """bf16 bits (uint16 [cols]) of the given weight rows of one tensor."""
    cols, C = spec["cols"], spec["chunk_symbols"]
    out = {}
    for r in rows:
        k = (r * cols) // C
        i0 = r * cols - k * C
        if i0 + cols <= C:
            row = chunk_symbols_from_oracle(blob, chunks, freq, k * C)[i0:i0 + cols]
        else:  # the row continues in the next chunk
            a = chunk_symbols_from_oracle(blob, chunks, freq, k * C)[i0:]
            b = chunk_symbols_from_oracle(blob, chunks, freq, (k + 1) * C)[:cols - a.size]
            row = np.concatenate([a, b])
        out[r] = oracle.dequant_tensor(row, 1, cols, spec["kind"], spec["scales"][r:r + 1])
    return out
