"""Pins of the oracle's tile order (oracle.tile_order / oracle.untile), the
library's own layout of chunks for the fused product (the pages leave the
order of symbols inside a segment open): positions worked out by hand from
the layout's definition, the round trip, and a coded container in tile
order decoding back to the source codes."""
import numpy as np
import pytest

import oracle

# rows = 32, cols = 64, C = 32: four chunks of 16 x 32 (b, c) = (0,0), (0,1),
# (1,0), (1,1). Within a chunk p = 256 t + 64 s + l holds row 16 b + l % 16,
# column 32 c + 16 t + 4 (l // 16) + s. Worked out by hand:
HAND = [
    (0, 0, 0),      # t 0, s 0, l 0
    (1, 1, 0),      # l 1: the next row, same column
    (15, 15, 0),    # l 15: the band's last row
    (16, 0, 4),     # l 16: back to row 0, four columns on
    (63, 15, 12),   # l 63: row 15, column 4 * 3
    (64, 0, 1),     # s 1, l 0: column 1
    (65, 1, 1),
    (255, 15, 15),  # t 0, s 3, l 63: the tile's last element
    (256, 0, 16),   # t 1: the next 16 columns
    (511, 15, 31),  # the first chunk's last element
    (512, 0, 32),   # chunk 1 = band 0, column chunk 1
    (1024, 16, 0),  # chunk 2 = band 1, column chunk 0
    (1300, 20, 20), # chunk 2, p 276 = 256 + 20: t 1, s 0, l 20 -> row 16 + 4, col 16 + 4 * 1
    (2047, 31, 63), # the last element
]


def test_hand_worked_positions():
    w = np.arange(32 * 64, dtype=np.int64).reshape(32, 64)
    st = oracle.tile_order(w, 32, 64, 32)
    for p, r, c in HAND:
        assert st[p] == w[r, c], (p, r, c)


@pytest.mark.parametrize("rows,cols,C", [(16, 16, 16), (32, 64, 32), (48, 768, 256),
                                         (64, 512, 512), (16, 4096, 1024)])
def test_round_trip_and_permutation(rows, cols, C):
    rng = np.random.default_rng(rows + cols + C)
    w = rng.integers(0, 256, (rows, cols), dtype=np.uint8)
    st = oracle.tile_order(w, rows, cols, C)
    assert st.size == w.size
    assert np.array_equal(oracle.untile(st, rows, cols, C), w)
    idx = oracle.tile_order(np.arange(rows * cols).reshape(rows, cols), rows, cols, C)
    assert np.array_equal(np.sort(idx), np.arange(rows * cols))  # a permutation
    # each chunk holds exactly its 16 x C block
    for k in range(rows * cols // (16 * C)):
        b, c = divmod(k, cols // C)
        blk = np.sort(idx[k * 16 * C:(k + 1) * 16 * C])
        want = np.sort(np.arange(rows * cols).reshape(rows, cols)[16 * b:16 * b + 16,
                                                                  c * C:(c + 1) * C].ravel())
        assert np.array_equal(blk, want), k


def test_rejects_shapes_outside_the_layout():
    w = np.zeros((24, 64), np.uint8)
    with pytest.raises(AssertionError):
        oracle.tile_order(w, 24, 64, 32)   # rows not a multiple of 16
    with pytest.raises(AssertionError):
        oracle.tile_order(w[:16], 16, 64, 24)  # C not a multiple of 16


def test_coded_container_in_tile_order_decodes_to_the_source():
    rng = np.random.default_rng(3)
    rows, cols, C = 48, 512, 256
    codes = np.clip(np.rint(rng.normal(0, 2.0, rows * cols)), -127, 127).astype(np.int8)
    st = oracle.tile_order(codes.view(np.uint8), rows, cols, C)
    c = oracle.encode_container([dict(kind=oracle.KIND_INT8, rows=rows, cols=cols, symbols=st,
                                      chunk_symbols=16 * C)])
    assert c.n_chunks == rows * cols // (16 * C)
    (sym,), status = oracle.decode_container_symbols(c)
    assert (status == 0).all()
    assert np.array_equal(oracle.untile(sym, rows, cols, C).ravel(), codes.view(np.uint8))
