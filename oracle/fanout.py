"""The oracle's single-threaded chunk decode and dequantisation, run over
disjoint row-aligned ranges of a tensor in a pool of threads.

TEST INFRASTRUCTURE, like the rest of this package: only the tests, the smoke
check and the CPU-baseline and parity legs of the benchmark use it. It adds
no arithmetic. Every output element comes from the oracle's own functions
(orc_decode_tensor, or orc_decode_chunk on a per-chunk-table region, then
orc_dequant_tensor), each called on its own range of whole chunks and whole
rows. ctypes releases the interpreter lock during those calls, so the ranges
run in parallel, as independent segments [EntroLLM summary, "Metodología"
item 3].
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import ADAPTIVE_TABLE_BYTES, CONTAINER_LANES, lib, table_valid


def default_threads() -> int:
    """Host threads for the fan-out: the cores this process may run on,
    capped by OMP_NUM_THREADS when that is set."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _ranges(n: int, C: int, cols: int, n_items: int):
    """Element ranges [e0, e1) that start and end on chunk and row
    boundaries (multiples of lcm(C, cols), or the tensor's end), about
    n / n_items long."""
    unit = C * cols // math.gcd(C, cols)
    span = max(unit, -(-max(n // max(n_items, 1), 1) // unit) * unit)
    return [(e0, min(e0 + span, n)) for e0 in range(0, n, span)]


class _Result:
    def __init__(self):
        self.mismatches = 0        # bf16 outputs that differ from `compare`
        self.first_mismatch = -1   # the first of them (element index)
        self.bad_chunks = 0        # chunks whose decode status is not OK
        self.code_mismatches = 0   # decoded codes that differ from `codes_compare`


def _compare(res: _Result, e0: int, got: np.ndarray, want: np.ndarray):
    ne = got != want
    k = int(np.count_nonzero(ne))
    if k:
        res.mismatches += k
        res.first_mismatch = e0 + int(np.argmax(ne))


def tensor_bf16(blob: np.ndarray, chunks: np.ndarray, freq, kind: int, rows: int, cols: int,
                scales: np.ndarray, n_threads: int = 0, compare=None, codes_compare=None,
                adaptive: bool = False, pool: ThreadPoolExecutor | None = None):
    """Decodes and dequantises one tensor with the oracle, range by range.

    blob      the compressed bytes (uint8); byte offsets below index it
    chunks    the tensor's chunks in element order, array [k, 4] of
              (n_symbols, n_words, byte_offset, elem_offset), all of one
              chunk size except a shorter last one
    freq      the tensor's table (uint16 [256]); None with adaptive=True,
              where each region starts with its own table
    compare   None: return the bf16 output (uint16 [rows * cols]);
              otherwise an array of rows * cols uint16 (e.g. a GPU's
              output) that each range is compared with, and no output is
              kept
    codes_compare  optional uint8 [rows * cols] the decoded codes must equal

    Returns (out or None, result) where result has mismatches,
    first_mismatch (element index, -1 if none), bad_chunks (status != 0),
    code_mismatches."""
    n = rows * cols
    chunks = np.ascontiguousarray(chunks, dtype=np.uint64).reshape(-1, 4)
    C = int(chunks[0, 0]) if chunks.shape[0] else max(n, 1)
    n_threads = n_threads or default_threads()
    out = None if compare is not None else np.empty(n, np.uint16)
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32).ravel()
    if not adaptive:
        freq = np.ascontiguousarray(freq, dtype=np.uint16)
    L = lib()
    results = []

    def work(e0: int, e1: int):
        res = _Result()
        k0, k1 = e0 // C, -(-e1 // C)
        sub = chunks[k0:k1].copy()
        sub[:, 3] -= np.uint64(e0)
        codes = np.zeros(e1 - e0, np.uint8)
        if adaptive:
            for c in sub:
                cn, nw, off, eo = (int(v) for v in c)
                fr = blob[off:off + ADAPTIVE_TABLE_BYTES].view("<u2").astype(np.uint16)
                if not table_valid(fr):
                    res.bad_chunks += 1
                    continue
                s0 = off + ADAPTIVE_TABLE_BYTES
                states = blob[s0:s0 + 4 * CONTAINER_LANES].view("<u4").astype(np.uint32)
                w0 = s0 + 4 * CONTAINER_LANES
                words = blob[w0:w0 + 2 * nw].view("<u2").astype(np.uint16)
                w = words if words.size else np.zeros(1, np.uint16)
                st = L.orc_decode_chunk(states, w, nw, cn, CONTAINER_LANES, fr,
                                        codes[eo:eo + cn])
                if st != 0:
                    res.bad_chunks += 1
        else:
            st = np.zeros(max(sub.shape[0], 1), np.int32)
            bad = L.orc_decode_tensor(blob.ctypes.data, sub, sub.shape[0], freq, codes, st)
            if bad < 0:
                raise ValueError(f"orc_decode_tensor failed ({bad})")
            res.bad_chunks += int(bad)
        if codes_compare is not None:
            res.code_mismatches = int(np.count_nonzero(codes != codes_compare[e0:e1]))
        r0, r1 = e0 // cols, e1 // cols
        dst = np.empty(e1 - e0, np.uint16) if out is None else out[e0:e1]
        L.orc_dequant_tensor(codes, r1 - r0, cols, kind, scales[r0:r1], dst)
        if compare is not None:
            _compare(res, e0, dst, compare[e0:e1])
        return res

    spans = _ranges(n, C, cols, 4 * n_threads) if n else []
    if pool is not None:
        results = [f.result() for f in [pool.submit(work, a, b) for a, b in spans]]
    else:
        with ThreadPoolExecutor(n_threads) as ex:
            results = list(ex.map(lambda ab: work(*ab), spans))
    total = _Result()
    for r in results:
        total.mismatches += r.mismatches
        total.bad_chunks += r.bad_chunks
        total.code_mismatches += r.code_mismatches
        if r.first_mismatch >= 0 and total.first_mismatch < 0:
            total.first_mismatch = r.first_mismatch
    return out, total
