"""Plain CPU oracle for entropy-coded weight decoding.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline leg
of the benchmark may import this package. The product (``entropy_coded_weight_amd``)
never imports it, and the two share no code.

The arithmetic lives in ``oracle.c`` (single-threaded, uint64 state
arithmetic, one function per step of the method, each citing its source).
This module only loads that library with ctypes and assembles multi-tensor
containers from the per-tensor encoder; ``pyrans.py`` is an independent,
pure-Python restatement of the coder used to cross-check ``oracle.c`` on small
inputs.

Sources (page titles as they appear in the reference text):
  * EntQuant -- "Float8@2bits: Entropy Coding Enables Data-Free Model
    Compression": 8-bit base codes, flattened and ANS coded; storage =
    bitstream + per-channel scales + metadata; decode on the device before a
    block's forward pass (technical summary §2, "Codificación de Pesos",
    "Decodificación en Tiempo de Inferencia").
  * DFloat11 write-up: exponent byte entropy coded, sign+mantissa raw,
    bit-exact reconstruction ("Formato DFloat11").
  * EntroLLM: the coded stream is cut into independently decodable segments
    ("Metodología", item 3).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle.so")
SRC_PATH = os.path.join(HERE, "oracle.c")

PROB_BITS = 12
M = 1 << PROB_BITS
L = 1 << 16
CONTAINER_LANES = 64

KIND_INT8, KIND_E4M3, KIND_BF16EXP = 0, 1, 2
STATUS_OK, STATUS_BAD_STATE, STATUS_BAD_WORDS, STATUS_BAD_TABLE = 0, 1, 2, 3


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into liboracle.so next to it."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
             "-o", tmp, SRC_PATH, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None

_u8p = np.ctypeslib.ndpointer(np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(np.uint16, flags="C_CONTIGUOUS")
_u32p = np.ctypeslib.ndpointer(np.uint32, flags="C_CONTIGUOUS")
_u64p = np.ctypeslib.ndpointer(np.uint64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(np.int32, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(np.float32, flags="C_CONTIGUOUS")


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        L_ = ctypes.CDLL(LIB_PATH)
        c = ctypes
        sig = {
            "orc_bf16_from_f32_bits": (c.c_uint16, [c.c_uint32]),
            "orc_e4m3_to_f32_bits": (c.c_uint32, [c.c_uint8]),
            "orc_int8_to_f32_bits": (c.c_uint32, [c.c_uint8]),
            "orc_dequant_bf16": (c.c_uint16, [c.c_uint8, c.c_int, c.c_float]),
            "orc_mul_f32_bits": (c.c_uint32, [c.c_uint32, c.c_uint32]),
            "orc_bf16_merge": (c.c_uint16, [c.c_uint8, c.c_uint8]),
            "orc_quantize_freqs": (c.c_int, [_u64p, _u16p]),
            "orc_table_valid": (c.c_int, [_u16p]),
            "orc_encode_chunk": (c.c_int64, [_u8p, c.c_uint32, c.c_uint32, _u16p, _u32p, _u16p]),
            "orc_decode_chunk": (c.c_int, [_u32p, _u16p, c.c_uint32, c.c_uint32, c.c_uint32, _u16p, _u8p]),
            "orc_n_chunks": (c.c_uint64, [c.c_uint64, c.c_uint32]),
            "orc_tensor_bound": (c.c_uint64, [c.c_uint64, c.c_uint32]),
            "orc_encode_tensor": (c.c_int64, [_u8p, c.c_uint64, c.c_uint32, _u16p, _u8p, c.c_uint64, _u64p]),
            "orc_decode_tensor": (c.c_int64, [c.c_void_p, _u64p, c.c_uint64, _u16p, _u8p, _i32p]),
            "orc_count_symbols": (None, [_u8p, c.c_uint64, _u64p]),
            "orc_dequant_tensor": (None, [_u8p, c.c_uint64, c.c_uint64, c.c_int, _f32p, _u16p]),
            "orc_bf16_split_array": (None, [_u16p, c.c_uint64, _u8p, _u8p]),
            "orc_bf16_merge_array": (None, [_u8p, _u8p, c.c_uint64, _u16p]),
            "orc_bf16_from_f32_array": (None, [_u32p, c.c_uint64, _u16p]),
            "orc_e4m3_table": (None, [_u32p]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L_, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L_
    return _lib


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def bf16_from_f32_bits(u32: np.ndarray) -> np.ndarray:
    u32 = np.ascontiguousarray(u32, dtype=np.uint32).ravel()
    out = np.empty(u32.size, np.uint16)
    lib().orc_bf16_from_f32_array(u32, u32.size, out)
    return out


def e4m3_table() -> np.ndarray:
    """fp32 bit patterns of the 256 e4m3 codes."""
    out = np.empty(256, np.uint32)
    lib().orc_e4m3_table(out)
    return out


def mul_f32_bits(vb: int, sb: int) -> int:
    return int(lib().orc_mul_f32_bits(vb & 0xFFFFFFFF, sb & 0xFFFFFFFF))


def dequant_bf16(code: int, kind: int, scale: float) -> int:
    return int(lib().orc_dequant_bf16(code & 0xFF, kind, ctypes.c_float(scale)))


def dequant_tensor(codes: np.ndarray, rows: int, cols: int, kind: int,
                   scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8).ravel()
    scales = np.ascontiguousarray(scales, dtype=np.float32).ravel()
    assert codes.size == rows * cols and scales.size >= rows
    out = np.empty(rows * cols, np.uint16)
    lib().orc_dequant_tensor(codes, rows, cols, kind, scales, out)
    return out


def bf16_split(w: np.ndarray):
    w = np.ascontiguousarray(w, dtype=np.uint16).ravel()
    e = np.empty(w.size, np.uint8)
    sm = np.empty(w.size, np.uint8)
    lib().orc_bf16_split_array(w, w.size, e, sm)
    return e, sm


def bf16_merge(e: np.ndarray, sm: np.ndarray) -> np.ndarray:
    e = np.ascontiguousarray(e, dtype=np.uint8).ravel()
    sm = np.ascontiguousarray(sm, dtype=np.uint8).ravel()
    assert e.size == sm.size
    out = np.empty(e.size, np.uint16)
    lib().orc_bf16_merge_array(e, sm, e.size, out)
    return out


# --------------------------------------------------------------------------
# frequency tables and the chunk coder
# --------------------------------------------------------------------------

def count_symbols(sym: np.ndarray) -> np.ndarray:
    sym = np.ascontiguousarray(sym, dtype=np.uint8).ravel()
    out = np.zeros(256, np.uint64)
    lib().orc_count_symbols(sym, sym.size, out)
    return out


def quantize_freqs(counts: np.ndarray) -> np.ndarray:
    counts = np.ascontiguousarray(counts, dtype=np.uint64)
    assert counts.size == 256
    f = np.zeros(256, np.uint16)
    lib().orc_quantize_freqs(counts, f)
    return f


def table_valid(freq: np.ndarray) -> bool:
    return bool(lib().orc_table_valid(np.ascontiguousarray(freq, dtype=np.uint16)))


def encode_chunk(sym: np.ndarray, K: int, freq: np.ndarray):
    """Returns (states[K] uint32, words uint16) for one chunk coded with K lanes."""
    sym = np.ascontiguousarray(sym, dtype=np.uint8).ravel()
    freq = np.ascontiguousarray(freq, dtype=np.uint16)
    states = np.zeros(max(K, 1), np.uint32)
    words = np.zeros(max(sym.size, 1), np.uint16)
    nw = lib().orc_encode_chunk(sym, sym.size, K, freq, states, words)
    if nw < 0:
        raise ValueError(f"orc_encode_chunk failed ({nw})")
    return states[:K].copy(), words[:nw].copy()


def decode_chunk(states: np.ndarray, words: np.ndarray, n: int, K: int, freq: np.ndarray):
    """Returns (symbols uint8[n], status)."""
    states = np.ascontiguousarray(states, dtype=np.uint32)
    words = np.ascontiguousarray(words, dtype=np.uint16)
    w = words if words.size else np.zeros(1, np.uint16)
    out = np.zeros(max(n, 1), np.uint8)
    st = lib().orc_decode_chunk(states, w, words.size, n, K,
                                np.ascontiguousarray(freq, dtype=np.uint16), out)
    if st < 0:
        raise ValueError(f"orc_decode_chunk failed ({st})")
    return out[:n].copy(), int(st)


def encode_tensor(sym: np.ndarray, chunk_symbols: int, freq: np.ndarray):
    """One tensor -> (blob uint8, desc uint64[k, 4] = n_symbols, n_words,
    byte_offset (relative to blob), elem_offset)."""
    sym = np.ascontiguousarray(sym, dtype=np.uint8).ravel()
    freq = np.ascontiguousarray(freq, dtype=np.uint16)
    n = sym.size
    k = int(lib().orc_n_chunks(n, chunk_symbols))
    cap = int(lib().orc_tensor_bound(n, chunk_symbols))
    blob = np.zeros(max(cap, 16), np.uint8)
    desc = np.zeros((max(k, 1), 4), np.uint64)
    nb = lib().orc_encode_tensor(sym if n else np.zeros(1, np.uint8), n, chunk_symbols,
                                 freq, blob, blob.size, desc)
    if nb < 0:
        raise ValueError(f"orc_encode_tensor failed ({nb})")
    return blob[:nb].copy(), desc[:k].copy()


def decode_tensor(blob: np.ndarray, desc: np.ndarray, freq: np.ndarray, n: int,
                  base_offset: int = 0):
    """Decode one tensor's chunks. desc byte offsets are relative to
    blob[base_offset:]. Returns (symbols uint8[n], status int32[k])."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    desc = np.ascontiguousarray(desc, dtype=np.uint64).reshape(-1, 4)
    out = np.zeros(max(n, 1), np.uint8)
    st = np.zeros(max(desc.shape[0], 1), np.int32)
    ptr = blob.ctypes.data + base_offset
    r = lib().orc_decode_tensor(ptr, desc if desc.size else np.zeros((1, 4), np.uint64),
                                desc.shape[0], np.ascontiguousarray(freq, dtype=np.uint16),
                                out, st)
    if r < 0:
        raise ValueError(f"orc_decode_tensor failed ({r})")
    return out[:n].copy(), st[:desc.shape[0]].copy()


# --------------------------------------------------------------------------
# multi-tensor container (a "layer": the tensors decoded together)
# --------------------------------------------------------------------------

class Container:
    """The compressed form of a list of tensors.

    blob    : uint8 array holding every chunk region, tensor after tensor,
              chunk after chunk (each region 16-byte aligned).
    tensors : list of dicts with kind, rows, cols, chunk_symbols, n_symbols,
              out_elem_offset, scale_row_offset and freq (uint16[256]).
    chunks  : uint64 array [n_chunks, 5] = tensor, n_symbols, n_words,
              byte_offset (from the start of blob), elem_offset (inside the
              tensor).
    """

    def __init__(self, blob, tensors, chunks):
        self.blob = blob
        self.tensors = tensors
        self.chunks = chunks

    @property
    def n_chunks(self):
        return int(self.chunks.shape[0])

    def payload_bytes(self):
        return int(self.blob.size)


def encode_container(specs, chunk_symbols_default: int = 65536) -> Container:
    """specs: list of dicts {kind, rows, cols, symbols (uint8 array of
    rows*cols), optional chunk_symbols}. Each tensor gets its own frequency
    table. Outputs of the tensors are laid out one after the other, as are
    their scale rows."""
    blobs, tensors, rows_ = [], [], []
    off = 0
    out_off = 0
    scale_off = 0
    for t, sp in enumerate(specs):
        sym = np.ascontiguousarray(sp["symbols"], dtype=np.uint8).ravel()
        rows, cols = int(sp["rows"]), int(sp["cols"])
        assert sym.size == rows * cols
        C = int(sp.get("chunk_symbols", chunk_symbols_default))
        freq = quantize_freqs(count_symbols(sym))
        if sym.size == 0:
            freq = np.zeros(256, np.uint16)
            freq[0] = M
        blob, desc = encode_tensor(sym, C, freq)
        for r in desc:
            rows_.append((t, int(r[0]), int(r[1]), off + int(r[2]), int(r[3])))
        blobs.append(blob)
        off += blob.size
        tensors.append(dict(kind=int(sp["kind"]), rows=rows, cols=cols, chunk_symbols=C,
                            n_symbols=sym.size, out_elem_offset=out_off,
                            scale_row_offset=scale_off, freq=freq))
        out_off += sym.size
        scale_off += rows
    blob = np.concatenate(blobs) if blobs else np.zeros(0, np.uint8)
    chunks = np.array(rows_, dtype=np.uint64).reshape(-1, 5)
    return Container(blob, tensors, chunks)


def decode_container_symbols(c: Container):
    """Returns (list of per-tensor symbol arrays, per-chunk status int32 in
    container chunk order)."""
    outs = []
    status = np.zeros(c.n_chunks, np.int32)
    for t, td in enumerate(c.tensors):
        idx = np.nonzero(c.chunks[:, 0] == t)[0]
        desc = np.stack([c.chunks[idx, 1], c.chunks[idx, 2], c.chunks[idx, 3],
                         c.chunks[idx, 4]], axis=1).astype(np.uint64) if idx.size else \
            np.zeros((0, 4), np.uint64)
        sym, st = decode_tensor(c.blob if c.blob.size else np.zeros(16, np.uint8), desc,
                                td["freq"], td["n_symbols"])
        status[idx] = st
        outs.append(sym)
    return outs, status


def decode_container_bf16(c: Container, scales: np.ndarray):
    """bf16 output (uint16) of every tensor laid out at out_elem_offset; int8
    and e4m3 tensors use scales[scale_row_offset + row]."""
    syms, status = decode_container_symbols(c)
    total = sum(t["n_symbols"] for t in c.tensors)
    out = np.zeros(total, np.uint16)
    for td, sym in zip(c.tensors, syms):
        o = td["out_elem_offset"]
        so = td["scale_row_offset"]
        out[o:o + td["n_symbols"]] = dequant_tensor(sym, td["rows"], td["cols"], td["kind"],
                                                    scales[so:so + td["rows"]])
    return out, status


# --------------------------------------------------------------------------
# per-chunk (adaptive) tables
# --------------------------------------------------------------------------
#
# EntroLLM names adaptive entropy coding as its next step (EntroLLM summary,
# "Significado y Afirmaciones"); the pages say no more. Reading taken here:
# every chunk is coded with the table of its own symbol counts (rule C2
# applied to the chunk), stored at the head of the chunk's region. The coder
# itself is unchanged.
#
# Region of a chunk: u16 freq[256] (little-endian), u32 states[64], u16
# words[n_words], zeros up to a 16-byte boundary.

ADAPTIVE_TABLE_BYTES = 2 * 256


# ---- tile-ordered chunks (the library's layout for the fused product) ----
#
# The pages cut a tensor's coded stream into independently decodable
# segments [EntroLLM, "Metodología", item 3] and leave the order of the
# symbols inside them open; the discussion under the DFloat11 write-up asks
# for tiles decompressed inside the matrix multiply. In this layout a tensor
# [rows x cols] (rows a multiple of 16, cols a multiple of C, C a multiple of
# 16) is cut into chunks of 16 rows x C columns: band b = rows 16b .. 16b+15,
# column chunk c = columns cC .. cC+C-1, chunk index b * (cols / C) + c.
# Inside a chunk, stream position p = 256 t + 64 s + l (t: 16-column tile,
# s: 0..3, l: 0..63) holds the weight at row 16 b + (l mod 16) and column
# c C + 16 t + 4 (l div 16) + s. The chunks follow one another in index order.
# Only the order of the symbols changes: counts, tables and the coder do not.

def tile_order(codes: np.ndarray, rows: int, cols: int, C: int) -> np.ndarray:
    """The tensor's symbols (row-major, rows x cols) in tile order."""
    assert rows % 16 == 0 and C % 16 == 0 and C > 0 and cols % C == 0
    w = np.ascontiguousarray(codes).reshape(rows, cols)
    out = np.empty(rows * cols, w.dtype)
    p = np.arange(16 * C)
    t, s, l = p // 256, (p // 64) % 4, p % 64
    r_in, c_in = l % 16, 16 * t + 4 * (l // 16) + s   # within the chunk
    k = 0
    for b in range(rows // 16):
        for c in range(cols // C):
            out[k * 16 * C:(k + 1) * 16 * C] = w[16 * b + r_in, c * C + c_in]
            k += 1
    return out


def untile(stream: np.ndarray, rows: int, cols: int, C: int) -> np.ndarray:
    """Inverse of tile_order: the row-major [rows, cols] tensor."""
    assert rows % 16 == 0 and C % 16 == 0 and C > 0 and cols % C == 0
    stream = np.ascontiguousarray(stream).ravel()
    w = np.empty((rows, cols), stream.dtype)
    p = np.arange(16 * C)
    t, s, l = p // 256, (p // 64) % 4, p % 64
    r_in, c_in = l % 16, 16 * t + 4 * (l // 16) + s
    k = 0
    for b in range(rows // 16):
        for c in range(cols // C):
            w[16 * b + r_in, c * C + c_in] = stream[k * 16 * C:(k + 1) * 16 * C]
            k += 1
    return w


def adaptive_region_bytes(n_words: int) -> int:
    return (ADAPTIVE_TABLE_BYTES + 4 * CONTAINER_LANES + 2 * n_words + 15) // 16 * 16


def encode_container_adaptive(specs, chunk_symbols_default: int = 65536) -> Container:
    """As encode_container, but each chunk carries its own table; the
    tensor records carry none (freq = None)."""
    regions, tensors, rows_ = [], [], []
    off = out_off = scale_off = 0
    for t, sp in enumerate(specs):
        sym = np.ascontiguousarray(sp["symbols"], dtype=np.uint8).ravel()
        rows, cols = int(sp["rows"]), int(sp["cols"])
        assert sym.size == rows * cols
        C = int(sp.get("chunk_symbols", chunk_symbols_default))
        for e0 in range(0, sym.size, C):
            part = sym[e0:e0 + C]
            freq = quantize_freqs(count_symbols(part))
            states, words = encode_chunk(part, CONTAINER_LANES, freq)
            region = np.zeros(adaptive_region_bytes(words.size), np.uint8)
            region[:ADAPTIVE_TABLE_BYTES] = freq.astype("<u2").view(np.uint8)
            s0 = ADAPTIVE_TABLE_BYTES
            region[s0:s0 + 4 * CONTAINER_LANES] = states.astype("<u4").view(np.uint8)
            w0 = s0 + 4 * CONTAINER_LANES
            region[w0:w0 + 2 * words.size] = words.astype("<u2").view(np.uint8)
            rows_.append((t, part.size, words.size, off, e0))
            regions.append(region)
            off += region.size
        tensors.append(dict(kind=int(sp["kind"]), rows=rows, cols=cols, chunk_symbols=C,
                            n_symbols=sym.size, out_elem_offset=out_off,
                            scale_row_offset=scale_off, freq=None))
        out_off += sym.size
        scale_off += rows
    blob = np.concatenate(regions) if regions else np.zeros(0, np.uint8)
    chunks = np.array(rows_, dtype=np.uint64).reshape(-1, 5)
    return Container(blob, tensors, chunks)


def decode_adaptive_chunk(blob: np.ndarray, byte_offset: int, n: int, n_words: int):
    """(symbols uint8[n], status) of one chunk region of an adaptive
    container; status STATUS_BAD_TABLE if its table does not sum to 4096."""
    r = blob[byte_offset:byte_offset + adaptive_region_bytes(n_words)]
    freq = r[:ADAPTIVE_TABLE_BYTES].view("<u2").astype(np.uint16)
    if not table_valid(freq):
        return np.zeros(n, np.uint8), STATUS_BAD_TABLE
    s0 = ADAPTIVE_TABLE_BYTES
    states = r[s0:s0 + 4 * CONTAINER_LANES].view("<u4").astype(np.uint32)
    w0 = s0 + 4 * CONTAINER_LANES
    words = r[w0:w0 + 2 * n_words].view("<u2").astype(np.uint16)
    return decode_chunk(states, words, n, CONTAINER_LANES, freq)


def decode_container_adaptive_symbols(c: Container):
    """(list of per-tensor symbol arrays, per-chunk status in container chunk
    order) of an adaptive container."""
    outs = [np.zeros(td["n_symbols"], np.uint8) for td in c.tensors]
    status = np.zeros(c.n_chunks, np.int32)
    for k, (t, n, nw, off, e0) in enumerate(c.chunks.astype(np.int64)):
        sym, st = decode_adaptive_chunk(c.blob, int(off), int(n), int(nw))
        outs[t][e0:e0 + n] = sym
        status[k] = st
    return outs, status


def decode_container_adaptive_bf16(c: Container, scales: np.ndarray):
    syms, status = decode_container_adaptive_symbols(c)
    total = sum(t["n_symbols"] for t in c.tensors)
    out = np.zeros(total, np.uint16)
    for td, sym in zip(c.tensors, syms):
        o, so = td["out_elem_offset"], td["scale_row_offset"]
        out[o:o + td["n_symbols"]] = dequant_tensor(sym, td["rows"], td["cols"], td["kind"],
                                                    scales[so:so + td["rows"]])
    return out, status


def decode_container_adaptive_split(c: Container, signmant: np.ndarray):
    """(bf16 words, per-chunk status) of an adaptive container of BF16EXP
    tensors: each tensor's decoded exponent bytes merged with its raw
    sign+mantissa bytes, signmant being indexed like the output [DFloat11
    write-up, "Formato DFloat11"]. Composition of the adaptive decode and
    bf16_merge, nothing else."""
    syms, status = decode_container_adaptive_symbols(c)
    total = max((t["out_elem_offset"] + t["n_symbols"] for t in c.tensors), default=0)
    out = np.zeros(total, np.uint16)
    for td, sym in zip(c.tensors, syms):
        o, n = td["out_elem_offset"], td["n_symbols"]
        out[o:o + n] = bf16_merge(sym, np.ascontiguousarray(signmant[o:o + n], np.uint8))
    return out, status


def _isnan_bits(u: int) -> bool:
    return (u & 0x7F800000) == 0x7F800000 and (u & 0x007FFFFF) != 0
