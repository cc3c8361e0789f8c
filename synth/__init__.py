"""Seeded synthetic inputs for entropy-coded weight decoding.

Input generation only -- no coder or dequantiser arithmetic lives here. Both
the oracle's tests and the GPU path's tests and benchmark take their inputs
from this module, so the two sides always see the same bytes.

Why synthetic: the pages measure on trained LLM weights (LLaMA-2 7B/13B/70B
after EntQuant's optimisation; BF16 checkpoints for DFloat11), which are not
available here and are not needed to exercise a decoder. The tensors below
have those models' shapes and the entropy regime the pages report: about 2
bits/parameter for EntQuant Int8 codes and about 6.5 bits for entropy-coded
Float8 (EntQuant summary "Float8@2bits ...", technical part §2 and Figure 4's
caption), and an exponent of about 2.6 bits for BF16 weights (DFloat11
write-up, "Margen de compresión restante en el exponente de BFloat16").

Recipe (all draws from the counter-based generator in synth.c, keyed by
(workload, layer, tensor, kind) with kind 0 = values, 1 = scales, 2 = sigma):
  * Int8 codes = round(X) clipped to [-127, 127] for X ~ N(0, sigma) or
    Laplace(0, b), sampled exactly by inverse CDF over the 255 integers
    (the distribution of the rounded value is computed in float64 here).
  * Per-row fp32 scales ~ U[1e-3, 1e-2].
  * Float8: w ~ N(0, 0.02) in fp32 (Box-Muller), scale = fl32(row absmax /
    448), codes = e4m3(fl32(w / scale)) with torch's round-to-nearest-even
    cast.
  * BF16: w ~ N(0, 0.02) in fp32, rounded to bf16 by torch's RNE cast.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsynth.so")
SRC_PATH = os.path.join(HERE, "synth.c")

MASK64 = (1 << 64) - 1


def build(force: bool = True) -> str:
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fPIC", "-shared", "-o", tmp, SRC_PATH,
                               "-lm", "-lpthread"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(LIB_PATH)
        c = ctypes
        lib.syn_mix64.restype = c.c_uint64
        lib.syn_mix64.argtypes = [c.c_uint64]
        lib.syn_draw.restype = c.c_uint64
        lib.syn_draw.argtypes = [c.c_uint64, c.c_uint64]
        lib.syn_codes_int8.restype = None
        lib.syn_codes_int8.argtypes = [c.c_uint64, c.c_void_p, c.c_uint64, c.c_void_p, c.c_int]
        lib.syn_normal_f32.restype = None
        lib.syn_normal_f32.argtypes = [c.c_uint64, c.c_double, c.c_uint64, c.c_void_p, c.c_int]
        lib.syn_uniform_f32.restype = None
        lib.syn_uniform_f32.argtypes = [c.c_uint64, c.c_double, c.c_double, c.c_uint64,
                                        c.c_void_p, c.c_int]
        _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def key(*parts: int) -> int:
    """Stream key of a tuple of small integers."""
    k = 0x6A09E667F3BCC908
    for p in parts:
        k = _L().syn_mix64((k ^ (int(p) & MASK64)) & MASK64)
    return int(k)


# --------------------------------------------------------------------------
# distributions of a rounded-and-clipped variable over -127..127
# --------------------------------------------------------------------------

def normal_cdf(x: float, sigma: float) -> float:
    return 0.5 * math.erfc(-x / (sigma * math.sqrt(2.0)))


def laplace_cdf(x: float, b: float) -> float:
    return 0.5 * math.exp(x / b) if x < 0 else 1.0 - 0.5 * math.exp(-x / b)


def rounded_pmf(cdf) -> np.ndarray:
    """P(clip(round(X), -127, 127) = v) for v = -127..127 (index v + 127)."""
    c = [cdf(v + 0.5) for v in range(-127, 127)]  # P(X < v + 1/2), v = -127..126
    p = np.empty(255)
    prev = 0.0
    for i, ci in enumerate(c):
        p[i] = ci - prev
        prev = ci
    p[254] = 1.0 - prev
    return p


def thresholds(cdf) -> np.ndarray:
    """256 uint64 thresholds for synth.c: entry k (k < 254) is
    floor(2^64 * P(code <= k - 127)); entries 254, 255 are 2^64 - 1."""
    t = np.full(256, MASK64, np.uint64)
    for k, v in enumerate(range(-127, 127)):
        q = cdf(v + 0.5)
        t[k] = min(MASK64, int(q * 2.0 ** 64)) if q > 0 else 0
    return t


def int8_codes(cdf, n: int, stream_key: int, nthreads: int | None = None) -> np.ndarray:
    thr = thresholds(cdf)
    out = np.empty(n, np.int8)
    if n:
        _L().syn_codes_int8(stream_key, thr.ctypes.data, n, out.ctypes.data,
                            nthreads or default_threads())
    return out


def normal_f32(sigma: float, n: int, stream_key: int, nthreads: int | None = None) -> np.ndarray:
    out = np.empty(n, np.float32)
    if n:
        _L().syn_normal_f32(stream_key, float(sigma), n, out.ctypes.data,
                            nthreads or default_threads())
    return out


def uniform_f32(lo: float, hi: float, n: int, stream_key: int,
                nthreads: int | None = None) -> np.ndarray:
    out = np.empty(n, np.float32)
    if n:
        _L().syn_uniform_f32(stream_key, float(lo), float(hi), n, out.ctypes.data,
                             nthreads or default_threads())
    return out


def uniform_scalar(lo: float, hi: float, stream_key: int) -> float:
    u = int(_L().syn_draw(stream_key, 0))
    return lo + (hi - lo) * ((u >> 11) * (1.0 / 9007199254740992.0))


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

KIND_INT8, KIND_E4M3, KIND_BF16EXP = 0, 1, 2

LLAMA2_13B_BLOCK = [("q", 5120, 5120), ("k", 5120, 5120), ("v", 5120, 5120),
                    ("o", 5120, 5120), ("gate", 13824, 5120), ("up", 13824, 5120),
                    ("down", 5120, 13824)]
LLAMA2_70B_LAYER = [("q", 8192, 8192), ("k", 1024, 8192), ("v", 1024, 8192),
                    ("o", 8192, 8192), ("gate", 28672, 8192), ("up", 28672, 8192),
                    ("down", 8192, 28672)]
LLAMA2_70B_LAYERS = 80

# workload ids (first element of every stream key)
W_TINY_LAPLACE, W_E4M3, W_13B_BLOCK, W_BF16_SPLIT, W_70B, W_70B_HEAD, W_BANDED = 1, 2, 3, 4, 5, 6, 7
LLAMA2_70B_VOCAB = 32000


def _scales(wid, layer, t, rows):
    return uniform_f32(1e-3, 1e-2, rows, key(wid, layer, t, 1))


def tiny_int8_laplace(rows: int = 256, cols: int = 256, b: float = 2.0):
    """Int8 codes round(Laplace(0, b)) clipped, one tensor; 4,096-symbol
    chunks."""
    codes = int8_codes(lambda x: laplace_cdf(x, b), rows * cols, key(W_TINY_LAPLACE, 0, 0, 0))
    return [dict(name="w", kind=KIND_INT8, rows=rows, cols=cols, chunk_symbols=4096,
                 symbols=codes.view(np.uint8), scales=_scales(W_TINY_LAPLACE, 0, 0, rows),
                 dist=("laplace", b))]


def e4m3_matrix(rows: int = 4096, cols: int = 4096, sigma: float = 0.02):
    """Float8 e4m3 codes of N(0, sigma) weights with per-row absmax/448
    scales; 65,536-symbol chunks."""
    import torch
    w = normal_f32(sigma, rows * cols, key(W_E4M3, 0, 0, 0)).reshape(rows, cols)
    absmax = np.abs(w).max(axis=1)
    scale = (absmax / np.float32(448.0)).astype(np.float32)
    q = (w / scale[:, None]).astype(np.float32)
    assert np.abs(q).max() < 464.0  # saturating and NaN-on-overflow casts agree here
    codes = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy().ravel()
    return [dict(name="w", kind=KIND_E4M3, rows=rows, cols=cols, chunk_symbols=65536,
                 symbols=codes.copy(), scales=scale, dist=("e4m3-normal", sigma))]


def llama2_13b_block(sigma: float = 1.0, shapes=None):
    """Int8 codes round(N(0, sigma)) clipped for the seven linears of one
    LLaMA-2-13B block, each with its own table; 65,536-symbol chunks."""
    out = []
    for t, (name, r, c) in enumerate(shapes or LLAMA2_13B_BLOCK):
        codes = int8_codes(lambda x: normal_cdf(x, sigma), r * c, key(W_13B_BLOCK, 0, t, 0))
        out.append(dict(name=name, kind=KIND_INT8, rows=r, cols=c, chunk_symbols=65536,
                        symbols=codes.view(np.uint8), scales=_scales(W_13B_BLOCK, 0, t, r),
                        dist=("normal", sigma)))
    return out


def bf16_weights(rows: int = 8192, cols: int = 8192, sigma: float = 0.02):
    """BF16 weights N(0, sigma) (RNE from fp32) as uint16 bit patterns;
    8,192-symbol chunks (one row of the 8192 x 8192 matrix) for the
    exponent stream."""
    import torch
    w = normal_f32(sigma, rows * cols, key(W_BF16_SPLIT, 0, 0, 0))
    bits = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return [dict(name="w", kind=KIND_BF16EXP, rows=rows, cols=cols, chunk_symbols=8192,
                 bf16=bits.copy(), dist=("bf16-normal", sigma))]


def llama2_70b_sigma(layer: int, t: int) -> float:
    return uniform_scalar(0.8, 3.0, key(W_70B, layer, t, 2))


def llama2_70b_layer(layer: int, shapes=None, nthreads: int | None = None):
    """Int8 codes for one LLaMA-2-70B layer: per-(layer, tensor) sigma ~
    U[0.8, 3.0] code units, round(N(0, sigma)) clipped; per-row scales;
    65,536-symbol chunks."""
    out = []
    for t, (name, r, c) in enumerate(shapes or LLAMA2_70B_LAYER):
        sigma = llama2_70b_sigma(layer, t)
        codes = int8_codes(lambda x, s=sigma: normal_cdf(x, s), r * c,
                           key(W_70B, layer, t, 0), nthreads)
        out.append(dict(name=name, kind=KIND_INT8, rows=r, cols=c, chunk_symbols=65536,
                        symbols=codes.view(np.uint8), scales=_scales(W_70B, layer, t, r),
                        dist=("normal", sigma)))
    return out


def llama2_70b_lm_head(nthreads: int | None = None, chunk_symbols: int = 65536):
    """Int8 codes for the LLaMA-2-70B output projection (vocabulary 32,000 x
    hidden 8,192), a tensor compressed on its own: sigma ~ U[0.8, 3.0] code
    units as for the layers, round(N(0, sigma)) clipped; per-row scales."""
    r, c = LLAMA2_70B_VOCAB, 8192
    sigma = uniform_scalar(0.8, 3.0, key(W_70B_HEAD, 0, 0, 2))
    codes = int8_codes(lambda x, s=sigma: normal_cdf(x, s), r * c, key(W_70B_HEAD, 0, 0, 0),
                       nthreads)
    return [dict(name="lm_head", kind=KIND_INT8, rows=r, cols=c, chunk_symbols=chunk_symbols,
                 symbols=codes.view(np.uint8), scales=_scales(W_70B_HEAD, 0, 0, r),
                 dist=("normal", sigma))]


def banded_int8_tensor(rows: int, cols: int, band_rows: int, seed: int, chunk_symbols: int,
                       lo: float = 0.3, hi: float = 4.0, nthreads: int | None = None):
    """Int8 codes whose spread changes along the tensor: every band of
    band_rows rows draws its own sigma ~ U[lo, hi] code units, round(N(0,
    sigma)) clipped. A tensor of this kind is what per-chunk tables are for
    (one table per tensor fits none of the bands)."""
    parts = []
    for b0 in range(0, rows, band_rows):
        r = min(band_rows, rows - b0)
        sigma = uniform_scalar(lo, hi, key(W_BANDED, seed, b0, 2))
        parts.append(int8_codes(lambda x, s=sigma: normal_cdf(x, s), r * cols,
                                key(W_BANDED, seed, b0, 0), nthreads))
    codes = np.concatenate(parts) if parts else np.zeros(0, np.int8)
    return dict(name=f"banded{seed}", kind=KIND_INT8, rows=rows, cols=cols,
                chunk_symbols=chunk_symbols, symbols=codes.view(np.uint8),
                scales=_scales(W_BANDED, seed, 0, rows), dist=("banded-normal", lo, hi, band_rows))


def random_int8_tensor(rows: int, cols: int, sigma: float, seed: int, chunk_symbols: int):
    """A small Int8 tensor for edge-case tests (any shape)."""
    codes = int8_codes(lambda x: normal_cdf(x, sigma), rows * cols, key(99, seed, 0, 0))
    return dict(name=f"r{seed}", kind=KIND_INT8, rows=rows, cols=cols,
                chunk_symbols=chunk_symbols, symbols=codes.view(np.uint8),
                scales=uniform_f32(1e-3, 1e-2, rows, key(99, seed, 0, 1)), dist=("normal", sigma))


def random_bytes(n: int, seed: int) -> np.ndarray:
    """Uniform random bytes (all 256 symbols), for table-stress tests."""
    out = np.empty(n, np.int8)
    thr = np.full(256, MASK64, np.uint64)
    # equal thresholds: code k - 127 for k in 0..254, close to uniform over 255 values
    for k in range(254):
        thr[k] = int((k + 1) * (2.0 ** 64) / 255.0)
    if n:
        _L().syn_codes_int8(key(98, seed, 0, 0), thr.ctypes.data, n, out.ctypes.data, 1)
    v = out.view(np.uint8).copy()
    # spread the 255 values over all 256 bytes: odd draws flip the top bit
    if n:
        flip = np.empty(n, np.float32)
        _L().syn_uniform_f32(key(98, seed, 1, 0), 0.0, 1.0, n, flip.ctypes.data, 1)
        v ^= np.where(flip < 0.5, 0x80, 0).astype(np.uint8)
    return v
