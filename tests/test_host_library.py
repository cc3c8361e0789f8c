"""CPU-only checks of libentq.so: it loads, exports every entry point that
include/entq.h declares, and its host-side encoder (offline compression)
agrees byte for byte with the oracle's. Plan validation errors are checked
with a dummy workspace address that the library never dereferences (every
case fails validation before any HIP call)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def E():
    import entropy_coded_weight_amd as E
    if not os.path.exists(E.LIB_PATH):
        from entropy_coded_weight_amd import build
        build.build()
    return E


def declared_functions():
    src = open(os.path.join(ROOT, "include", "entq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(entq_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function(E):
    names = declared_functions()
    assert "entq_plan" in names and "entq_decode" in names and "entq_decode_bf16_split" in names
    L = ctypes.CDLL(E.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert sorted(E.EXPORTED) == names


def test_status_strings(E):
    assert E.lib().entq_status_str(0) == b"ok"
    assert b"4096" in E.lib().entq_status_str(-2)


def test_build_freq_matches_oracle(E):
    rng = np.random.default_rng(0)
    for trial in range(400):
        k = int(rng.integers(0, 257))
        counts = np.zeros(256, np.uint64)
        if k:
            idx = rng.choice(256, size=k, replace=False)
            counts[idx] = np.maximum(1, rng.exponential(10 ** rng.uniform(0, 10), size=k)).astype(np.uint64)
        np.testing.assert_array_equal(E.build_freq(counts), oracle.quantize_freqs(counts))


def test_count_symbols_matches_oracle(E):
    sym = synth.random_bytes(1_000_003, 1)
    np.testing.assert_array_equal(E.count_symbols(sym, 4), oracle.count_symbols(sym))


@pytest.mark.parametrize("n,C", [(1, 64), (63, 4096), (4096, 4096), (4097, 4096),
                                 (100_000, 4096), (300_000, 65536), (65536 * 3 + 5, 65536)])
def test_encoder_matches_oracle_byte_for_byte(E, n, C):
    t = synth.random_int8_tensor(1, n, 2.0, n % 97, C)
    sym = t["symbols"]
    f = oracle.quantize_freqs(oracle.count_symbols(sym))
    blob_o, desc_o = oracle.encode_tensor(sym, C, f)
    blob_e, ch = E.encode_tensor(sym, C, f, tensor_id=3, base_offset=4096, n_threads=3)
    np.testing.assert_array_equal(blob_e, blob_o)
    assert np.all(ch["tensor"] == 3)
    np.testing.assert_array_equal(ch["n_symbols"], desc_o[:, 0])
    np.testing.assert_array_equal(ch["n_words"], desc_o[:, 1])
    np.testing.assert_array_equal(ch["byte_offset"], desc_o[:, 2] + 4096)
    np.testing.assert_array_equal(ch["elem_offset"], desc_o[:, 3])


def test_encoder_extreme_tables_match_oracle(E):
    rng = np.random.default_rng(3)
    for trial in range(30):
        sym = synth.random_bytes(int(rng.integers(1, 20000)), 100 + trial)
        if trial % 3 == 0:
            sym[:] = sym[0]  # one symbol
        f = oracle.quantize_freqs(oracle.count_symbols(sym))
        C = int(rng.choice([64, 128, 4096]))
        blob_o, desc_o = oracle.encode_tensor(sym, C, f)
        blob_e, ch = E.encode_tensor(sym, C, f, n_threads=int(rng.integers(1, 9)))
        np.testing.assert_array_equal(blob_e, blob_o)
        np.testing.assert_array_equal(ch["n_words"], desc_o[:, 1])


def test_encoder_rejects_symbol_without_frequency(E):
    f = np.zeros(256, np.uint16)
    f[1] = 4096
    with pytest.raises(E.EntqError):
        E.encode_tensor(np.array([1, 1, 2], np.uint8), 64, f)
    f[1] = 4095
    with pytest.raises(E.EntqError):
        E.encode_tensor(np.array([1, 1], np.uint8), 64, f)


def test_bf16_split_matches_oracle(E):
    w = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    e1, s1 = E.bf16_split(w, 2)
    e2, s2 = oracle.bf16_split(w)
    np.testing.assert_array_equal(e1, e2)
    np.testing.assert_array_equal(s1, s2)


@pytest.mark.parametrize("rows,cols,C", [(16, 16, 16), (32, 64, 32), (48, 768, 256),
                                         (64, 4096, 1024), (16, 28672, 4096)])
def test_tile_order_matches_oracle(E, rows, cols, C):
    rng = np.random.default_rng(rows * 7 + C)
    w = rng.integers(0, 256, rows * cols, dtype=np.uint8)
    np.testing.assert_array_equal(E.tile_order(w, rows, cols, C, n_threads=3),
                                  oracle.tile_order(w, rows, cols, C))


def test_tile_order_rejects_shapes_outside_the_layout(E):
    w = np.zeros(64 * 48, np.uint8)
    for rows, cols, C in ((24, 128, 64), (48, 64, 24), (48, 64, 48), (48, 64, 0)):
        with pytest.raises(E.EntqError):
            E.tile_order(w[:rows * cols], rows, cols, C)


def test_encode_batch_matches_oracle_container(E):
    specs = [synth.random_int8_tensor(64, 192, 1.5, s, 4096) for s in range(3)]
    b = E.encode_batch(specs, n_threads=2)
    c = oracle.encode_container(specs)
    np.testing.assert_array_equal(b.blob, c.blob)
    np.testing.assert_array_equal(b.chunks["tensor"], c.chunks[:, 0])
    np.testing.assert_array_equal(b.chunks["byte_offset"], c.chunks[:, 3])
    for t, td in enumerate(c.tensors):
        np.testing.assert_array_equal(b.freq[t], td["freq"])
        assert int(b.tensors[t]["out_elem_offset"]) == td["out_elem_offset"]


# ---- plan validation (fails before any HIP call) -------------------------

FAKE_WS = 1 << 20  # an aligned address that validation failures never touch


def _try_plan(E, tensors, freq, chunks, blob_bytes, ws_bytes=1 << 24, ws=FAKE_WS):
    h = ctypes.c_void_p()
    tensors = np.ascontiguousarray(tensors, E.TENSOR_DESC)
    chunks = np.ascontiguousarray(chunks, E.CHUNK_DESC)
    freq = np.ascontiguousarray(freq, np.uint16)
    st = E.lib().entq_plan(tensors.ctypes.data, tensors.size, freq.ctypes.data,
                           chunks.ctypes.data if chunks.size else None, chunks.size,
                           blob_bytes, ws, ws_bytes, None, ctypes.byref(h))
    assert not h.value
    return st


def _small_batch(E):
    specs = [synth.random_int8_tensor(8, 640, 1.5, 7, 1024)]
    return E.encode_batch(specs, n_threads=1)


def test_plan_rejects_bad_inputs(E):
    b = _small_batch(E)
    assert b.chunks.size == 5
    bb = b.blob.size
    # bad table sum
    f = b.freq.copy()
    f[0, np.nonzero(f[0])[0][0]] += 1
    assert _try_plan(E, b.tensors, f, b.chunks, bb) == -2
    # a hole in the tiling
    assert _try_plan(E, b.tensors, b.freq, b.chunks[:-1], bb) == -3
    # a duplicate
    ch = b.chunks.copy()
    ch[1] = ch[0]
    assert _try_plan(E, b.tensors, b.freq, ch, bb) == -3
    # misaligned region
    ch = b.chunks.copy()
    ch[2]["byte_offset"] += 8
    assert _try_plan(E, b.tensors, b.freq, ch, bb) == -4
    # region past the blob
    assert _try_plan(E, b.tensors, b.freq, b.chunks, bb - 16) == -3
    # more words than symbols
    ch = b.chunks.copy()
    ch[0]["n_words"] = ch[0]["n_symbols"] + 1
    assert _try_plan(E, b.tensors, b.freq, ch, bb) == -3
    # wrong chunk length
    ch = b.chunks.copy()
    ch[4]["n_symbols"] -= 1
    assert _try_plan(E, b.tensors, b.freq, ch, bb) == -3
    # chunk size not a multiple of 64
    t = b.tensors.copy()
    t[0]["chunk_symbols"] = 1000
    assert _try_plan(E, t, b.freq, b.chunks, bb) == -1
    # rows * cols != n_symbols
    t = b.tensors.copy()
    t[0]["rows"] = 9
    assert _try_plan(E, t, b.freq, b.chunks, bb) == -1
    # unknown kind
    t = b.tensors.copy()
    t[0]["kind"] = 7
    assert _try_plan(E, t, b.freq, b.chunks, bb) == -1
    # unknown flag bits
    t = b.tensors.copy()
    t[0]["kind"] = E.KIND_INT8 | 0x200
    assert _try_plan(E, t, b.freq, b.chunks, bb) == -1
    # workspace too small
    assert _try_plan(E, b.tensors, b.freq, b.chunks, bb, ws_bytes=1000) == -5
    # misaligned workspace
    assert _try_plan(E, b.tensors, b.freq, b.chunks, bb, ws=FAKE_WS + 64) == -4


def test_plan_checks_the_tile_layout(E):
    """A tensor marked ENTQ_LAYOUT_TILES needs rows in 16-row bands, whole
    16 x 16 tiles per chunk and a chunk width dividing the columns (exponent
    streams take it too)."""
    def tiled(rows, cols, C, kind=E.KIND_INT8, seed=11):
        sp = synth.random_int8_tensor(rows, cols, 1.5, seed, 16 * C)
        sp["kind"] = kind | E.LAYOUT_TILES
        return E.encode_batch([sp], n_threads=1)
    b = tiled(32, 512, 256)   # accepted shape: validation passes up to the workspace
    assert _try_plan(E, b.tensors, b.freq, b.chunks, b.blob.size, ws_bytes=1000) == -5
    for rows, cols, C in ((24, 512, 256), (32, 512, 192), (32, 768, 512)):
        b = tiled(rows, cols, C)
        assert _try_plan(E, b.tensors, b.freq, b.chunks, b.blob.size) == -1, (rows, cols, C)
    b = tiled(32, 512, 256)
    t = b.tensors.copy()
    t[0]["kind"] = E.KIND_BF16EXP | E.LAYOUT_TILES
    assert _try_plan(E, t, b.freq, b.chunks, b.blob.size, ws_bytes=1000) == -5


def test_plan_rejects_overlapping_outputs(E):
    specs = [synth.random_int8_tensor(8, 640, 1.5, s, 1024) for s in range(2)]
    b = E.encode_batch(specs, n_threads=1)
    t = b.tensors.copy()
    t[1]["out_elem_offset"] = 100
    assert _try_plan(E, t, b.freq, b.chunks, b.blob.size) == -1


def test_workspace_bytes_grows_with_inputs(E):
    a = E.lib().entq_plan_workspace_bytes(1, 10)
    b = E.lib().entq_plan_workspace_bytes(7, 13056)
    assert 0 < a < b
    assert b >= 7 * 4096 * 8 + 13056 * 48


def test_missing_library_fails_loudly():
    """No CPU fallback: without the built library every call raises."""
    import subprocess
    import sys
    code = ("import entropy_coded_weight_amd as E\n"
            "E.LIB_PATH = '/nonexistent/libentq.so'\n"
            "E._lib = None\n"
            "try:\n"
            "    E.build_freq(__import__('numpy').ones(256, 'uint64'))\n"
            "except ImportError as e:\n"
            "    print('raised', e)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0 and "raised" in r.stdout and "no CPU fallback" in r.stdout


def test_device_calls_validate_before_launching(E):
    """Argument checks of the device-encoder and fused-product entry points
    return their codes before any HIP call (fake device addresses)."""
    L = E.lib()
    fake = 1 << 20                                   # 256-byte aligned, never touched
    # per-chunk counts: chunk size not a multiple of 64, then a misaligned array
    job = np.zeros(1, E.CHUNK_COUNT_JOB)
    job[0] = (fake, 4096, 100, 0, fake)
    assert L.entq_count_chunks_device_batch(job.ctypes.data, 1, None) == -1
    job[0] = (fake + 8, 4096, 64, 0, fake)
    assert L.entq_count_chunks_device_batch(job.ctypes.data, 1, None) == -4
    assert L.entq_count_chunks_device_batch(None, -1, None) == -1
    # device tables: only 4- and 8-byte counts
    assert L.entq_build_freq_device(fake, 3, 1, fake, None) == -1
    assert L.entq_build_freq_device(fake + 4, 8, 1, fake, None) == -4
    assert L.entq_build_freq_device(None, 4, 0, None, None) == 0  # nothing to do
    # per-chunk encode: missing tables, then a too-small scratch
    enc = np.zeros(1, E.ENCODE_JOB)
    enc[0] = (fake, 8192, 4096, 0, 0, fake, 1 << 30, fake)
    assert L.entq_encode_device_adaptive_batch(enc.ctypes.data, 1, None) == -1
    enc[0] = (fake, 8192, 4096, 0, fake, fake, 16, fake)
    assert L.entq_encode_device_adaptive_batch(enc.ctypes.data, 1, None) == -5
    # regions headed by tables: misaligned offsets, misaligned tables
    assert L.entq_region_offsets_device_adaptive(fake, 4, 8, fake, fake, None) == -4
    pack = np.zeros(1, E.PACK_ADAPTIVE_JOB)
    pack[0] = (fake, 8192, 4096, 0, fake, fake, fake + 2)
    assert L.entq_pack_device_adaptive_batch(pack.ctypes.data, 1, fake, None) == -4
    pack[0] = (fake, 8192, 4096, 0, fake, fake, 0)
    assert L.entq_pack_device_adaptive_batch(pack.ctypes.data, 1, fake, None) == -1
    # fused product: workspace size of no plan
    assert L.entq_decode_gemm_workspace_bytes(None, 16) == 0
    assert L.entq_decode_gemm_tiles_workspace_bytes(None, 16) == 0
    assert L.entq_decode_gemm_tiles(None, fake, fake, fake, 16, None, 0, None, None) == -1
