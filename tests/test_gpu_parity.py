"""GPU parity: the HIP decoder (through the C ABI) against the CPU oracle,
element by element, on the same seeded inputs.

Containers fed to the GPU are written by the oracle's encoder (for the
largest workload, by the library's encoder, which the CPU suite proves
byte-identical to the oracle's, and the expected values are then the
oracle's dequantisation of the source codes). The bar is bit-exact for every
output byte and bf16 word: all arithmetic is integer except the dequant,
which is defined as one fp32 product rounded to nearest even, then rounded
to bf16."""
import os
import sys

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-parity] {msg}", flush=True)


@pytest.fixture(scope="module")
def E():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import entropy_coded_weight_amd as E
    E.lib()  # loud failure if libentq.so is missing
    return E


def plan_from_container(E, c: oracle.Container, order=None):
    import torch
    tens = np.zeros(len(c.tensors), E.TENSOR_DESC)
    freq = np.zeros((len(c.tensors), 256), np.uint16)
    for t, td in enumerate(c.tensors):
        tens[t] = (td["kind"], td["rows"], td["cols"], td["chunk_symbols"], td["n_symbols"],
                   td["out_elem_offset"], td["scale_row_offset"])
        freq[t] = td["freq"]
    ch = np.zeros(c.n_chunks, E.CHUNK_DESC)
    if c.n_chunks:
        ch["tensor"] = c.chunks[:, 0]
        ch["n_symbols"] = c.chunks[:, 1]
        ch["n_words"] = c.chunks[:, 2]
        ch["byte_offset"] = c.chunks[:, 3]
        ch["elem_offset"] = c.chunks[:, 4]
    if order is not None:
        ch = ch[order]
    blob = torch.from_numpy(c.blob if c.blob.size else np.zeros(16, np.uint8)).cuda()
    p = E.plan(tens, freq, ch, c.blob.size)
    return p, blob


def gpu_decode(E, c, out_kind, scales=None, order=None, split_sm=None):
    import torch
    p, blob = plan_from_container(E, c, order)
    total = max([t["out_elem_offset"] + t["n_symbols"] for t in c.tensors] + [1])
    status = torch.full((max(c.n_chunks, 1),), -7, dtype=torch.int32, device="cuda")
    if split_sm is not None:
        out = torch.zeros(total, dtype=torch.int16, device="cuda")
        sm = torch.from_numpy(split_sm).cuda()
        E.decode_bf16_split(p, blob, sm, out, status)
    elif out_kind == E.OUT_CODES:
        out = torch.zeros(total, dtype=torch.uint8, device="cuda")
        E.decode(p, blob, out, E.OUT_CODES, None, status)
    else:
        out = torch.zeros(total, dtype=torch.int16, device="cuda")
        sc = torch.from_numpy(np.ascontiguousarray(scales, np.float32)).cuda()
        E.decode(p, blob, out, E.OUT_BF16, sc, status)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    st = status.cpu().numpy()[:c.n_chunks]
    if order is not None:
        # status is indexed by position in the chunk index the plan was given
        st_c = np.empty_like(st)
        st_c[order] = st
        st = st_c
    p.close()
    return (o.view(np.uint16) if o.dtype == np.int16 else o), st


def expected_codes(c):
    syms, st = oracle.decode_container_symbols(c)
    total = max([t["out_elem_offset"] + t["n_symbols"] for t in c.tensors] + [1])
    out = np.zeros(total, np.uint8)
    for td, s in zip(c.tensors, syms):
        out[td["out_elem_offset"]:td["out_elem_offset"] + td["n_symbols"]] = s
    return out, st


def all_scales(specs):
    return np.concatenate([np.asarray(s["scales"], np.float32) for s in specs])


def check_codes_and_bf16(E, specs, order=None):
    c = oracle.encode_container(specs)
    want_codes, st = expected_codes(c)
    assert np.all(st == 0)
    got, gst = gpu_decode(E, c, E.OUT_CODES, order=order)
    np.testing.assert_array_equal(got, want_codes)
    np.testing.assert_array_equal(gst, st)
    scales = all_scales(specs)
    want_bf16, _ = oracle.decode_container_bf16(c, scales)
    got, gst = gpu_decode(E, c, E.OUT_BF16, scales=scales, order=order)
    np.testing.assert_array_equal(got, want_bf16)
    np.testing.assert_array_equal(gst, st)


# ---------------------------------------------------------------- workloads

def test_tiny_int8_laplace_256x256(E):
    _say("tiny int8 laplace 256x256, C=4096")
    check_codes_and_bf16(E, synth.tiny_int8_laplace())


def test_e4m3_4096x4096(E):
    _say("e4m3 4096x4096, C=65536")
    check_codes_and_bf16(E, synth.e4m3_matrix())


def test_llama2_13b_block_bf16(E):
    _say("llama2-13b block, 7 tensors, bf16")
    specs = synth.llama2_13b_block()
    c = oracle.encode_container(specs)
    scales = all_scales(specs)
    want, st = oracle.decode_container_bf16(c, scales)
    assert np.all(st == 0)
    got, gst = gpu_decode(E, c, E.OUT_BF16, scales=scales)
    np.testing.assert_array_equal(gst, st)
    np.testing.assert_array_equal(got, want)
    want_codes, st = expected_codes(c)
    got, gst = gpu_decode(E, c, E.OUT_CODES)
    np.testing.assert_array_equal(gst, st)
    np.testing.assert_array_equal(got, want_codes)


@pytest.mark.parametrize("C", [8192, 65536])
def test_bf16_exponent_split_8192x8192(E, C):
    _say(f"bf16 exponent split 8192x8192, {C}-symbol chunks")
    w = synth.bf16_weights()[0]
    e, sm = oracle.bf16_split(w["bf16"])
    spec = dict(kind=oracle.KIND_BF16EXP, rows=w["rows"], cols=w["cols"], symbols=e,
                chunk_symbols=C)
    c = oracle.encode_container([spec])
    got, gst = gpu_decode(E, c, None, split_sm=sm)
    assert np.all(gst == 0)
    np.testing.assert_array_equal(got, w["bf16"])


def test_llama2_70b_layer0_full(E):
    """One full 70B-shaped layer (855.6 M symbols, 13,056 chunks) in the
    launch configuration the benchmark times: one decode of the whole layer
    into one bf16 buffer."""
    _say("llama2-70b layer 0, full, oracle-encoded")
    specs = synth.llama2_70b_layer(0)
    c = oracle.encode_container(specs)
    scales = all_scales(specs)
    want, st = oracle.decode_container_bf16(c, scales)
    assert np.all(st == 0)
    got, gst = gpu_decode(E, c, E.OUT_BF16, scales=scales)
    assert np.all(gst == 0)
    np.testing.assert_array_equal(got, want)
    del got, want
    # codes output of the same container: the source codes (the oracle decode of this
    # container, inside decode_container_bf16, returned every chunk with status 0)
    _say("llama2-70b layer 0, codes")
    got, gst = gpu_decode(E, c, E.OUT_CODES)
    assert np.all(gst == 0)
    np.testing.assert_array_equal(got, np.concatenate([np.asarray(s["symbols"], np.uint8)
                                                       for s in specs]))


def test_llama2_70b_last_layer_against_source(E):
    """Layer 79, encoded by the library's encoder (byte-identical to the
    oracle's on the CPU suite); expected = the oracle's dequantisation of the
    generated source codes."""
    import torch
    _say("llama2-70b layer 79, library-encoded, vs oracle dequant of source")
    specs = synth.llama2_70b_layer(79)
    b = E.encode_batch(specs)
    p = E.plan(b.tensors, b.freq, b.chunks, b.blob.size)
    blob = torch.from_numpy(b.blob).cuda()
    sc = torch.from_numpy(all_scales(specs)).cuda()
    out = torch.empty(b.out_elems, dtype=torch.int16, device="cuda")
    st = torch.full((b.chunks.size,), -7, dtype=torch.int32, device="cuda")
    E.decode(p, blob, out, E.OUT_BF16, sc, st)
    torch.cuda.synchronize()
    assert int((st != 0).sum()) == 0
    got = out.cpu().numpy().view(np.uint16)
    for t, sp in enumerate(specs):
        o = int(b.tensors[t]["out_elem_offset"])
        n = sp["rows"] * sp["cols"]
        want = oracle.dequant_tensor(sp["symbols"], sp["rows"], sp["cols"], sp["kind"], sp["scales"])
        np.testing.assert_array_equal(got[o:o + n], want, err_msg=sp["name"])
    p.close()


# --------------------------------------------------------------- edge cases

def test_ragged_shapes_and_odd_columns(E):
    _say("ragged shapes")
    specs = [
        synth.random_int8_tensor(1, 1, 1.0, 1, 64),          # one symbol
        synth.random_int8_tensor(1, 63, 1.0, 2, 64),         # one partial step
        synth.random_int8_tensor(3, 65, 2.0, 3, 128),        # cols not a multiple of 64
        synth.random_int8_tensor(7, 13, 0.7, 4, 64),         # cols < 64
        synth.random_int8_tensor(17, 4099, 3.0, 5, 4096),    # ragged chunks and steps
        synth.random_int8_tensor(2, 100003, 1.3, 6, 65536),  # long rows, ragged tail
        synth.random_int8_tensor(40, 2048, 1.0, 7, 1 << 20), # chunk of 2^20 (one chunk)
    ]
    check_codes_and_bf16(E, specs)


def test_shuffled_chunk_index_and_status_positions(E):
    _say("shuffled chunk index")
    specs = [synth.random_int8_tensor(64, 1000, 1.5, s, 1024) for s in range(3)]
    c = oracle.encode_container(specs)
    order = np.random.default_rng(0).permutation(c.n_chunks)
    check_codes_and_bf16(E, specs, order=order)


def test_one_symbol_and_all_symbol_tensors(E):
    _say("one-symbol and 256-symbol tables")
    const = dict(name="c", kind=oracle.KIND_INT8, rows=33, cols=64, chunk_symbols=256,
                 symbols=np.full(33 * 64, 0xF3, np.uint8),
                 scales=synth.uniform_f32(1e-3, 1e-2, 33, synth.key(97, 1, 0, 1)))
    allb = dict(name="a", kind=oracle.KIND_INT8, rows=64, cols=1024, chunk_symbols=4096,
                symbols=synth.random_bytes(64 * 1024, 3),
                scales=synth.uniform_f32(-1.0, 1.0, 64, synth.key(97, 2, 0, 1)))
    check_codes_and_bf16(E, [const, allb])


def test_e4m3_every_code_including_nan(E):
    _say("e4m3 all 256 codes incl. NaN")
    sym = synth.random_bytes(128 * 512, 11)
    sym[:256] = np.arange(256, dtype=np.uint8)
    sc = synth.uniform_f32(1e-3, 4.0, 128, synth.key(97, 3, 0, 1))
    sc[:3] = np.array([1.0, -1.0, 3.0e38], np.float32)
    spec = dict(name="e", kind=oracle.KIND_E4M3, rows=128, cols=512, chunk_symbols=8192,
                symbols=sym, scales=sc)
    check_codes_and_bf16(E, [spec])


def test_mixed_kinds_and_empty_tensor_in_one_batch(E):
    _say("mixed kinds + empty tensor")
    e4 = synth.e4m3_matrix(256, 320)[0]
    specs = [synth.random_int8_tensor(30, 700, 2.0, 8, 2048), e4,
             dict(name="z", kind=oracle.KIND_INT8, rows=0, cols=64, chunk_symbols=64,
                  symbols=np.zeros(0, np.uint8), scales=np.zeros(0, np.float32)),
             synth.random_int8_tensor(5, 64, 1.0, 9, 64)]
    check_codes_and_bf16(E, specs)


def test_gaps_in_output_and_scale_layout(E):
    """Tensors placed at arbitrary output and scale offsets (with gaps) land
    exactly there and nothing else is written."""
    import torch
    _say("output/scale gaps")
    specs = [synth.random_int8_tensor(9, 320, 1.5, 12 + s, 1024) for s in range(2)]
    b = E.encode_batch(specs, n_threads=2)
    t = b.tensors.copy()
    t[0]["out_elem_offset"], t[1]["out_elem_offset"] = 5000, 64
    t[0]["scale_row_offset"], t[1]["scale_row_offset"] = 20, 3
    p = E.plan(t, b.freq, b.chunks, b.blob.size)
    scales = np.zeros(40, np.float32)
    scales[20:29] = specs[0]["scales"]
    scales[3:12] = specs[1]["scales"]
    out = torch.full((5000 + 2880 + 64,), 0x5A5A, dtype=torch.int16, device="cuda")
    E.decode(p, torch.from_numpy(b.blob).cuda(), out, E.OUT_BF16, torch.from_numpy(scales).cuda())
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    w0 = oracle.dequant_tensor(specs[0]["symbols"], 9, 320, 0, specs[0]["scales"])
    w1 = oracle.dequant_tensor(specs[1]["symbols"], 9, 320, 0, specs[1]["scales"])
    np.testing.assert_array_equal(got[5000:5000 + 2880], w0)
    np.testing.assert_array_equal(got[64:64 + 2880], w1)
    untouched = np.ones(got.size, bool)
    untouched[5000:5000 + 2880] = False
    untouched[64:64 + 2880] = False
    assert np.all(got[untouched] == 0x5A5A)
    p.close()


def _far_plan(E, c, byte_shift, elem_shift, row_shift, adaptive=False):
    """A plan of container c with every chunk region moved byte_shift bytes
    into the blob, every tensor's output elem_shift elements on and its
    scale rows row_shift rows on."""
    tens = np.zeros(len(c.tensors), E.TENSOR_DESC)
    freq = None if adaptive else np.zeros((len(c.tensors), 256), np.uint16)
    for t, td in enumerate(c.tensors):
        tens[t] = (td["kind"], td["rows"], td["cols"], td["chunk_symbols"], td["n_symbols"],
                   td["out_elem_offset"] + elem_shift, td["scale_row_offset"] + row_shift)
        if not adaptive:
            freq[t] = td["freq"]
    ch = np.zeros(c.n_chunks, E.CHUNK_DESC)
    ch["tensor"], ch["n_symbols"], ch["n_words"] = c.chunks[:, 0], c.chunks[:, 1], c.chunks[:, 2]
    ch["byte_offset"] = c.chunks[:, 3] + np.uint64(byte_shift)
    ch["elem_offset"] = c.chunks[:, 4]
    return E.plan(tens, freq, ch, byte_shift + c.blob.size)


def _far_blob(c, byte_shift):
    import torch
    blob = torch.empty(byte_shift + c.blob.size, dtype=torch.uint8, device="cuda")
    blob[byte_shift:] = torch.from_numpy(c.blob).cuda()
    return blob


def _check_far_output(out, shift, want, fill):
    """out[shift:] equals want; nothing before it was written (checked on
    the device, without copying gigabytes back)."""
    import torch
    torch.cuda.synchronize()
    assert not bool((out[:shift] != fill).any()), "a write landed before the tensor's offset"
    got = out[shift:].cpu().numpy()
    np.testing.assert_array_equal(got.view(want.dtype), want)


def test_offsets_past_4_gib(E):
    """Chunk regions more than 4 GiB into the blob, outputs more than 4 GiB
    into the output buffer (codes, bf16 and exponent-split outputs) and scale
    rows far into the scale array land exactly where the chunk index and the
    tensor table put them, for the streaming, element-wise and per-chunk-table
    kernels: every offset and address is 64-bit."""
    import torch
    G = 1 << 32
    specs = [synth.random_int8_tensor(16, 1024, 2.0, 41, 4096),   # streaming kernel
             dict(synth.e4m3_matrix(24, 512)[0], chunk_symbols=4096),
             synth.random_int8_tensor(7, 333, 1.5, 42, 960)]      # element-wise kernel
    row_shift = (1 << 22) + 5
    for adaptive in (False, True):
        # per-chunk tables take rows of whole 256-symbol blocks only
        sp = specs[:2] if adaptive else specs
        scales = all_scales(sp)
        far_scales = torch.zeros(row_shift + scales.size, dtype=torch.float32, device="cuda")
        far_scales[row_shift:] = torch.from_numpy(scales).cuda()
        c = oracle.encode_container_adaptive(sp) if adaptive else oracle.encode_container(sp)
        if adaptive:
            syms, st = oracle.decode_container_adaptive_symbols(c)
            want_codes = np.concatenate(syms)
            want_bf16, _ = oracle.decode_container_adaptive_bf16(c, scales)
        else:
            want_codes, st = expected_codes(c)
            want_bf16, _ = oracle.decode_container_bf16(c, scales)
        assert np.all(st == 0)
        total = want_codes.size
        blob = _far_blob(c, G + 4096)
        # codes: byte offsets past 4 GiB
        shift = G + 48
        _say(f"offsets past 4 GiB ({'per-chunk' if adaptive else 'shared'} tables): codes")
        p = _far_plan(E, c, G + 4096, shift, 0, adaptive)
        status = torch.full((c.n_chunks,), -7, dtype=torch.int32, device="cuda")
        out = torch.full((shift + total,), 0x5A, dtype=torch.uint8, device="cuda")
        E.decode(p, blob, out, E.OUT_CODES, None, status)
        _check_far_output(out, shift, want_codes, 0x5A)
        assert np.all(status.cpu().numpy() == 0)
        p.close()
        del out
        # bf16: element offsets past 2^31 (bytes past 4 GiB), scale rows past 4 M
        shift = (G >> 1) + 16
        _say(f"offsets past 4 GiB ({'per-chunk' if adaptive else 'shared'} tables): bf16")
        p = _far_plan(E, c, G + 4096, shift, row_shift, adaptive)
        out = torch.full((shift + total,), 0x5A5A, dtype=torch.int16, device="cuda")
        E.decode(p, blob, out, E.OUT_BF16, far_scales, status)
        _check_far_output(out, shift, want_bf16, 0x5A5A)
        assert np.all(status.cpu().numpy() == 0)
        p.close()
        del out, blob
        torch.cuda.empty_cache()
    # exponent streams: output and sign/mantissa bytes past 2^31 elements
    w = synth.bf16_weights(3, 70_000, sigma=0.5)[0]["bf16"]
    e, sm = oracle.bf16_split(w)
    for C in (4096, 960):
        _say(f"offsets past 4 GiB: exponent stream, C{C}")
        c = oracle.encode_container([dict(kind=oracle.KIND_BF16EXP, rows=3, cols=70_000,
                                          symbols=e, chunk_symbols=C)])
        blob = _far_blob(c, G + 4096)
        shift = (G >> 1) + 16
        p = _far_plan(E, c, G + 4096, shift, 0)
        far_sm = torch.zeros(shift + sm.size, dtype=torch.uint8, device="cuda")
        far_sm[shift:] = torch.from_numpy(sm).cuda()
        status = torch.full((c.n_chunks,), -7, dtype=torch.int32, device="cuda")
        out = torch.full((shift + w.size,), 0x5A5A, dtype=torch.int16, device="cuda")
        E.decode_bf16_split(p, blob, far_sm, out, status)
        _check_far_output(out, shift, w, 0x5A5A)
        assert np.all(status.cpu().numpy() == 0)
        p.close()
        del out, blob, far_sm
        torch.cuda.empty_cache()


def test_corrupt_streams_report_the_oracles_status(E):
    _say("corruption statuses")
    specs = [synth.random_int8_tensor(16, 4096, 2.0, 20, 4096)]
    c = oracle.encode_container(specs)
    rng = np.random.default_rng(5)
    blob = c.blob.copy()
    chunks = c.chunks.copy()
    # chunk 0: flip a word bit; chunk 1: drop the last word from the count;
    # chunk 2: flip a state bit; chunk 3: claim one word more than coded
    # (the padding word); others intact
    off0, nw0 = int(chunks[0, 3]), int(chunks[0, 2])
    blob[off0 + 256 + 2 * int(rng.integers(0, nw0))] ^= 0x10
    chunks[1, 2] -= 1
    blob[int(chunks[2, 3]) + 4 * 7] ^= 0x01
    if (256 + 2 * int(chunks[3, 2])) % 16:
        chunks[3, 2] += 1
    bad = oracle.Container(blob, c.tensors, chunks)
    _, want_st = oracle.decode_container_symbols(bad)
    assert want_st[0] != 0 and want_st[1] == 2 and want_st[4:].max() == 0
    _, gst = gpu_decode(E, bad, E.OUT_CODES)
    np.testing.assert_array_equal(gst, want_st)


def test_repeat_runs_are_identical(E):
    _say("determinism")
    specs = synth.llama2_13b_block(shapes=[("k", 1024, 5120), ("d", 512, 13824)])
    c = oracle.encode_container(specs)
    scales = all_scales(specs)
    a, _ = gpu_decode(E, c, E.OUT_BF16, scales=scales)
    b, _ = gpu_decode(E, c, E.OUT_BF16, scales=scales)
    np.testing.assert_array_equal(a, b)


def test_stream_kernel_high_entropy_ring_wraps(E):
    """All 256 byte values, near-uniform: ~8 bits/symbol, so a wave's word
    ring wraps every ~64 steps and the mirror tail is used constantly; chunk
    sizes 512 .. 2^20 with ragged tails, output offsets 16-aligned so every
    tensor takes the streaming kernel."""
    _say("high-entropy streaming path")
    specs = []
    for i, (rows, cols, C) in enumerate([(4, 512, 512), (3, 1024, 1024), (7, 4096, 8192),
                                         (2, 1 << 19, 1 << 20), (1, 700_000, 65536),
                                         (5, 512 * 37, 4096)]):
        sym = synth.random_bytes(rows * cols, 40 + i)
        specs.append(dict(name=f"u{i}", kind=oracle.KIND_INT8, rows=rows, cols=cols,
                          chunk_symbols=C, symbols=sym,
                          scales=synth.uniform_f32(1e-3, 1e-2, rows, synth.key(97, 40 + i, 0, 1))))
    c = oracle.encode_container(specs)
    assert all(t["out_elem_offset"] % 16 == 0 for t in c.tensors)
    want_codes, st = expected_codes(c)
    got, gst = gpu_decode(E, c, E.OUT_CODES)
    np.testing.assert_array_equal(gst, st)
    np.testing.assert_array_equal(got, want_codes)
    scales = all_scales(specs)
    want, _ = oracle.decode_container_bf16(c, scales)
    got, gst = gpu_decode(E, c, E.OUT_BF16, scales=scales)
    np.testing.assert_array_equal(got, want)


def test_split_stream_ragged_and_high_entropy(E):
    """bf16 split on the streaming path with partial blocks and a random
    (high-entropy) exponent stream."""
    _say("split streaming ragged")
    rng = np.random.default_rng(3)
    words = rng.integers(0, 1 << 16, size=3 * 70_001 + 5, dtype=np.uint64).astype(np.uint16)
    words[: words.size // 2] = synth.bf16_weights(1, words.size // 2)[0]["bf16"]
    e, sm = oracle.bf16_split(words)
    spec = dict(kind=oracle.KIND_BF16EXP, rows=1, cols=words.size, symbols=e,
                chunk_symbols=65536)
    c = oracle.encode_container([spec])
    got, gst = gpu_decode(E, c, None, split_sm=sm)
    assert np.all(gst == 0)
    np.testing.assert_array_equal(got, words)


def test_split_block_counts_around_the_prefetch_depth(E):
    """bf16 split on the streaming path, chunks of 0 to 9 full blocks
    (256 symbols) with and without a partial block, and multi-chunk tensors
    whose chunks hold 1 to 9 blocks: the sign+mantissa bytes run several
    blocks ahead of the decode, so every count below and around that depth
    and every remainder of the unrolled block loop is covered."""
    _say("split block counts around the prefetch depth")
    specs, parts = [], []
    seed = 0
    for k in range(10):
        for r in (0, 48):
            if k == 0 and r == 0:
                continue
            parts.append((256 * k + r, 65536))
    for blocks in range(1, 10):
        parts.append((7 * 256 * blocks + 160, 256 * blocks))
    for n, C in parts:
        seed += 1
        w = synth.bf16_weights(1, n, sigma=float([0.02, 1.0, 300.0][seed % 3]))[0]["bf16"]
        specs.append((w, C))
    words = np.concatenate([w for w, _ in specs])
    e_all, sm = oracle.bf16_split(words)
    tens, at = [], 0
    for w, C in specs:
        tens.append(dict(kind=oracle.KIND_BF16EXP, rows=1, cols=w.size,
                         symbols=e_all[at:at + w.size], chunk_symbols=C))
        at += w.size
    c = oracle.encode_container(tens)
    assert [t["out_elem_offset"] for t in c.tensors] == list(np.cumsum([0] + [w.size for w, _ in specs])[:-1])
    got, gst = gpu_decode(E, c, None, split_sm=sm)
    assert np.all(gst == 0)
    np.testing.assert_array_equal(got, words)


@pytest.mark.parametrize("cols", [320, 512])
def test_nan_and_inf_scales_both_kernels(E, cols):
    """Non-finite scales and e4m3 NaN codes: cols=320 runs the simple
    kernel, cols=512 the streaming one; both must give the oracle's NaN
    propagation."""
    _say(f"nan/inf scales cols={cols}")
    rows = 12
    specs = []
    for kind in (oracle.KIND_INT8, oracle.KIND_E4M3):
        sym = synth.random_bytes(rows * cols, 60 + kind)
        sym[:256] = np.arange(256, dtype=np.uint8)
        sc = np.array([0x3F800000, 0xBF800000, 0x7FC00000, 0xFFC00000, 0x7FC12345, 0xFFA00001,
                       0x7F800000, 0xFF800000, 0x7F7FFFFF, 0x00000001, 0x00000000, 0x80000000],
                      np.uint32).view(np.float32)
        specs.append(dict(name=f"k{kind}", kind=kind, rows=rows, cols=cols, chunk_symbols=512,
                          symbols=sym, scales=sc))
    check_codes_and_bf16(E, specs)


@pytest.mark.parametrize("seed", range(6))
def test_random_batches_of_shapes_chunk_sizes_and_kinds(E, seed):
    """Batches of 1-5 tensors with random rows, row lengths (block-aligned or
    not), chunk sizes (multiples of 64 up to 2^16), kinds and spreads, so both
    kernels get a share: codes and bf16 equal the oracle's."""
    rng = np.random.default_rng(1000 + seed)
    specs = []
    for i in range(int(rng.integers(1, 6))):
        rows = int(rng.integers(1, 40))
        cols = int(rng.choice([64, 192, 256, 320, 512, 768, 1000, 2048, 4096, 4160]))
        C = int(rng.choice([64, 256, 512, 768, 4096, 16384, 65536]))
        if rng.random() < 0.3:
            sp = synth.e4m3_matrix(rows=rows, cols=cols)[0]
            sp["chunk_symbols"] = C
        else:
            sp = synth.random_int8_tensor(rows, cols, float(rng.uniform(0.3, 6.0)),
                                          100 * seed + i, C)
        specs.append(sp)
    _say(f"random batch {seed}: " + ", ".join(f"{s['rows']}x{s['cols']}/C{s['chunk_symbols']}"
                                             for s in specs))
    check_codes_and_bf16(E, specs)


@pytest.mark.parametrize("seed", range(3))
def test_random_exponent_streams(E, seed):
    rng = np.random.default_rng(2000 + seed)
    n = int(rng.integers(1, 300_000))
    C = int(rng.choice([64, 256, 4096, 65536]))
    w = synth.bf16_weights(1, n, sigma=float(rng.choice([0.02, 1.0, 300.0])))[0]["bf16"]
    e, sm = oracle.bf16_split(w)
    c = oracle.encode_container([dict(kind=oracle.KIND_BF16EXP, rows=1, cols=n, symbols=e,
                                      chunk_symbols=C)])
    _say(f"random exponent stream {seed}: {n} weights, C{C}")
    got, gst = gpu_decode(E, c, None, split_sm=sm)
    assert np.all(gst == 0)
    np.testing.assert_array_equal(got, w)
