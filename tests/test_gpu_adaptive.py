"""GPU parity of the per-chunk-table (adaptive) decode through the C ABI:
codes and bf16 output equal the oracle's adaptive decode; BF16 exponent
streams with per-chunk tables rebuild every bf16 word; a chunk whose table
is corrupt reports ENTQ_CHUNK_BAD_TABLE while its neighbours decode; a whole
70B-shaped layer is checked chunk by chunk, every element."""
import numpy as np
import pytest

import oracle
import oracle_rows
import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-adaptive] {msg}", flush=True)


@pytest.fixture(scope="module")
def E():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import entropy_coded_weight_amd as E
    E.lib()
    return E


def _plan(E, c, blob=None):
    import torch
    tens = np.zeros(len(c.tensors), E.TENSOR_DESC)
    for t, td in enumerate(c.tensors):
        tens[t] = (td["kind"], td["rows"], td["cols"], td["chunk_symbols"], td["n_symbols"],
                   td["out_elem_offset"], td["scale_row_offset"])
    ch = np.zeros(c.n_chunks, E.CHUNK_DESC)
    ch["tensor"], ch["n_symbols"], ch["n_words"] = c.chunks[:, 0], c.chunks[:, 1], c.chunks[:, 2]
    ch["byte_offset"], ch["elem_offset"] = c.chunks[:, 3], c.chunks[:, 4]
    b = c.blob if blob is None else blob
    return E.plan(tens, None, ch, b.size), torch.from_numpy(b).cuda()


def _decode(E, p, blob, total, out_kind, scales=None):
    import torch
    status = torch.full((p.n_chunks,), -7, dtype=torch.int32, device="cuda")
    if out_kind == E.OUT_CODES:
        out = torch.zeros(total, dtype=torch.uint8, device="cuda")
        E.decode(p, blob, out, E.OUT_CODES, None, status)
    else:
        out = torch.zeros(total, dtype=torch.int16, device="cuda")
        E.decode(p, blob, out, E.OUT_BF16, torch.from_numpy(scales).cuda(), status)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    return (o.view(np.uint16) if o.dtype == np.int16 else o), status.cpu().numpy()


def _specs():
    specs = [synth.random_int8_tensor(r, c, 0.6 + 0.5 * i, 140 + i, C)
             for i, (r, c, C) in enumerate([(3, 256, 256), (17, 512, 4096), (5, 4352, 4096),
                                            (33, 1024, 65536)])]
    one = synth.random_int8_tensor(16, 256, 1.0, 150, 1024)
    one["symbols"] = np.full(one["symbols"].shape, 77, np.uint8)
    allb = synth.random_int8_tensor(64, 512, 1.0, 151, 4096)
    allb["symbols"] = synth.random_bytes(64 * 512, 151).view(np.uint8)
    e = synth.e4m3_matrix(rows=48, cols=768)[0]
    e["chunk_symbols"] = 768 * 4
    specs += [one, allb, e, synth.banded_int8_tensor(48, 2816, 4, 6, 2816 * 4)]
    return specs


def test_codes_and_bf16_match_the_oracle(E):
    specs = _specs()
    _say(f"{len(specs)} tensors, per-chunk tables")
    c = oracle.encode_container_adaptive(specs)
    p, blob = _plan(E, c)
    total = sum(td["n_symbols"] for td in c.tensors)
    syms, st = oracle.decode_container_adaptive_symbols(c)
    assert (st == 0).all()
    got, gst = _decode(E, p, blob, total, E.OUT_CODES)
    np.testing.assert_array_equal(got, np.concatenate(syms))
    np.testing.assert_array_equal(gst, st)
    scales = np.concatenate([np.asarray(s["scales"], np.float32) for s in specs])
    want, _ = oracle.decode_container_adaptive_bf16(c, scales)
    got, gst = _decode(E, p, blob, total, E.OUT_BF16, scales)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(gst, st)


def test_e4m3_every_code_including_nan(E):
    """Every e4m3 code, the two NaN codes included, through the per-chunk-table
    bf16 path (its stage holds each code in the low byte of a 16-bit slot):
    equal to the oracle bit for bit, with negative, huge and small scales."""
    _say("per-chunk tables: e4m3 all 256 codes incl. NaN")
    sym = synth.random_bytes(64 * 512, 12)
    sym[:256] = np.arange(256, dtype=np.uint8)
    sym[4096:4352] = np.arange(256, dtype=np.uint8)[::-1]
    sc = synth.uniform_f32(1e-3, 4.0, 64, synth.key(98, 3, 0, 1))
    sc[:3] = np.array([1.0, -1.0, 3.0e38], np.float32)
    sp = dict(name="e", kind=oracle.KIND_E4M3, rows=64, cols=512, chunk_symbols=4096,
              symbols=sym, scales=sc)
    c = oracle.encode_container_adaptive([sp])
    p, blob = _plan(E, c)
    want, st = oracle.decode_container_adaptive_bf16(c, sc)
    assert (st == 0).all()
    got, gst = _decode(E, p, blob, sym.size, E.OUT_BF16, sc)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(gst, st)
    codes, _ = _decode(E, p, blob, sym.size, E.OUT_CODES)
    np.testing.assert_array_equal(codes, sym)


def test_corrupt_table_is_reported_per_chunk(E):
    sp = synth.random_int8_tensor(32, 512, 1.5, 152, 1024)
    c = oracle.encode_container_adaptive([sp])
    blob = c.blob.copy()
    off = int(c.chunks[3, 3])
    blob[off + 2 * 130] ^= 4   # chunk 3's table no longer sums to 4096
    bad = oracle.Container(blob, c.tensors, c.chunks)
    syms, st = oracle.decode_container_adaptive_symbols(bad)
    assert st.tolist() == [0, 0, 0, oracle.STATUS_BAD_TABLE] + [0] * (c.n_chunks - 4)
    p, b = _plan(E, bad, blob)
    got, gst = _decode(E, p, b, sp["rows"] * sp["cols"], E.OUT_CODES)
    np.testing.assert_array_equal(gst, st)
    src = sp["symbols"]
    for k, (t, n, nw, o, e0) in enumerate(c.chunks.astype(np.int64)):
        if st[k] == 0:
            np.testing.assert_array_equal(got[e0:e0 + n], src[e0:e0 + n])
        else:
            assert (got[e0:e0 + n] == 0).all()  # no output for the rejected chunk


def test_other_calls_reject_adaptive_plans(E):
    import torch
    c = oracle.encode_container_adaptive([synth.random_int8_tensor(16, 512, 1.0, 153, 1024)])
    p, blob = _plan(E, c)
    x = torch.zeros(2, 512, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(2, 16, dtype=torch.float32, device="cuda")
    scales = torch.ones(16, dtype=torch.float32, device="cuda")
    with pytest.raises(E.EntqError):
        E.decode_gemm(p, blob, scales, [x], [y])
    out = torch.zeros(16 * 512, dtype=torch.int16, device="cuda")
    sm = torch.zeros(16 * 512, dtype=torch.uint8, device="cuda")
    with pytest.raises(E.EntqError):
        E.decode_bf16_split(p, blob, sm, out)


def test_llama2_70b_layer_every_chunk(E):
    import torch
    _say("70B-shaped layer 0 with per-chunk tables (library host encoder), every element")
    specs = synth.llama2_70b_layer(0)
    b = E.encode_batch_adaptive(specs)
    p = E.plan(b.tensors, None, b.chunks, b.blob.size)
    blob = torch.from_numpy(b.blob).cuda()
    scales = np.concatenate([s["scales"] for s in specs])
    total = sum(s["rows"] * s["cols"] for s in specs)
    got, gst = _decode(E, p, blob, total, E.OUT_BF16, scales)
    assert (gst == 0).all()
    for t, sp in enumerate(specs):
        o = int(b.tensors[t]["out_elem_offset"])
        n = sp["rows"] * sp["cols"]
        want = oracle_rows.tensor_from_oracle(b.blob, b.chunks[b.chunks["tensor"] == t], None,
                                              sp, adaptive=True)
        np.testing.assert_array_equal(got[o:o + n], want.ravel(), err_msg=sp["name"])


def test_exponent_streams_with_per_chunk_tables(E):
    """entq_decode_bf16_split on a per-chunk-table plan: a 2048 x 8192 BF16
    matrix and a random (high-entropy) stream with a ragged last block; the
    bf16 words equal the source and the oracle's merge, the codes output the
    exponent bytes. The fused product still rejects such a plan."""
    import torch
    w1 = synth.bf16_weights(2048, 8192)[0]["bf16"]
    rng = np.random.default_rng(21)
    w2 = rng.integers(0, 1 << 16, size=3 * 70_001 + 5, dtype=np.uint64).astype(np.uint16)
    specs, sms, exps = [], [], []
    for w, cols in ((w1, 8192), (w2, w2.size)):
        e, sm = oracle.bf16_split(w)
        specs.append(dict(kind=oracle.KIND_BF16EXP, rows=w.size // cols, cols=cols, symbols=e,
                          chunk_symbols=65536))
        sms.append(sm)
        exps.append(e)
    _say(f"exponent streams, per-chunk tables: {w1.size + w2.size} weights")
    c = oracle.encode_container_adaptive(specs)
    sm_all = np.concatenate(sms)
    want, st = oracle.decode_container_adaptive_split(c, sm_all)
    assert (st == 0).all()
    np.testing.assert_array_equal(want, np.concatenate([w1, w2]))
    p, blob = _plan(E, c)
    total = w1.size + w2.size
    status = torch.full((p.n_chunks,), -7, dtype=torch.int32, device="cuda")
    out = torch.zeros(total, dtype=torch.int16, device="cuda")
    E.decode_bf16_split(p, blob, torch.from_numpy(sm_all).cuda(), out, status)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint16), want)
    np.testing.assert_array_equal(status.cpu().numpy(), st)
    got, gst = _decode(E, p, blob, total, E.OUT_CODES)
    np.testing.assert_array_equal(got, np.concatenate(exps))
    np.testing.assert_array_equal(gst, st)
    x = torch.zeros(1, 8192, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(1, 2048, dtype=torch.float32, device="cuda")
    x2 = torch.zeros(1, w2.size + 3, dtype=torch.bfloat16, device="cuda")
    y2 = torch.zeros(1, 1, dtype=torch.float32, device="cuda")
    with pytest.raises(E.EntqError):
        E.decode_gemm_bf16_split(p, blob, torch.from_numpy(sm_all).cuda(), [x, x2], [y, y2])


@pytest.mark.parametrize("seed", range(4))
def test_random_batches_with_per_chunk_tables(E, seed):
    """Batches of 1-6 tensors with per-chunk tables: random rows, block-aligned
    row lengths, chunk sizes (multiples of 256 up to 2^16, some not dividing
    the tensor), int8 of random spread or e4m3, now and then a one-symbol or a
    uniformly random tensor. Codes and bf16 equal the oracle's adaptive decode,
    statuses too."""
    rng = np.random.default_rng(3000 + seed)
    specs = []
    for i in range(int(rng.integers(1, 7))):
        rows = int(rng.integers(1, 48))
        cols = int(rng.choice([256, 512, 768, 1024, 2560, 4096]))
        C = int(rng.choice([256, 512, 1280, 4096, 16384, 65536]))
        u = rng.random()
        if u < 0.25:
            sp = synth.e4m3_matrix(rows=rows, cols=cols)[0]
            sp["chunk_symbols"] = C
        else:
            sp = synth.random_int8_tensor(rows, cols, float(rng.uniform(0.3, 6.0)),
                                          4000 + 10 * seed + i, C)
            if u > 0.9:
                sp["symbols"] = np.full(sp["symbols"].shape, int(rng.integers(0, 256)), np.uint8)
            elif u > 0.8:
                sp["symbols"] = synth.random_bytes(rows * cols, 4100 + 10 * seed + i).view(np.uint8)
        specs.append(sp)
    _say(f"random per-chunk-table batch {seed}: " + ", ".join(
        f"{s['rows']}x{s['cols']}/C{s['chunk_symbols']}" for s in specs))
    c = oracle.encode_container_adaptive(specs)
    p, blob = _plan(E, c)
    total = sum(td["n_symbols"] for td in c.tensors)
    syms, st = oracle.decode_container_adaptive_symbols(c)
    assert (st == 0).all()
    got, gst = _decode(E, p, blob, total, E.OUT_CODES)
    np.testing.assert_array_equal(got, np.concatenate(syms))
    np.testing.assert_array_equal(gst, st)
    scales = np.concatenate([np.asarray(s["scales"], np.float32) for s in specs])
    want, _ = oracle.decode_container_adaptive_bf16(c, scales)
    got, gst = _decode(E, p, blob, total, E.OUT_BF16, scales)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(gst, st)
