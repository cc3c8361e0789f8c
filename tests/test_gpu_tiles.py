"""GPU parity of the fused product on tile-ordered chunks
(entq_decode_gemm_tiles, through the C ABI). The container holds each
tensor's codes in the library's tile order (oracle.tile_order pins it); the
expected weights are the oracle's: its decode of the container's chunks,
put back in row-major order by oracle.untile and dequantised by the oracle.
With one-hot activation rows every output is 1.0 * w, so the kernel must
return the oracle's bf16 weights bit for bit; with random activations the
fp32 result may differ from the fp64 product by at most cols * 2^-24 *
sum |x w| (products of two bf16 are exact in fp32; at most cols additions,
each rounding once)."""
import numpy as np
import pytest

import oracle
import oracle_rows
import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-tiles] {msg}", flush=True)


@pytest.fixture(scope="module")
def E():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import entropy_coded_weight_amd as E
    E.lib()
    return E


def _f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _tiled(E, specs, C_of):
    """specs with their symbols put in tile order (C = C_of(spec) columns
    per chunk), the container, plan and device buffers."""
    import torch
    tiled = []
    for sp in specs:
        C = C_of(sp)
        st = E.tile_order(sp["symbols"], sp["rows"], sp["cols"], C)
        tiled.append(dict(sp, symbols=st, chunk_symbols=16 * C, C=C,
                          kind=sp["kind"] | E.LAYOUT_TILES))
    b = E.encode_batch(tiled)
    p = E.plan(b.tensors, b.freq, b.chunks, b.blob.size)
    blob = torch.from_numpy(b.blob).cuda()
    scales = torch.from_numpy(np.concatenate([sp["scales"] for sp in specs])).cuda()
    return tiled, b, p, blob, scales


def _oracle_weights(b, tiled):
    """bf16 bits [rows, cols] of every tensor from the oracle's decode of the
    container, untiled and dequantised by the oracle."""
    out = []
    for t, sp in enumerate(tiled):
        ch = b.chunks[b.chunks["tensor"] == t]
        desc = oracle_rows.desc_of(ch)
        sym, st = oracle.decode_tensor(b.blob, desc, b.freq[t], sp["rows"] * sp["cols"])
        assert (st == 0).all()
        codes = oracle.untile(sym, sp["rows"], sp["cols"], sp["C"])
        w = oracle.dequant_tensor(codes.ravel(), sp["rows"], sp["cols"], sp["kind"] & 0xFF,
                                  sp["scales"])
        out.append(w.reshape(sp["rows"], sp["cols"]))
    return out


def _run(E, p, blob, scales, xs_host, specs, pad_x=0, pad_y=0, extra_rows=0, workspace=None):
    import torch
    xs, ys = [], []
    for x, sp in zip(xs_host, specs):
        m, c = x.shape
        xd = torch.zeros(m, c + pad_x, dtype=torch.bfloat16)
        xd[:, :c] = torch.from_numpy(x).to(torch.bfloat16)
        xs.append(xd.cuda())
        ys.append(torch.full((m + extra_rows, sp["rows"] + pad_y), float("nan"),
                             dtype=torch.float32, device="cuda"))
    m = xs_host[0].shape[0]
    status = torch.full((p.n_chunks,), -7, dtype=torch.int32, device="cuda")
    E.decode_gemm_tiles(p, blob, scales, xs, [y[:m] for y in ys], status, workspace=workspace)
    torch.cuda.synchronize()
    assert (status.cpu().numpy() == 0).all()
    return [y.cpu().numpy() for y in ys]


def _mixed():
    """int8 48 x 512 in 2 column chunks of 256; e4m3 32 x 768 in one chunk
    per band (results straight to Y); int8 64 x 2816 in 11 column chunks of
    256: 63 chunks. Returns the specs and their columns per chunk."""
    specs = [synth.random_int8_tensor(48, 512, 1.4, 720, 512),
             synth.e4m3_matrix(rows=32, cols=768)[0],
             synth.random_int8_tensor(64, 2816, 2.3, 721, 2816)]
    Cs = {sp["name"]: c for sp, c in zip(specs, (256, 768, 256))}
    return specs, (lambda sp: Cs[sp["name"]])


def test_decode_writes_the_row_major_tensors(E):
    """entq_decode of tile-ordered tensors writes their ordinary row-major
    outputs: the source codes, and bf16 equal to the oracle's dequantisation
    of the source codes, every element (and every chunk status 0)."""
    import torch
    specs, C_of = _mixed()
    tiled, b, p, blob, scales = _tiled(E, specs, C_of)
    codes = torch.empty(p.out_elems, dtype=torch.uint8, device="cuda")
    bf = torch.full((p.out_elems,), 0x5A5A, dtype=torch.int16, device="cuda")
    st = torch.full((p.n_chunks,), -7, dtype=torch.int32, device="cuda")
    E.decode(p, blob, codes, E.OUT_CODES, None, st)
    E.decode(p, blob, bf, E.OUT_BF16, scales, st)
    torch.cuda.synchronize()
    assert (st.cpu().numpy() == 0).all()
    got_c, got_b = codes.cpu().numpy(), bf.cpu().numpy().view(np.uint16)
    off = 0
    for sp in specs:
        n = sp["rows"] * sp["cols"]
        src = np.ascontiguousarray(sp["symbols"]).view(np.uint8)
        assert np.array_equal(got_c[off:off + n], src), sp["name"]
        want = oracle.dequant_tensor(src, sp["rows"], sp["cols"], sp["kind"], sp["scales"])
        assert np.array_equal(got_b[off:off + n], want), sp["name"]
        off += n


def test_linear_beyond_64_rows_on_tiles(E):
    """linear() on a tiled plan: the tiled product up to 64 rows, above that
    the row-major bf16 decode and library GEMMs; both within the bound."""
    import torch
    from entropy_coded_weight_amd.linear import linear
    specs, C_of = _mixed()
    tiled, b, p, blob, scales = _tiled(E, specs, C_of)
    W = _oracle_weights(b, tiled)
    rng = np.random.default_rng(48)
    for m in (64, 80):
        _say(f"linear on tiles, m={m}")
        xs_h = [_f32(rng.integers(0, 65536, (m, sp["cols"]), dtype=np.uint64).astype(np.uint16)
                     & np.uint16(0xBFFF)) for sp in specs]
        xs = [torch.from_numpy(x).to(torch.bfloat16).cuda() for x in xs_h]
        ys = [torch.full((m, sp["rows"]), float("nan"), dtype=torch.float32, device="cuda")
              for sp in specs]
        linear(p, blob, scales, xs, ys)
        torch.cuda.synchronize()
        for t, sp in enumerate(specs):
            assert oracle_rows.check_product(ys[t].cpu().numpy(), xs_h[t], W[t]) == sp["rows"]


def test_one_hot_activations_return_the_oracle_weights_exactly(E):
    specs, C_of = _mixed()
    tiled, b, p, blob, scales = _tiled(E, specs, C_of)
    W = _oracle_weights(b, tiled)
    rng = np.random.default_rng(41)
    for m in (1, 5, 16, 17, 33, 64):
        _say(f"one-hot, m={m}")
        xs, hit = [], []
        for sp in specs:
            c = rng.choice(sp["cols"], m, replace=False)
            x = np.zeros((m, sp["cols"]), np.float32)
            x[np.arange(m), c] = 1.0
            xs.append(x)
            hit.append(c)
        ys = _run(E, p, blob, scales, xs, specs, extra_rows=1)
        for t in range(len(specs)):
            want = _f32(W[t][:, hit[t]]).T
            assert np.array_equal(ys[t][:m].view(np.uint32), want.view(np.uint32)), (t, m)
            assert np.isnan(ys[t][m]).all(), (t, m)  # nothing written past m rows


def test_random_activations_within_the_accumulation_bound(E):
    specs, C_of = _mixed()
    tiled, b, p, blob, scales = _tiled(E, specs, C_of)
    W = _oracle_weights(b, tiled)
    rng = np.random.default_rng(42)
    for m, pad_x, pad_y in ((16, 0, 0), (3, 12, 2), (40, 4, 0), (64, 0, 5)):
        _say(f"random, m={m}, padded strides {pad_x}/{pad_y}")
        xs = [_f32(rng.integers(0, 65536, (m, sp["cols"]), dtype=np.uint64).astype(np.uint16)
                   & np.uint16(0xBFFF)) for sp in specs]  # finite bf16 values, |x| < 4
        ys = _run(E, p, blob, scales, xs, specs, pad_x, pad_y)
        for t, sp in enumerate(specs):
            assert oracle_rows.check_product(ys[t][:, :sp["rows"]], xs[t], W[t]) == sp["rows"]
            if pad_y:
                assert np.isnan(ys[t][:, sp["rows"]:]).all()


def test_results_are_reproducible_and_the_workspace_is_checked(E):
    import torch
    specs, C_of = _mixed()
    tiled, b, p, blob, scales = _tiled(E, specs, C_of)
    rng = np.random.default_rng(43)
    for m in (1, 4, 16, 40):
        _say(f"workspace over stale bytes, m={m}")
        xs = [rng.standard_normal((m, sp["cols"])).astype(np.float32) for sp in specs]
        n = int(E.lib().entq_decode_gemm_tiles_workspace_bytes(p.handle, m))
        # partial sums of the two tensors split in columns (2 x 48 and 11 x 64
        # rows, x m x 4 bytes) and the packed activations
        groups = -(-m // 16)
        want = sum(-(-4 * k * m * r // 256) * 256 for k, r in ((2, 48), (11, 64)))
        want += sum(-(-32 * groups * sp["cols"] // 256) * 256 for sp in specs)
        assert n == want, m
        ws = torch.full((n,), 0x7F, dtype=torch.uint8, device="cuda")  # stale bytes
        a = _run(E, p, blob, scales, xs, specs, workspace=ws)
        c = _run(E, p, blob, scales, xs, specs)
        for t in range(len(specs)):
            assert np.array_equal(a[t].view(np.uint32), c[t].view(np.uint32)), (t, m)
    xd = [torch.zeros(m, sp["cols"], dtype=torch.bfloat16, device="cuda") for sp in specs]
    yd = [torch.zeros(m, sp["rows"], dtype=torch.float32, device="cuda") for sp in specs]
    n = int(E.lib().entq_decode_gemm_tiles_workspace_bytes(p.handle, m))
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    with pytest.raises(E.EntqError):
        E.decode_gemm_tiles(p, blob, scales, xd, yd, workspace=ws[:n - 256])
    raw = torch.empty(n + 512, dtype=torch.uint8, device="cuda")
    base = (-raw.data_ptr()) % 256
    with pytest.raises(E.EntqError):
        E.decode_gemm_tiles(p, blob, scales, xd, yd, workspace=raw[base + 16:base + 16 + n])


def test_layouts_are_kept_apart(E):
    """Tile-ordered tensors are refused by the row-major fused calls, row-major
    ones by the tiled call, and a plan mixing the two layouts by the decode."""
    import torch
    specs, C_of = _mixed()
    tiled, b, p, blob, scales = _tiled(E, specs, C_of)
    m = 2
    xs = [torch.zeros(m, sp["cols"], dtype=torch.bfloat16, device="cuda") for sp in specs]
    ys = [torch.zeros(m, sp["rows"], dtype=torch.float32, device="cuda") for sp in specs]
    with pytest.raises(E.EntqError):
        E.decode_gemm(p, blob, scales, xs, ys)
    with pytest.raises(E.EntqError):
        E.decode_gemm_static(p, blob, scales, xs, ys)
    # the same codes, row-major, in chunks of the same size: refused by the tiled call
    rm = [dict(sp, chunk_symbols=16 * C_of(sp)) for sp in specs]
    b2 = E.encode_batch(rm)
    p2 = E.plan(b2.tensors, b2.freq, b2.chunks, b2.blob.size)
    with pytest.raises(E.EntqError):
        E.decode_gemm_tiles(p2, torch.from_numpy(b2.blob).cuda(), scales, xs, ys)
    # one tensor in tile order, the others row-major: the decode refuses the plan
    mixed = [tiled[0]] + rm[1:]
    b3 = E.encode_batch(mixed)
    p3 = E.plan(b3.tensors, b3.freq, b3.chunks, b3.blob.size)
    out = torch.empty(p3.out_elems, dtype=torch.int16, device="cuda")
    with pytest.raises(E.EntqError):
        E.decode(p3, torch.from_numpy(b3.blob).cuda(), out, E.OUT_BF16, scales)


def test_corrupt_chunks_report_the_decodes_status(E):
    import torch
    specs, C_of = _mixed()
    tiled, b, p, blob, scales = _tiled(E, specs, C_of)
    rng = np.random.default_rng(44)
    blob_h = b.blob.copy()
    bad = rng.choice(b.chunks.size, 20, replace=False)
    for c in bad:
        ch = b.chunks[c]
        lo = int(ch["byte_offset"]) + 256
        pos = rng.integers(lo, lo + 2 * int(ch["n_words"]), 3)
        blob_h[pos] ^= np.uint8(0x5A)
    blob = torch.from_numpy(blob_h).cuda()
    out = torch.empty(p.out_elems, dtype=torch.uint8, device="cuda")
    want = torch.full((p.n_chunks,), -7, dtype=torch.int32, device="cuda")
    E.decode(p, blob, out, E.OUT_CODES, None, want)
    torch.cuda.synchronize()
    want = want.cpu().numpy()
    assert (want != 0).sum() >= 10
    for m in (1, 16, 40):
        _say(f"corrupt chunks, m={m}")
        xs = [torch.ones(m, sp["cols"], dtype=torch.bfloat16, device="cuda") for sp in specs]
        ys = [torch.empty(m, sp["rows"], dtype=torch.float32, device="cuda") for sp in specs]
        got = torch.full((p.n_chunks,), -7, dtype=torch.int32, device="cuda")
        E.decode_gemm_tiles(p, blob, scales, xs, ys, got)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), want), m


def test_llama2_70b_layer_every_row(E):
    """A whole 70B-shaped layer in tile order with 4,096 columns per chunk
    (65,536 symbols: 2 column chunks of the 8,192-column tensors, 7 of the
    down projection), every output row against the oracle's weights, for
    m = 16, 64 and 1."""
    specs = synth.llama2_70b_layer(0)
    tiled, b, p, blob, scales = _tiled(E, specs, lambda sp: 4096)
    rng = np.random.default_rng(45)
    runs = []
    for m in (16, 64, 1):
        _say(f"70B-shaped layer 0 in tile order, m = {m}")
        xs = [(rng.standard_normal((m, sp["cols"])) * 0.5).astype(np.float32) for sp in specs]
        xs = [_f32((x.view(np.uint32) >> 16).astype(np.uint16)) for x in xs]  # bf16 values
        runs.append((m, xs, _run(E, p, blob, scales, xs, specs)))
    _say("oracle weights of layer 0")
    W = _oracle_weights(b, tiled)
    for t, sp in enumerate(specs):
        for m, xs, ys in runs:
            assert oracle_rows.check_product(ys[t], xs[t], W[t]) == sp["rows"], (sp["name"], m)


def test_lm_head_in_tile_order_every_row(E):
    """The 32,000 x 8,192 output projection alone, in tile order with 2,048
    columns per chunk (8,000 chunks, 4 column chunks per band: the partial
    sums and their reduction at full size), every output row at m = 16."""
    specs = synth.llama2_70b_lm_head(chunk_symbols=32768)
    tiled, b, p, blob, scales = _tiled(E, specs, lambda sp: 2048)
    rng = np.random.default_rng(46)
    m = 16
    _say("LM head in tile order, m = 16")
    x = _f32(((rng.standard_normal((m, 8192)) * 0.5).astype(np.float32).view(np.uint32)
              >> 16).astype(np.uint16))
    ys = _run(E, p, blob, scales, [x], specs)
    W = _oracle_weights(b, tiled)
    assert oracle_rows.check_product(ys[0], x, W[0]) == specs[0]["rows"]


# ---- BF16 exponent streams in tile order (entq_decode_gemm_tiles_bf16_split) ----

def _split_tiled(E, w, rows, cols, C):
    """bf16 words w [rows, cols]: exponent and sign+mantissa bytes, both in
    tile order; the container, plan and device buffers. The oracle's decode
    of the container, put back in row-major order and merged, must be w."""
    import torch
    e, sm = oracle.bf16_split(w.ravel())
    e_t = E.tile_order(e, rows, cols, C)
    sm_t = E.tile_order(sm, rows, cols, C)
    spec = dict(kind=E.KIND_BF16EXP | E.LAYOUT_TILES, rows=rows, cols=cols, symbols=e_t,
                chunk_symbols=16 * C)
    b = E.encode_batch([spec])
    p = E.plan(b.tensors, b.freq, b.chunks, b.blob.size)
    sym, st = oracle.decode_tensor(b.blob, oracle_rows.desc_of(b.chunks), b.freq[0], rows * cols)
    assert (st == 0).all()
    merged = oracle.bf16_merge(oracle.untile(sym, rows, cols, C).ravel(),
                               oracle.untile(sm_t, rows, cols, C).ravel())
    assert np.array_equal(merged.reshape(rows, cols), w)
    return p, torch.from_numpy(b.blob).cuda(), torch.from_numpy(sm_t).cuda()


def _run_split(E, p, blob, sm, x, rows, workspace=None):
    import torch
    xd = torch.from_numpy(x).to(torch.bfloat16).cuda()
    y = torch.full((x.shape[0] + 1, rows), float("nan"), dtype=torch.float32, device="cuda")
    status = torch.full((p.n_chunks,), -7, dtype=torch.int32, device="cuda")
    E.decode_gemm_tiles_bf16_split(p, blob, sm, [xd], [y[:x.shape[0]]], status,
                                   workspace=workspace)
    torch.cuda.synchronize()
    assert (status.cpu().numpy() == 0).all()
    out = y.cpu().numpy()
    assert np.isnan(out[-1]).all()  # nothing written past m rows
    return out[:-1]


@pytest.mark.parametrize("rows,cols,C", [(48, 768, 256), (32, 512, 512), (64, 1792, 256)])
def test_bf16_split_one_hot_returns_the_source_weights(E, rows, cols, C):
    rng = np.random.default_rng(rows + cols)
    w = rng.integers(0, 1 << 16, size=rows * cols, dtype=np.uint64).astype(np.uint16)
    w[(w & 0x7F80) == 0x7F80] &= 0xBFFF  # finite weights, so that 1.0 * w is w
    w[w == 0x8000] = 0  # a -0 weight would come out +0 (+0 + -0 = +0 in the sums)
    w = w.reshape(rows, cols)
    p, blob, sm = _split_tiled(E, w, rows, cols, C)
    for m in (1, 3, 16, 40):
        _say(f"bf16 split in tile order, {rows}x{cols}, C={C}, one-hot, m={m}")
        c = rng.choice(cols, m, replace=False)
        x = np.zeros((m, cols), np.float32)
        x[np.arange(m), c] = 1.0
        y = _run_split(E, p, blob, sm, x, rows)
        assert np.array_equal(y.view(np.uint32), _f32(w[:, c]).T.view(np.uint32)), m


def test_bf16_split_decode_rebuilds_the_source(E):
    """entq_decode_bf16_split of tile-ordered exponent streams writes the
    source bf16 in row-major order, every word."""
    import torch
    rng = np.random.default_rng(49)
    rows, cols, C = 64, 1792, 256
    w = rng.integers(0, 1 << 16, size=rows * cols, dtype=np.uint64).astype(np.uint16)
    w = w.reshape(rows, cols)
    p, blob, sm = _split_tiled(E, w, rows, cols, C)
    out = torch.empty(rows * cols, dtype=torch.int16, device="cuda")
    st = torch.full((p.n_chunks,), -7, dtype=torch.int32, device="cuda")
    E.decode_bf16_split(p, blob, sm, out, st)
    torch.cuda.synchronize()
    assert (st.cpu().numpy() == 0).all()
    assert np.array_equal(out.cpu().numpy().view(np.uint16), w.ravel())


def test_bf16_split_8192x8192_every_row(E):
    rows = cols = 8192
    w = synth.bf16_weights(rows, cols)[0]["bf16"].reshape(rows, cols)
    p, blob, sm = _split_tiled(E, w, rows, cols, 2048)
    rng = np.random.default_rng(47)
    for m in (16, 1):
        _say(f"bf16 split 8192x8192 in tile order, m = {m}, every row")
        x = _f32(((rng.standard_normal((m, cols)) * 0.5).astype(np.float32).view(np.uint32)
                  >> 16).astype(np.uint16))
        y = _run_split(E, p, blob, sm, x, rows)
        assert oracle_rows.check_product(y, x, w) == rows


@pytest.mark.parametrize("seed", [101, 102, 103, 104])
def test_random_batches(E, seed):
    """Random plans in tile order: 1 to 5 tensors (int8 and e4m3), bands of
    16 rows, chunk widths 16 to 512 columns dividing 1 to 5 column chunks,
    random m; one-hot activations return the oracle's weights exactly and
    random ones stay within the bound."""
    rng = np.random.default_rng(seed)
    specs, Cs = [], {}
    for i in range(int(rng.integers(1, 6))):
        C = int(rng.choice([16, 48, 256, 512]))
        rows, cols = 16 * int(rng.integers(1, 9)), C * int(rng.integers(1, 6))
        if i % 3 == 2:
            sp = synth.e4m3_matrix(rows=rows, cols=cols)[0]
            sp["name"] = f"e{seed}_{i}"
        else:
            sp = synth.random_int8_tensor(rows, cols, float(rng.uniform(0.8, 3.0)),
                                          seed * 10 + i, 16 * C)
        Cs[sp["name"]] = C
        specs.append(sp)
    tiled, b, p, blob, scales = _tiled(E, specs, lambda sp: Cs[sp["name"]])
    W = _oracle_weights(b, tiled)
    m = int(rng.integers(1, 65))
    _say(f"random batch {seed}: {len(specs)} tensors, m={m}")
    xs, hit = [], []
    for sp in specs:
        c = rng.choice(sp["cols"], m, replace=True)  # (a column may be hit twice)
        x = np.zeros((m, sp["cols"]), np.float32)
        x[np.arange(m), c] = 1.0
        xs.append(x)
        hit.append(c)
    ys = _run(E, p, blob, scales, xs, specs, extra_rows=1)
    for t in range(len(specs)):
        want = _f32(W[t][:, hit[t]]).T
        assert np.array_equal(ys[t][:m].view(np.uint32), want.view(np.uint32)), t
    xs = [_f32(rng.integers(0, 65536, (m, sp["cols"]), dtype=np.uint64).astype(np.uint16)
               & np.uint16(0xBFFF)) for sp in specs]
    ys = _run(E, p, blob, scales, xs, specs, pad_x=4, pad_y=2)
    for t, sp in enumerate(specs):
        assert oracle_rows.check_product(ys[t][:, :sp["rows"]], xs[t], W[t]) == sp["rows"]


@pytest.mark.parametrize("rows,cols,C", [(16, 16, 16), (48, 768, 256), (64, 2816, 256),
                                         (32, 28672, 7168)])
def test_tile_order_on_the_device_matches_the_oracle(E, rows, cols, C):
    import torch
    rng = np.random.default_rng(rows + cols)
    w = rng.integers(0, 256, rows * cols, dtype=np.uint8)
    got = E.tile_order_device(torch.from_numpy(w).cuda(), rows, cols, C)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), oracle.tile_order(w, rows, cols, C))
