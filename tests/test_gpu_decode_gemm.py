"""GPU parity of the fused decode + product (entq_decode_gemm, through the C
ABI). Expected values come from the oracle: its decoded bf16 weights times
the activations in fp64. With one-hot activation rows every output is one
product 1.0 * w, so the kernel must return the oracle's bf16 weights exactly;
with random activations the fp32 accumulation may differ from the fp64 sum
by at most cols * 2^-24 * sum |x w| (each of at most cols additions rounds
once, products of two bf16 are exact in fp32)."""
import numpy as np
import pytest

import oracle
import oracle_rows
import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-decode-gemm] {msg}", flush=True)


@pytest.fixture(scope="module")
def E():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import entropy_coded_weight_amd as E
    E.lib()
    return E


def _oracle_weights(b, specs):
    """bf16 bits [rows, cols] of every tensor, decoded by the oracle from the
    container's bytes."""
    out = []
    for t, sp in enumerate(specs):
        ch = b.chunks[b.chunks["tensor"] == t]
        desc = np.stack([ch["n_symbols"], ch["n_words"], ch["byte_offset"], ch["elem_offset"]],
                        axis=1).astype(np.uint64)
        sym, st = oracle.decode_tensor(b.blob, desc, b.freq[t], sp["rows"] * sp["cols"])
        assert (st == 0).all()
        w = oracle.dequant_tensor(sym, sp["rows"], sp["cols"], sp["kind"], sp["scales"])
        out.append(w.reshape(sp["rows"], sp["cols"]))
    return out


def _f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _setup(E, specs):
    import torch
    b = E.encode_batch(specs)
    p = E.plan(b.tensors, b.freq, b.chunks, b.blob.size)
    blob = torch.from_numpy(b.blob).cuda()
    scales = torch.from_numpy(np.concatenate([sp["scales"] for sp in specs])).cuda()
    return b, p, blob, scales


def _run(E, p, blob, scales, xs_host, specs, pad_x=0, pad_y=0, workspace=None):
    """xs_host: list of float32 arrays [m, cols] (values already bf16)."""
    import torch
    xs, ys = [], []
    for x, sp in zip(xs_host, specs):
        m, c = x.shape
        xd = torch.zeros(m, c + pad_x, dtype=torch.bfloat16)
        xd[:, :c] = torch.from_numpy(x).to(torch.bfloat16)
        xs.append(xd.cuda())
        ys.append(torch.full((m, sp["rows"] + pad_y), float("nan"), dtype=torch.float32,
                             device="cuda"))
    status = torch.full((p.n_chunks,), -7, dtype=torch.int32, device="cuda")
    E.decode_gemm(p, blob, scales, [x[:, :] for x in xs], ys, status, workspace=workspace)
    torch.cuda.synchronize()
    assert (status.cpu().numpy() == 0).all()
    return [y.cpu().numpy() for y in ys]


def _mixed_specs():
    specs = []
    # int8, 512 columns (2 blocks), 4 rows per chunk: 12 chunks, one partial group
    sp = synth.random_int8_tensor(48, 512, 1.4, 700, 512 * 4)
    specs.append(sp)
    # e4m3, 768 columns (3 blocks, odd), 3 rows per chunk, last chunk one row
    e = synth.e4m3_matrix(rows=40, cols=768)[0]
    e["chunk_symbols"] = 768 * 3
    specs.append(e)
    # int8, 2816 columns (11 blocks), one row per chunk: 100 chunks, 7 groups
    specs.append(synth.random_int8_tensor(100, 2816, 2.3, 702, 2816))
    return specs


def test_one_hot_activations_return_the_oracle_weights_exactly(E):
    specs = _mixed_specs()
    b, p, blob, scales = _setup(E, specs)
    W = _oracle_weights(b, specs)
    rng = np.random.default_rng(4)
    for m in (1, 7, 16, 17, 40, 64):
        _say(f"one-hot, m={m}")
        xs, cols_hit = [], []
        for sp in specs:
            c = rng.choice(sp["cols"], m, replace=False)
            x = np.zeros((m, sp["cols"]), np.float32)
            x[np.arange(m), c] = 1.0
            xs.append(x)
            cols_hit.append(c)
        ys = _run(E, p, blob, scales, xs, specs)
        for t, sp in enumerate(specs):
            want = _f32(W[t][:, cols_hit[t]]).T          # [m, rows]
            assert np.array_equal(ys[t].view(np.uint32), want.view(np.uint32)), (t, m)


def test_regions_and_scale_rows_far_out(E):
    """Chunk regions more than 4 GiB into the blob and scale rows more than
    4 M rows into the scale array: one-hot products still return the
    oracle's weights exactly (64-bit offsets in the fused kernel)."""
    import torch
    specs = _mixed_specs()
    b = E.encode_batch(specs)
    W = _oracle_weights(b, specs)
    G = (1 << 32) + 4096
    row_shift = (1 << 22) + 3
    t = b.tensors.copy()
    t["scale_row_offset"] += row_shift
    ch = b.chunks.copy()
    ch["byte_offset"] += np.uint64(G)
    p = E.plan(t, b.freq, ch, G + b.blob.size)
    blob = torch.empty(G + b.blob.size, dtype=torch.uint8, device="cuda")
    blob[G:] = torch.from_numpy(b.blob).cuda()
    sc = np.concatenate([sp["scales"] for sp in specs])
    scales = torch.zeros(row_shift + sc.size, dtype=torch.float32, device="cuda")
    scales[row_shift:] = torch.from_numpy(sc).cuda()
    rng = np.random.default_rng(9)
    for m in (1, 16, 40):
        _say(f"one-hot, far regions and scale rows, m={m}")
        xs, cols_hit = [], []
        for sp in specs:
            c = rng.choice(sp["cols"], m, replace=False)
            x = np.zeros((m, sp["cols"]), np.float32)
            x[np.arange(m), c] = 1.0
            xs.append(x)
            cols_hit.append(c)
        ys = _run(E, p, blob, scales, xs, specs)
        for k, sp in enumerate(specs):
            want = _f32(W[k][:, cols_hit[k]]).T
            assert np.array_equal(ys[k].view(np.uint32), want.view(np.uint32)), (k, m)
    p.close()
    del blob
    torch.cuda.empty_cache()


def test_more_tensors_than_one_launch_takes(E):
    """19 tensors (a launch takes 16): int8 and e4m3, 1 to 11 blocks per row,
    1 to 4 rows per chunk, in an order the launcher rearranges (longest rows
    first). One-hot activations return the oracle's weights exactly."""
    rng = np.random.default_rng(21)
    specs = []
    for i in range(19):
        cols = int(rng.choice([256, 512, 768, 1024, 2816]))
        rows = int(rng.integers(3, 41))
        chunk_rows = int(rng.integers(1, 5))
        if i % 5 == 2:
            sp = synth.e4m3_matrix(rows=rows, cols=cols)[0]
        else:
            sp = synth.random_int8_tensor(rows, cols, float(rng.uniform(0.8, 3.0)), 800 + i,
                                          cols * chunk_rows)
        sp["chunk_symbols"] = cols * chunk_rows
        specs.append(sp)
    b, p, blob, scales = _setup(E, specs)
    W = _oracle_weights(b, specs)
    for m in (2, 5, 33):  # (more than 16 tensors: the matrix cores also for m <= 4)
        _say(f"19 tensors, one-hot, m={m}")
        xs, cols_hit = [], []
        for sp in specs:
            c = rng.choice(sp["cols"], m, replace=False)
            x = np.zeros((m, sp["cols"]), np.float32)
            x[np.arange(m), c] = 1.0
            xs.append(x)
            cols_hit.append(c)
        ys = _run(E, p, blob, scales, xs, specs)
        for t, sp in enumerate(specs):
            want = _f32(W[t][:, cols_hit[t]]).T
            assert np.array_equal(ys[t].view(np.uint32), want.view(np.uint32)), (t, m)


def test_random_activations_within_the_accumulation_bound(E):
    specs = _mixed_specs()
    b, p, blob, scales = _setup(E, specs)
    W = _oracle_weights(b, specs)
    rng = np.random.default_rng(5)
    for m, pad_x, pad_y in ((16, 0, 0), (5, 12, 3), (1, 4, 0), (33, 8, 1), (64, 0, 0)):
        _say(f"random, m={m}, padded strides {pad_x}/{pad_y}")
        xs = [_f32(rng.integers(0, 65536, (m, sp["cols"]), dtype=np.uint64).astype(np.uint16)
                   & np.uint16(0xBFFF)) for sp in specs]  # finite bf16 values, |x| < 4
        ys = _run(E, p, blob, scales, xs, specs, pad_x, pad_y)
        for t, sp in enumerate(specs):
            w = _f32(W[t]).astype(np.float64)
            x = xs[t].astype(np.float64)
            ref = x @ w.T
            bound = sp["cols"] * 2.0 ** -24 * (np.abs(x) @ np.abs(w).T)
            got = ys[t][:, :sp["rows"]]
            assert (np.abs(got - ref) <= bound + 1e-30).all(), (t, m)
            if pad_y:
                assert np.isnan(ys[t][:, sp["rows"]:]).all()  # nothing written past the rows


def test_linear_with_more_than_64_rows(E):
    """linear(): beyond 64 activation rows the layer is decoded once and each
    product is a library GEMM in fp32 accumulation -- within the same bound
    of the fp64 product of the oracle's weights; up to 64 rows it is the
    fused kernel, bit for bit."""
    import torch
    from entropy_coded_weight_amd.linear import FUSED_MAX_ROWS, linear
    specs = _mixed_specs()
    b, p, blob, scales = _setup(E, specs)
    W = _oracle_weights(b, specs)
    rng = np.random.default_rng(11)
    weights = torch.empty(p.out_elems, dtype=torch.int16, device="cuda")
    for m in (FUSED_MAX_ROWS, FUSED_MAX_ROWS + 1, 300):
        _say(f"linear, m={m}")
        xs_h = [_f32(rng.integers(0, 65536, (m, sp["cols"]), dtype=np.uint64).astype(np.uint16)
                     & np.uint16(0xBFFF)) for sp in specs]
        xs = [torch.from_numpy(x).to(torch.bfloat16).cuda() for x in xs_h]
        ys = [torch.full((m, sp["rows"]), float("nan"), dtype=torch.float32, device="cuda")
              for sp in specs]
        status = torch.full((p.n_chunks,), -7, dtype=torch.int32, device="cuda")
        linear(p, blob, scales, xs, ys, weights=weights, chunk_status=status)
        torch.cuda.synchronize()
        assert (status.cpu().numpy() == 0).all()
        if m <= FUSED_MAX_ROWS:
            fused = _run(E, p, blob, scales, xs_h, specs)
        for t, sp in enumerate(specs):
            w = _f32(W[t]).astype(np.float64)
            x = xs_h[t].astype(np.float64)
            ref = x @ w.T
            bound = sp["cols"] * 2.0 ** -24 * (np.abs(x) @ np.abs(w).T)
            got = ys[t].cpu().numpy()
            assert (np.abs(got - ref) <= bound + 1e-30).all(), (t, m)
            if m <= FUSED_MAX_ROWS:
                assert np.array_equal(got.view(np.uint32), fused[t].view(np.uint32)), (t, m)


def test_packed_activations_give_the_same_bits(E):
    """With a workspace the activations are first copied into the waves'
    read order; the products are the same bit for bit, padded strides and
    partial 16-row groups included."""
    import torch
    specs = _mixed_specs()
    b, p, blob, scales = _setup(E, specs)
    rng = np.random.default_rng(9)
    for m, pad_x in ((1, 0), (16, 4), (17, 0), (40, 12), (64, 0)):
        _say(f"packed vs unpacked activations, m={m}")
        xs = [rng.standard_normal((m, sp["cols"])).astype(np.float32) for sp in specs]
        n = int(E.lib().entq_decode_gemm_workspace_bytes(p.handle, m))
        groups = -(-m // 16)
        assert n == sum(-(-32 * groups * sp["cols"] // 256) * 256 for sp in specs)
        ws = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")  # stale bytes
        plain = _run(E, p, blob, scales, xs, specs, pad_x, workspace="none")
        packed = _run(E, p, blob, scales, xs, specs, pad_x, workspace=ws)
        for t in range(len(specs)):
            assert np.array_equal(plain[t].view(np.uint32), packed[t].view(np.uint32)), (t, m)


def test_workspace_size_and_alignment_are_checked(E):
    import torch
    specs = _mixed_specs()
    b, p, blob, scales = _setup(E, specs)
    m = 33
    xs = [torch.zeros(m, sp["cols"], dtype=torch.bfloat16, device="cuda") for sp in specs]
    ys = [torch.zeros(m, sp["rows"], dtype=torch.float32, device="cuda") for sp in specs]
    n = int(E.lib().entq_decode_gemm_workspace_bytes(p.handle, m))
    raw = torch.empty(n + 512, dtype=torch.uint8, device="cuda")
    base = (-raw.data_ptr()) % 256
    with pytest.raises(E.EntqError):
        E.decode_gemm(p, blob, scales, xs, ys, workspace=raw[base:base + n - 256])  # short
    with pytest.raises(E.EntqError):
        E.decode_gemm(p, blob, scales, xs, ys, workspace=raw[base + 16:base + 16 + n])  # 16 off
    assert int(E.lib().entq_decode_gemm_workspace_bytes(p.handle, 65)) == 0


def test_results_are_reproducible(E):
    specs = _mixed_specs()
    b, p, blob, scales = _setup(E, specs)
    rng = np.random.default_rng(6)
    xs = [rng.standard_normal((16, sp["cols"])).astype(np.float32) for sp in specs]
    a = _run(E, p, blob, scales, xs, specs)
    c = _run(E, p, blob, scales, xs, specs)
    for t in range(len(specs)):
        assert np.array_equal(a[t].view(np.uint32), c[t].view(np.uint32))


def test_rejects_more_than_64_activation_rows(E):
    import torch
    specs = _mixed_specs()[:1]
    b, p, blob, scales = _setup(E, specs)
    x = torch.zeros(65, specs[0]["cols"], dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(65, specs[0]["rows"], dtype=torch.float32, device="cuda")
    with pytest.raises(E.EntqError):
        E.decode_gemm(p, blob, scales, [x], [y])


def test_rejects_chunks_that_split_rows(E):
    import torch
    sp = synth.random_int8_tensor(16, 512, 1.0, 703, 4096 + 64 * 3)  # not a multiple of cols
    b, p, blob, scales = _setup(E, [sp])
    x = torch.zeros(4, 512, dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(4, 16, dtype=torch.float32, device="cuda")
    with pytest.raises(E.EntqError):
        E.decode_gemm(p, blob, scales, [x], [y])


def test_llama2_70b_layer_every_row(E):
    """A whole 70B-shaped layer in chunks of whole rows (at most 65,536
    symbols: 8 rows of 8,192 columns, 2 of 28,672), every output row against
    the oracle's weights, for m = 16 (matrix cores) and m = 4 and 1 (the
    vector-unit product, several chunks per wave)."""
    specs = synth.llama2_70b_layer(0)
    for sp in specs:
        sp["chunk_symbols"] = sp["cols"] * max(1, 65536 // sp["cols"])
    b, p, blob, scales = _setup(E, specs)
    rng = np.random.default_rng(7)
    runs = []
    for m in (16, 4, 1):
        _say(f"70B-shaped layer 0 with row-aligned chunks, m = {m}")
        xs = [(rng.standard_normal((m, sp["cols"])) * 0.5).astype(np.float32) for sp in specs]
        xs = [_f32((x.view(np.uint32) >> 16).astype(np.uint16)) for x in xs]  # bf16 values
        runs.append((m, xs, _run(E, p, blob, scales, xs, specs)))
    for t, sp in enumerate(specs):
        W = oracle_rows.tensor_from_oracle(b.blob, b.chunks[b.chunks["tensor"] == t], b.freq[t],
                                           sp)
        for m, xs, ys in runs:
            assert oracle_rows.check_product(ys[t], xs[t], W) == sp["rows"], (sp["name"], m)


# ---- up to 4 activation rows: the product on the vector units ----

def _few_row_specs():
    """More chunks (1,350) than the GPU holds workgroups, so waves take
    several chunks in turn; chunks of 1, 2 and 8 rows (the last one 3 rows);
    int8 and e4m3; 2, 3 and 11 blocks per row."""
    specs = [synth.random_int8_tensor(1024, 512, 1.7, 710, 512)]
    e = synth.e4m3_matrix(rows=600, cols=768)[0]
    e["chunk_symbols"] = 768 * 2
    specs.append(e)
    specs.append(synth.random_int8_tensor(203, 2816, 2.6, 711, 2816 * 8))
    return specs


def test_few_rows_one_hot_return_the_oracle_weights_exactly(E):
    import torch
    specs = _few_row_specs()
    b, p, blob, scales = _setup(E, specs)
    assert p.n_chunks == 1024 + 300 + 26
    W = _oracle_weights(b, specs)
    rng = np.random.default_rng(31)
    for m in (1, 2, 3, 4):
        _say(f"few rows, one-hot, m={m}")
        xs, ys, hit = [], [], []
        for sp in specs:
            c = rng.choice(sp["cols"], m, replace=False)
            x = np.zeros((m, sp["cols"]), np.float32)
            x[np.arange(m), c] = 1.0
            xs.append(torch.from_numpy(x).to(torch.bfloat16).cuda())
            # one row more than m: it must stay untouched
            ys.append(torch.full((m + 1, sp["rows"]), float("nan"), dtype=torch.float32,
                                 device="cuda"))
            hit.append(c)
        status = torch.full((p.n_chunks,), -7, dtype=torch.int32, device="cuda")
        E.decode_gemm(p, blob, scales, xs, [y[:m] for y in ys], status)
        torch.cuda.synchronize()
        assert (status.cpu().numpy() == 0).all()
        for t in range(len(specs)):
            y = ys[t].cpu().numpy()
            want = _f32(W[t][:, hit[t]]).T
            assert np.array_equal(y[:m].view(np.uint32), want.view(np.uint32)), (t, m)
            assert np.isnan(y[m]).all(), (t, m)


def test_few_rows_random_within_the_accumulation_bound(E):
    specs = _few_row_specs()
    b, p, blob, scales = _setup(E, specs)
    W = _oracle_weights(b, specs)
    rng = np.random.default_rng(32)
    for m, pad_x, pad_y in ((1, 0, 0), (2, 4, 1), (3, 12, 0), (4, 0, 5)):
        _say(f"few rows, random, m={m}, padded strides {pad_x}/{pad_y}")
        xs = [_f32(rng.integers(0, 65536, (m, sp["cols"]), dtype=np.uint64).astype(np.uint16)
                   & np.uint16(0xBFFF)) for sp in specs]  # finite bf16 values, |x| < 4
        ys = _run(E, p, blob, scales, xs, specs, pad_x, pad_y)
        for t, sp in enumerate(specs):
            assert oracle_rows.check_product(ys[t][:, :sp["rows"]], xs[t], W[t]) == sp["rows"]
            if pad_y:
                assert np.isnan(ys[t][:, sp["rows"]:]).all()


def test_few_rows_report_the_decodes_chunk_status(E):
    """Corrupt chunks: the product reports, chunk by chunk, the status the
    decode reports for the same bytes (m = 1 and 3; the vector-unit kernel
    shares the decode's word ring and end check)."""
    import torch
    specs = _few_row_specs()
    b = E.encode_batch(specs)
    rng = np.random.default_rng(33)
    blob_h = b.blob.copy()
    bad = rng.choice(b.chunks.size, 40, replace=False)
    for c in bad:  # flip bytes inside the chunk's word stream
        ch = b.chunks[c]
        lo = int(ch["byte_offset"]) + 256
        hi = lo + 2 * int(ch["n_words"])
        pos = rng.integers(lo, hi, 3)
        blob_h[pos] ^= np.uint8(0x5A)
    p = E.plan(b.tensors, b.freq, b.chunks, b.blob.size)
    blob = torch.from_numpy(blob_h).cuda()
    scales = torch.from_numpy(np.concatenate([sp["scales"] for sp in specs])).cuda()
    out = torch.empty(p.out_elems, dtype=torch.int16, device="cuda")
    want = torch.full((p.n_chunks,), -7, dtype=torch.int32, device="cuda")
    E.decode(p, blob, out, E.OUT_BF16, scales, want)
    torch.cuda.synchronize()
    want = want.cpu().numpy()
    assert (want != 0).sum() >= 20 and (want[np.setdiff1d(np.arange(p.n_chunks), bad)] == 0).all()
    for m in (1, 3):
        _say(f"few rows, corrupt chunks, m={m}")
        xs = [torch.ones(m, sp["cols"], dtype=torch.bfloat16, device="cuda") for sp in specs]
        ys = [torch.empty(m, sp["rows"], dtype=torch.float32, device="cuda") for sp in specs]
        got = torch.full((p.n_chunks,), -7, dtype=torch.int32, device="cuda")
        E.decode_gemm(p, blob, scales, xs, ys, got)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), want), m


def _bf16_setup(E, rows, cols, C):
    import torch
    w = synth.bf16_weights(rows, cols)[0]["bf16"]
    e, sm = oracle.bf16_split(w)
    spec = dict(kind=oracle.KIND_BF16EXP, rows=rows, cols=cols, symbols=e, chunk_symbols=C)
    b = E.encode_batch([spec])
    p = E.plan(b.tensors, b.freq, b.chunks, b.blob.size)
    # the oracle's own decode of the exponent stream, merged, is the source
    ch = b.chunks
    desc = np.stack([ch["n_symbols"], ch["n_words"], ch["byte_offset"], ch["elem_offset"]],
                    axis=1).astype(np.uint64)
    sym, st = oracle.decode_tensor(b.blob, desc, b.freq[0], rows * cols)
    assert (st == 0).all()
    assert np.array_equal(oracle.bf16_merge(sym, sm), w)
    return (p, torch.from_numpy(b.blob).cuda(), torch.from_numpy(sm).cuda(),
            w.reshape(rows, cols))


def _run_split(E, p, blob, sm, x, rows):
    import torch
    xd = torch.from_numpy(x).to(torch.bfloat16).cuda()
    y = torch.full((x.shape[0], rows), float("nan"), dtype=torch.float32, device="cuda")
    status = torch.full((p.n_chunks,), -7, dtype=torch.int32, device="cuda")
    E.decode_gemm_bf16_split(p, blob, sm, [xd], [y], status)
    torch.cuda.synchronize()
    assert (status.cpu().numpy() == 0).all()
    return y.cpu().numpy()


@pytest.mark.parametrize("rows,blocks,chunk_rows,ms", [
    (72, 3, 4, (1, 2, 16, 33)),  # 3 blocks per row; 18 chunks: a partial second workgroup
    (40, 5, 3, (3, 16)),         # 5 and 7 blocks per row: the sign+mantissa prefetch's
    (35, 7, 2, (4, 7, 64)),      # unrolled loop plus a remainder; the last chunk short
])
def test_bf16_split_one_hot_returns_the_source_weights(E, rows, blocks, chunk_rows, ms):
    cols = 256 * blocks
    p, blob, sm, w = _bf16_setup(E, rows, cols, cols * chunk_rows)
    rng = np.random.default_rng(11)
    for m in ms:
        _say(f"bf16 split one-hot, {rows}x{cols}, {chunk_rows}-row chunks, m={m}")
        c = rng.choice(cols, m, replace=False)
        x = np.zeros((m, cols), np.float32)
        x[np.arange(m), c] = 1.0
        y = _run_split(E, p, blob, sm, x, rows)
        assert np.array_equal(y.view(np.uint32), _f32(w[:, c]).T.view(np.uint32)), m


def test_bf16_split_over_more_tensors_than_one_launch_takes(E):
    """18 exponent-stream tensors (a launch takes 16), 1 to 7 blocks per row and
    1 to 4 rows per chunk, reordered by the launcher (longest rows first): with
    one-hot activations every output is a source bf16 weight, bit for bit."""
    import torch
    rng = np.random.default_rng(23)
    specs, ws, sms = [], [], []
    for i in range(18):
        cols = 256 * int(rng.integers(1, 8))
        rows = int(rng.integers(2, 30))
        w = rng.integers(0, 1 << 16, size=rows * cols, dtype=np.uint64).astype(np.uint16)
        w[(w & 0x7F80) == 0x7F80] &= 0xBFFF  # finite weights, so that 1.0 * w is w
        w[w == 0x8000] = 0  # a -0 weight would come out +0 (+0 + -0 = +0 in the sums)
        e, sm = oracle.bf16_split(w)
        specs.append(dict(kind=oracle.KIND_BF16EXP, rows=rows, cols=cols, symbols=e,
                          chunk_symbols=cols * int(rng.integers(1, 5))))
        ws.append(w.reshape(rows, cols))
        sms.append(sm)
    b = E.encode_batch(specs)
    p = E.plan(b.tensors, b.freq, b.chunks, b.blob.size)
    blob = torch.from_numpy(b.blob).cuda()
    sm_all = torch.from_numpy(np.concatenate(sms)).cuda()
    for m in (9, 3):  # (more than 16 tensors: the matrix cores also for m <= 4)
        _split_one_hot_many(E, p, blob, sm_all, specs, ws, rng, m)
    p.close()


def _split_one_hot_many(E, p, blob, sm_all, specs, ws, rng, m):
    import torch
    xs, ys, hit = [], [], []
    for sp in specs:
        c = rng.choice(sp["cols"], m, replace=False)
        x = np.zeros((m, sp["cols"]), np.float32)
        x[np.arange(m), c] = 1.0
        xs.append(torch.from_numpy(x).to(torch.bfloat16).cuda())
        ys.append(torch.full((m, sp["rows"]), float("nan"), dtype=torch.float32, device="cuda"))
        hit.append(c)
    status = torch.full((p.n_chunks,), -7, dtype=torch.int32, device="cuda")
    _say(f"bf16 split, 18 tensors, one-hot, m={m}")
    E.decode_gemm_bf16_split(p, blob, sm_all, xs, ys, status)
    torch.cuda.synchronize()
    assert (status.cpu().numpy() == 0).all()
    for t in range(len(specs)):
        want = _f32(ws[t][:, hit[t]]).T
        assert np.array_equal(ys[t].cpu().numpy().view(np.uint32), want.view(np.uint32)), (t, m)


def test_bf16_split_8192x8192_within_the_accumulation_bound(E):
    rows = cols = 8192
    p, blob, sm, w = _bf16_setup(E, rows, cols, 65536)
    rng = np.random.default_rng(12)
    for m in (16, 1):  # matrix cores; the vector-unit product (two chunks per wave)
        _say(f"bf16 split 8192x8192, 8-row chunks, m = {m}, every row")
        x = (rng.standard_normal((m, cols)) * 0.5).astype(np.float32)
        x = _f32((x.view(np.uint32) >> 16).astype(np.uint16))
        y = _run_split(E, p, blob, sm, x, rows)
        assert oracle_rows.check_product(y, x, w) == rows  # every row


def test_bf16_split_rejects_code_tensors(E):
    import torch
    specs = _mixed_specs()[:1]
    b, p, blob, scales = _setup(E, specs)
    x = torch.zeros(2, specs[0]["cols"], dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(2, specs[0]["rows"], dtype=torch.float32, device="cuda")
    sm = torch.zeros(specs[0]["rows"] * specs[0]["cols"], dtype=torch.uint8, device="cuda")
    with pytest.raises(E.EntqError):
        E.decode_gemm_bf16_split(p, blob, sm, [x], [y])
