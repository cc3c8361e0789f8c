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


def test_llama2_70b_layer_sampled_rows(E):
    import torch
    _say("70B-shaped layer 0 with row-aligned chunks, m = 16")
    specs = synth.llama2_70b_layer(0)
    for sp in specs:
        sp["chunk_symbols"] = sp["cols"] * max(1, 65536 // sp["cols"])
    b, p, blob, scales = _setup(E, specs)
    rng = np.random.default_rng(7)
    xs = [(rng.standard_normal((16, sp["cols"])) * 0.5).astype(np.float32) for sp in specs]
    xs = [_f32((x.view(np.uint32) >> 16).astype(np.uint16)) for x in xs]  # bf16 values
    ys = _run(E, p, blob, scales, xs, specs)
    for t, sp in enumerate(specs):
        rows = sorted(set([0, sp["rows"] - 1] + list(rng.integers(0, sp["rows"], 6))))
        W = oracle_rows.rows_from_oracle(b.blob, b.chunks[b.chunks["tensor"] == t], b.freq[t],
                                         sp, rows)
        for r in rows:
            w = _f32(W[r]).astype(np.float64)
            x = xs[t].astype(np.float64)
            ref = x @ w
            bound = sp["cols"] * 2.0 ** -24 * (np.abs(x) @ np.abs(w))
            assert (np.abs(ys[t][:, r] - ref) <= bound).all(), (t, r)


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
    (72, 3, 4, (1, 16, 33)),   # 3 blocks per row; 18 chunks: a partial second workgroup
    (40, 5, 3, (16,)),         # 5 and 7 blocks per row: the sign+mantissa prefetch's
    (35, 7, 2, (7, 64)),       # unrolled loop plus a remainder; the last chunk short
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


def test_bf16_split_8192x8192_within_the_accumulation_bound(E):
    _say("bf16 split 8192x8192, 8-row chunks, m = 16")
    rows = cols = 8192
    p, blob, sm, w = _bf16_setup(E, rows, cols, 65536)
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((16, cols)) * 0.5).astype(np.float32)
    x = _f32((x.view(np.uint32) >> 16).astype(np.uint16))
    y = _run_split(E, p, blob, sm, x, rows)
    picks = sorted(set([0, rows - 1] + [int(v) for v in rng.integers(0, rows, 30)]))
    wf = _f32(w[picks]).astype(np.float64)
    ref = x.astype(np.float64) @ wf.T
    bound = cols * 2.0 ** -24 * (np.abs(x.astype(np.float64)) @ np.abs(wf).T)
    assert (np.abs(y[:, picks] - ref) <= bound).all()


def test_bf16_split_rejects_code_tensors(E):
    import torch
    specs = _mixed_specs()[:1]
    b, p, blob, scales = _setup(E, specs)
    x = torch.zeros(2, specs[0]["cols"], dtype=torch.bfloat16, device="cuda")
    y = torch.zeros(2, specs[0]["rows"], dtype=torch.float32, device="cuda")
    sm = torch.zeros(specs[0]["rows"] * specs[0]["cols"], dtype=torch.uint8, device="cuda")
    with pytest.raises(E.EntqError):
        E.decode_gemm_bf16_split(p, blob, sm, [x], [y])
