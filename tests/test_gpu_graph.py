"""GPU test: the decode and the allocation-free fused product captured into a
HIP graph (torch's CUDAGraph over its capture stream) and replayed several
times, with eager work and synchronisations between the replays. Every replay
must equal the eager result bit for bit, and the eager result the oracle's
dequantisation of the source codes: the calls record no memset and allocate
nothing while captured, and a replay reads its buffers as they are when it
runs (new activations between replays give the new products)."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-graph] {msg}", flush=True)


@pytest.fixture(scope="module")
def E():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import entropy_coded_weight_amd as E
    E.lib()
    return E


def _specs(fused_only=False):
    specs = [synth.random_int8_tensor(64, 1024, 2.0, 950, 4096),
             dict(synth.e4m3_matrix(32, 512)[0], chunk_symbols=4096)]
    if not fused_only:  # rows of 333 columns: the element-wise kernel
        specs.append(synth.random_int8_tensor(7, 333, 1.5, 951, 960))
    return specs


def _setup(E, specs):
    import torch
    b = E.encode_batch(specs, n_threads=4)
    p = E.plan(b.tensors, b.freq, b.chunks, b.blob.size)
    blob = torch.from_numpy(b.blob).cuda()
    scales = torch.from_numpy(np.concatenate([sp["scales"] for sp in specs])).cuda()
    return b, p, blob, scales


def test_decode_graph_replays(E):
    import torch
    specs = _specs()
    b, p, blob, scales = _setup(E, specs)
    want = np.concatenate([oracle.dequant_tensor(sp["symbols"], sp["rows"], sp["cols"], sp["kind"],
                                                 sp["scales"]) for sp in specs])
    out = torch.full((p.out_elems,), 0x5A5A, dtype=torch.int16, device="cuda")
    status = torch.full((p.n_chunks,), -7, dtype=torch.int32, device="cuda")
    _say("eager decode")
    E.decode(p, blob, out, E.OUT_BF16, scales, status)
    torch.cuda.synchronize()
    eager = out.cpu().numpy().view(np.uint16).copy()
    np.testing.assert_array_equal(eager, want)
    assert (status.cpu().numpy() == 0).all()
    g = torch.cuda.CUDAGraph()
    _say("capture")
    with torch.cuda.graph(g):
        E.decode(p, blob, out, E.OUT_BF16, scales, status)
    for r in range(3):
        out.fill_(0x5A5A)  # eager work between replays
        status.fill_(-7)
        torch.cuda.synchronize()
        _say(f"replay {r}")
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy().view(np.uint16), eager)
        assert (status.cpu().numpy() == 0).all()
    del g
    p.close()


@pytest.mark.parametrize("m", [16, 1])  # matrix cores; the vector-unit product
def test_static_fused_product_graph_replays(E, m):
    import torch
    specs = _specs(fused_only=True)
    b, p, blob, scales = _setup(E, specs)
    rng = np.random.default_rng(3)

    def fill_activations(xs):
        for x in xs:
            bits = rng.integers(0, 65536, tuple(x.shape), dtype=np.uint64).astype(np.uint16)
            bits &= np.uint16(0xBFFF)  # finite bf16 values
            x.copy_(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda())

    xs = [torch.empty(m, sp["cols"], dtype=torch.bfloat16, device="cuda") for sp in specs]
    ys = [torch.empty(m, sp["rows"], dtype=torch.float32, device="cuda") for sp in specs]
    ye = [torch.empty_like(y) for y in ys]
    status = torch.full((p.n_chunks,), -7, dtype=torch.int32, device="cuda")
    fill_activations(xs)
    _say(f"eager static fused product, m={m}")
    E.decode_gemm_static(p, blob, scales, xs, ye, status)  # also looks the scratch up once
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    _say("capture")
    with torch.cuda.graph(g):
        E.decode_gemm_static(p, blob, scales, xs, ys, status)
    for r in range(3):
        if r:
            fill_activations(xs)  # new inputs in the same buffers
            E.decode_gemm_static(p, blob, scales, xs, ye, status)  # eager reference
        for y in ys:
            y.fill_(float("nan"))
        status.fill_(-7)
        torch.cuda.synchronize()
        want = [y.cpu().numpy().view(np.uint32).copy() for y in ye]
        _say(f"replay {r}")
        g.replay()
        torch.cuda.synchronize()
        for t in range(len(specs)):
            assert np.array_equal(ys[t].cpu().numpy().view(np.uint32), want[t]), (r, t)
        assert (status.cpu().numpy() == 0).all()
    del g
    p.close()


def test_tiled_fused_product_graph_replays(E):
    """entq_decode_gemm_tiles with its workspace given (activation copy,
    product and the column chunks' reduction: three kernels, no memset)
    captured and replayed, new activations between replays."""
    import torch
    specs = _specs(fused_only=True)
    C = {0: 256, 1: 512}
    tiled = [dict(sp, symbols=E.tile_order(sp["symbols"], sp["rows"], sp["cols"], C[i]),
                  chunk_symbols=16 * C[i], kind=sp["kind"] | E.LAYOUT_TILES)
             for i, sp in enumerate(specs)]
    b, p, blob, scales = _setup(E, tiled)
    rng = np.random.default_rng(4)
    m = 24
    n = int(E.lib().entq_decode_gemm_tiles_workspace_bytes(p.handle, m))
    raw = torch.empty(n + 256, dtype=torch.uint8, device="cuda")
    ws = raw[(-raw.data_ptr()) % 256:][:n]

    def fill_activations(xs):
        for x in xs:
            bits = rng.integers(0, 65536, tuple(x.shape), dtype=np.uint64).astype(np.uint16)
            bits &= np.uint16(0xBFFF)  # finite bf16 values
            x.copy_(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda())

    xs = [torch.empty(m, sp["cols"], dtype=torch.bfloat16, device="cuda") for sp in specs]
    ys = [torch.empty(m, sp["rows"], dtype=torch.float32, device="cuda") for sp in specs]
    ye = [torch.empty_like(y) for y in ys]
    status = torch.full((p.n_chunks,), -7, dtype=torch.int32, device="cuda")
    fill_activations(xs)
    _say("eager tiled product")
    E.decode_gemm_tiles(p, blob, scales, xs, ye, status, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    _say("capture")
    with torch.cuda.graph(g):
        E.decode_gemm_tiles(p, blob, scales, xs, ys, status, workspace=ws)
    for r in range(3):
        if r:
            fill_activations(xs)
            E.decode_gemm_tiles(p, blob, scales, xs, ye, status, workspace=ws)
        for y in ys:
            y.fill_(float("nan"))
        status.fill_(-7)
        torch.cuda.synchronize()
        want = [y.cpu().numpy().view(np.uint32).copy() for y in ye]
        _say(f"replay {r}")
        g.replay()
        torch.cuda.synchronize()
        for t in range(len(specs)):
            assert np.array_equal(ys[t].cpu().numpy().view(np.uint32), want[t]), (r, t)
        assert (status.cpu().numpy() == 0).all()
    del g
    p.close()
