"""GPU tests of the decode/compute overlap (LayerPipeline): the overlapped
schedule (decode of layer l+1 on its own stream during layer l's GEMMs,
two layer buffers) must give exactly the outputs of the serial schedule,
pass after pass, and those outputs must match an fp32 product of the
oracle's decoded weights."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

N_LAYERS = 5
SHAPES = [("q", 1024, 1024), ("k", 256, 1024), ("down", 1024, 2816)]


def _say(msg):
    print(f"[gpu-overlap] {msg}", flush=True)


@pytest.fixture(scope="module")
def model():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import entropy_coded_weight_amd as E
    from entropy_coded_weight_amd.layer_pipeline import LayerPipeline
    dev = torch.device("cuda", 0)
    layers, ref_w = [], []
    for layer in range(N_LAYERS):
        specs = [synth.random_int8_tensor(r, c, 0.9 + 0.4 * t + 0.1 * layer, 500 + 10 * layer + t,
                                          4096) for t, (n, r, c) in enumerate(SHAPES)]
        b = E.encode_batch(specs)
        p = E.plan(b.tensors, b.freq, b.chunks, b.blob.size)
        scales = np.concatenate([sp["scales"] for sp in specs])
        layers.append((p, torch.from_numpy(b.blob).to(dev), torch.from_numpy(scales).to(dev)))
        # the oracle's bf16 weights of this layer, from the same container
        ws = []
        for t, sp in enumerate(specs):
            ch = b.chunks[b.chunks["tensor"] == t]
            desc = np.stack([ch["n_symbols"], ch["n_words"], ch["byte_offset"], ch["elem_offset"]],
                            axis=1).astype(np.uint64)
            sym, st = oracle.decode_tensor(b.blob, desc, b.freq[t], sp["rows"] * sp["cols"])
            assert (st == 0).all()
            ws.append(oracle.dequant_tensor(sym, sp["rows"], sp["cols"], sp["kind"], sp["scales"]))
        ref_w.append(ws)
    out_elems = sum(r * c for _, r, c in SHAPES)
    pipe = LayerPipeline(layers, out_elems, dev)
    return E, pipe, ref_w


def _consumer(T, seed):
    import torch
    gen = torch.Generator().manual_seed(seed)
    X = (torch.randn(T, 1024, generator=gen) * 0.5).to(torch.bfloat16).cuda()
    H = (torch.randn(T, 2816, generator=gen) * 0.5).to(torch.bfloat16).cuda()
    outs = [{n: torch.full((T, r), float("nan"), dtype=torch.bfloat16, device="cuda")
             for n, r, c in SHAPES} for _ in range(N_LAYERS)]
    offs = np.concatenate([[0], np.cumsum([r * c for _, r, c in SHAPES])])

    def consume(layer, W):
        for t, (n, r, c) in enumerate(SHAPES):
            w = W[int(offs[t]):int(offs[t]) + r * c].view(r, c)
            torch.mm(H if n == "down" else X, w.t(), out=outs[layer][n])

    return X, H, outs, consume


def _host(outs):
    return [{n: o.float().cpu().numpy() for n, o in d.items()} for d in outs]


def test_overlapped_equals_serial(model):
    import torch
    E, pipe, _ = model
    for T in (1, 33, 256):
        _say(f"T={T}: serial vs overlapped, {N_LAYERS} layers")
        _, _, s_outs, s_consume = _consumer(T, 1)
        pipe.run_serial(s_consume)
        torch.cuda.synchronize()
        _, _, o_outs, o_consume = _consumer(T, 1)
        pipe.run_overlapped(o_consume)
        torch.cuda.synchronize()
        a, b = _host(s_outs), _host(o_outs)
        for layer in range(N_LAYERS):
            for n in a[layer]:
                assert not np.isnan(b[layer][n]).any(), (T, layer, n)
                assert np.array_equal(a[layer][n], b[layer][n]), (T, layer, n)


def test_back_to_back_passes_without_host_sync(model):
    import torch
    E, pipe, _ = model
    _, _, ref_outs, ref_consume = _consumer(64, 2)
    pipe.run_serial(ref_consume)
    torch.cuda.synchronize()
    ref = _host(ref_outs)
    passes = [_consumer(64, 2) for _ in range(3)]
    for _, _, _, consume in passes:   # enqueued back to back: buffer reuse across passes
        pipe.run_overlapped(consume)
    torch.cuda.synchronize()
    for _, _, outs, _ in passes:
        got = _host(outs)
        for layer in range(N_LAYERS):
            for n in got[layer]:
                assert np.array_equal(got[layer][n], ref[layer][n]), (layer, n)


def test_outputs_match_fp32_product_of_oracle_weights(model):
    import torch
    E, pipe, ref_w = model
    X, H, outs, consume = _consumer(48, 3)
    pipe.run_overlapped(consume)
    torch.cuda.synchronize()
    got = _host(outs)
    xf, hf = X.float().cpu().numpy(), H.float().cpu().numpy()
    for layer in range(N_LAYERS):
        for t, (n, r, c) in enumerate(SHAPES):
            w = (ref_w[layer][t].astype(np.uint32) << 16).view(np.float32).reshape(r, c)
            ref = (hf if n == "down" else xf).astype(np.float64) @ w.T.astype(np.float64)
            # bf16 output of an fp32-accumulated product: a few bf16 ulps
            tol = 2.0 ** -7 * np.abs(ref) + 1e-3 * np.abs(ref).max()
            assert (np.abs(got[layer][n] - ref) <= tol).all(), (layer, n)
