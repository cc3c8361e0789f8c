"""GPU parity of a single large tensor decoded on its own: the LLaMA-2-70B
output projection (32,000 x 8,192 int8 codes), through the bf16 decode and
through the fused decode + product (logits for 16 activation rows).
Expected values: the oracle's decode + dequant of every element, and the
fp64 product with those weights for every output row."""
import numpy as np
import pytest

import oracle_rows
import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-lm-head] {msg}", flush=True)


def _f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.fixture(scope="module")
def E():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import entropy_coded_weight_amd as E
    E.lib()
    return E


def _container(E, chunk_symbols):
    import torch
    specs = synth.llama2_70b_lm_head(chunk_symbols=chunk_symbols)
    b = E.encode_batch(specs)
    p = E.plan(b.tensors, b.freq, b.chunks, b.blob.size)
    return specs, b, p, torch.from_numpy(b.blob).cuda(), torch.from_numpy(specs[0]["scales"]).cuda()


def test_lm_head_bf16_decode(E):
    import torch
    _say("LM head 32000 x 8192, 65,536-symbol chunks, bf16 decode, every element")
    specs, b, p, blob, scales = _container(E, 65536)
    sp = specs[0]
    out = torch.empty(sp["rows"] * sp["cols"], dtype=torch.int16, device="cuda")
    status = torch.full((p.n_chunks,), -7, dtype=torch.int32, device="cuda")
    E.decode(p, blob, out, E.OUT_BF16, scales, status)
    torch.cuda.synchronize()
    assert (status.cpu().numpy() == 0).all()
    got = out.cpu().numpy().view(np.uint16).reshape(sp["rows"], sp["cols"])
    want = oracle_rows.tensor_from_oracle(b.blob, b.chunks, b.freq[0], sp)
    np.testing.assert_array_equal(got, want)


def test_lm_head_fused_logits(E):
    import torch
    _say("LM head, row-aligned 32,768-symbol chunks, fused logits for 16 rows, every row")
    specs, b, p, blob, scales = _container(E, 32768)
    sp = specs[0]
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((16, sp["cols"])) * 0.5).astype(np.float32)
    x = _f32((x.view(np.uint32) >> 16).astype(np.uint16))  # bf16 values
    xd = torch.from_numpy(x).to(torch.bfloat16).cuda()
    y = torch.full((16, sp["rows"]), float("nan"), dtype=torch.float32, device="cuda")
    E.decode_gemm(p, blob, scales, [xd], [y])
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    assert not np.isnan(got).any()
    W = oracle_rows.tensor_from_oracle(b.blob, b.chunks, b.freq[0], sp)
    assert oracle_rows.check_product(got, x, W) == sp["rows"]
