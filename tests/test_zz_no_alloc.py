"""GPU test of entq_decode_gemm_static, the fused decode + product that keeps
its packed activations in the library's static device scratch instead of a
caller's workspace. Through the C ABI, its results must equal
entq_decode_gemm's (with a workspace of its own) bit for bit, on two calls in
a row -- the second with a smaller plan and fewer activation rows, over what
the first call left in the scratch -- and a request whose packed activations
exceed the scratch must be refused before any launch."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-no-alloc] {msg}", flush=True)


@pytest.fixture(scope="module")
def E():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import entropy_coded_weight_amd as E
    E.lib()
    return E


def _setup(E, specs):
    import torch
    b = E.encode_batch(specs, n_threads=4)
    p = E.plan(b.tensors, b.freq, b.chunks, b.blob.size)
    blob = torch.from_numpy(b.blob).cuda()
    scales = torch.from_numpy(np.concatenate([sp["scales"] for sp in specs])).cuda()
    return p, blob, scales


def _activations(specs, m, seed):
    import torch
    rng = np.random.default_rng(seed)
    xs = []
    for sp in specs:
        bits = rng.integers(0, 65536, (m, sp["cols"]), dtype=np.uint64).astype(np.uint16)
        bits &= np.uint16(0xBFFF)  # finite bf16 values, |x| < 4
        xs.append(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda())
    return xs


def _both(E, p, blob, scales, specs, xs):
    """(static-scratch results, workspace results) as host float32 bit arrays."""
    import torch
    m = xs[0].shape[0]
    res = []
    for path in ("static", "workspace"):
        ys = [torch.full((m, sp["rows"]), float("nan"), dtype=torch.float32, device="cuda")
              for sp in specs]
        status = torch.full((p.n_chunks,), -7, dtype=torch.int32, device="cuda")
        if path == "static":
            E.decode_gemm_static(p, blob, scales, xs, ys, status)
        else:
            n = int(E.lib().entq_decode_gemm_workspace_bytes(p.handle, m))
            raw = torch.full((n + 256,), 0xA5, dtype=torch.uint8, device="cuda")
            shift = (-raw.data_ptr()) % 256
            E.decode_gemm(p, blob, scales, xs, ys, status, workspace=raw[shift:shift + n])
        torch.cuda.synchronize()
        assert (status.cpu().numpy() == 0).all(), path
        res.append([y.cpu().numpy().view(np.uint32) for y in ys])
    return res


def test_static_scratch_matches_the_workspace_path_on_two_calls(E):
    # call 1: three tensors (int8 and e4m3, 2, 3 and 11 blocks per row), m = 40
    specs1 = [synth.random_int8_tensor(48, 512, 1.4, 900, 512 * 4)]
    e = synth.e4m3_matrix(rows=40, cols=768)[0]
    e["chunk_symbols"] = 768 * 3
    specs1.append(e)
    specs1.append(synth.random_int8_tensor(100, 2816, 2.3, 902, 2816))
    p1, blob1, sc1 = _setup(E, specs1)
    _say("call 1: 3 tensors, m=40")
    got, want = _both(E, p1, blob1, sc1, specs1, _activations(specs1, 40, 11))
    for t in range(len(specs1)):
        assert np.array_equal(got[t], want[t]), t
        assert not np.isnan(got[t].view(np.float32)).any()
    # call 2: a smaller plan and fewer rows, over call 1's scratch contents
    specs2 = [synth.random_int8_tensor(16, 256, 3.0, 903, 256 * 2)]
    p2, blob2, sc2 = _setup(E, specs2)
    _say("call 2: 1 tensor, m=17")
    got, want = _both(E, p2, blob2, sc2, specs2, _activations(specs2, 17, 12))
    assert np.array_equal(got[0], want[0])
    assert not np.isnan(got[0].view(np.float32)).any()


def test_request_beyond_the_scratch_is_refused(E):
    import torch
    # 2 bytes x 64 rows x 131,328 columns > 16 MiB of packed activations
    cols = 131328
    specs = [synth.random_int8_tensor(1, cols, 2.0, 904, cols)]
    p, blob, sc = _setup(E, specs)
    assert int(E.lib().entq_decode_gemm_workspace_bytes(p.handle, 64)) > E.GEMM_STATIC_SCRATCH_BYTES
    xs = [torch.zeros(64, cols, dtype=torch.bfloat16, device="cuda")]
    ys = [torch.zeros(64, 1, dtype=torch.float32, device="cuda")]
    _say("request beyond the scratch")
    with pytest.raises(E.EntqError) as ei:
        E.decode_gemm_static(p, blob, sc, xs, ys)
    assert ei.value.status == E.ETOOLARGE
    # 32 rows fit (2 x 32 x 131,328 bytes < 16 MiB) and agree with the workspace path
    got, want = _both(E, p, blob, sc, specs, _activations(specs, 32, 13))
    assert np.array_equal(got[0], want[0])
