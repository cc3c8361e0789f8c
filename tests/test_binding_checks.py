"""CPU checks of the binding's argument validation: every decode entry point
refuses, before any library call, a buffer the kernels could overrun or
could not address (too small, wrong element size or dtype, another device,
not contiguous). The plan here is a stand-in with the fields the checks
read and a null handle, so nothing reaches the library or a GPU."""
import ctypes
import os

import numpy as np
import pytest
import torch


@pytest.fixture(scope="module")
def E():
    import entropy_coded_weight_amd as E
    if not os.path.exists(E.LIB_PATH):
        from entropy_coded_weight_amd import build
        build.build()
    return E


@pytest.fixture()
def P(E):
    """A 2-tensor plan: 4 x 256 and 3 x 512 int8 codes, 5 chunks, 900-byte blob."""
    p = object.__new__(E.Plan)
    p.workspace = torch.empty(0, dtype=torch.uint8)
    p._h = ctypes.c_void_p()
    p.n_tensors, p.n_chunks = 2, 5
    p.tensors = np.zeros(2, E.TENSOR_DESC)
    p.tensors[0] = (E.KIND_INT8, 4, 256, 256, 1024, 0, 0)
    p.tensors[1] = (E.KIND_INT8, 3, 512, 512, 1536, 1024, 4)
    p.blob_bytes, p.out_elems, p.scale_rows = 900, 2560, 7
    p.adaptive = False
    return p


def good(P):
    return dict(compressed=torch.zeros(900, dtype=torch.uint8),
                out=torch.zeros(2560, dtype=torch.int16),
                scales=torch.ones(7, dtype=torch.float32),
                chunk_status=torch.zeros(5, dtype=torch.int32))


def _rejects(E, fn, *a, match=None, **k):
    with pytest.raises(E.EntqError, match=match) as ei:
        fn(*a, **k)
    assert ei.value.status == E.EINVAL


@pytest.mark.parametrize("field,bad,match", [
    ("compressed", torch.zeros(899, dtype=torch.uint8), "compressed holds 899"),
    ("compressed", np.zeros(900, np.uint8), "torch tensor"),
    ("out", torch.zeros(2559, dtype=torch.int16), "out holds 2559"),
    ("out", torch.zeros(2560, dtype=torch.uint8), "1-byte elements, expected 2"),
    ("out", torch.zeros(2560, dtype=torch.float32), "4-byte elements, expected 2"),
    ("out", torch.zeros(2560 * 2, dtype=torch.int16)[::2], "not contiguous"),
    ("scales", torch.ones(6, dtype=torch.float32), "scales holds 6"),
    ("scales", torch.ones(7, dtype=torch.float64), "dtype torch.float64"),
    ("scales", None, "scales are required"),
    ("chunk_status", torch.zeros(4, dtype=torch.int32), "chunk_status holds 4"),
    ("chunk_status", torch.zeros(5, dtype=torch.int64), "dtype torch.int64"),
    ("out", torch.zeros(2560, dtype=torch.int16, device="meta"), "is on meta"),
])
def test_decode_bf16_refuses(E, P, field, bad, match):
    a = good(P)
    a[field] = bad
    _rejects(E, E.decode, P, a["compressed"], a["out"], E.OUT_BF16, a["scales"],
             a["chunk_status"], stream=0, match=match)


def test_decode_codes_checks_one_byte_outputs(E, P):
    a = good(P)
    _rejects(E, E.decode, P, a["compressed"], a["out"], E.OUT_CODES, None, None, stream=0,
             match="2-byte elements, expected 1")
    _rejects(E, E.decode, P, a["compressed"], torch.zeros(2559, dtype=torch.uint8),
             E.OUT_CODES, None, None, stream=0, match="out holds 2559")
    _rejects(E, E.decode, P, a["compressed"], a["out"], 7, None, None, stream=0,
             match="out_kind")


def test_blob_of_wider_elements_counts_bytes(E, P):
    a = good(P)
    # 225 int32 = 900 bytes passes the size check and fails only at the null plan
    with pytest.raises(E.EntqError) as ei:
        E.decode(P, torch.zeros(225, dtype=torch.int32), a["out"], E.OUT_BF16, a["scales"],
                 None, stream=0)
    assert "entq_decode" in str(ei.value)
    _rejects(E, E.decode, P, torch.zeros(224, dtype=torch.int32), a["out"], E.OUT_BF16,
             a["scales"], None, stream=0, match="compressed holds 224")


def test_split_decode_refuses(E, P):
    blob = torch.zeros(900, dtype=torch.uint8)
    sm = torch.zeros(2560, dtype=torch.uint8)
    out = torch.zeros(2560, dtype=torch.int16)
    _rejects(E, E.decode_bf16_split, P, blob, sm[:2559], out, stream=0, match="signmant holds")
    _rejects(E, E.decode_bf16_split, P, blob, sm.view(torch.int16), out, stream=0,
             match="2-byte elements, expected 1")
    _rejects(E, E.decode_bf16_split, P, blob, sm, out[:100], stream=0, match="out holds 100")
    _rejects(E, E.decode_bf16_split, P, blob[:10], sm, out, stream=0, match="exp_stream holds")
    _rejects(E, E.decode_bf16_split, P, blob, sm, out, torch.zeros(1, dtype=torch.int32),
             stream=0, match="chunk_status holds 1")


def _xy(m, shapes, xdt=torch.bfloat16, ydt=torch.float32):
    xs = [torch.zeros(m, c, dtype=xdt) for r, c in shapes]
    ys = [torch.zeros(m, r, dtype=ydt) for r, c in shapes]
    return xs, ys


def test_fused_refuses_mismatched_activations_and_results(E, P):
    blob = torch.zeros(900, dtype=torch.uint8)
    sc = torch.ones(7, dtype=torch.float32)
    xs, ys = _xy(3, [(4, 256), (3, 512)])
    _rejects(E, E.decode_gemm, P, blob, sc, xs[:1], ys[:1], stream=0, match="for 2 tensors")
    bad = [xs[0], torch.zeros(3, 511, dtype=torch.bfloat16)]
    _rejects(E, E.decode_gemm, P, blob, sc, bad, ys, stream=0, match="x\\[1\\] has 511 columns")
    bad = [ys[0], torch.zeros(3, 2, dtype=torch.float32)]
    _rejects(E, E.decode_gemm, P, blob, sc, xs, bad, stream=0, match="y\\[1\\] has 2 columns")
    bad = [xs[0], torch.zeros(2, 512, dtype=torch.bfloat16)]
    _rejects(E, E.decode_gemm, P, blob, sc, bad, ys, stream=0, match="expected")
    bad = [xs[0].float(), xs[1]]
    _rejects(E, E.decode_gemm, P, blob, sc, bad, ys, stream=0, match="expected")
    bad = [xs[0], torch.zeros(512, 3, dtype=torch.bfloat16).t()]
    _rejects(E, E.decode_gemm, P, blob, sc, bad, ys, stream=0, match="unit-stride")
    bad = [xs[0], torch.zeros(3, 512, dtype=torch.bfloat16, device="meta")]
    _rejects(E, E.decode_gemm, P, blob, sc, bad, ys, stream=0, match="must be a tensor on cpu")
    _rejects(E, E.decode_gemm, P, blob, sc[:6], xs, ys, stream=0, match="scales holds 6")
    _rejects(E, E.decode_gemm, P, blob[:899], sc, xs, ys, stream=0, match="compressed holds")
    sm = torch.zeros(2560, dtype=torch.uint8)
    _rejects(E, E.decode_gemm_bf16_split, P, blob, sm[:5], xs, ys, stream=0,
             match="signmant holds 5")


def test_tiled_product_refuses(E, P):
    blob = torch.zeros(900, dtype=torch.uint8)
    sc = torch.ones(7, dtype=torch.float32)
    xs, ys = _xy(3, [(4, 256), (3, 512)])
    _rejects(E, E.decode_gemm_tiles, P, blob, sc, xs[:1], ys[:1], stream=0,
             match="for 2 tensors")
    _rejects(E, E.decode_gemm_tiles, P, blob, sc[:6], xs, ys, stream=0, match="scales holds 6")
    _rejects(E, E.decode_gemm_tiles, P, blob[:899], sc, xs, ys, stream=0,
             match="compressed holds")
    _rejects(E, E.decode_gemm_tiles, P, blob, sc, xs, ys, torch.zeros(4, dtype=torch.int32),
             stream=0, match="chunk_status holds 4")
    _rejects(E, E.decode_gemm_tiles, P, blob, sc, xs, ys, stream=0,
             workspace=torch.zeros(16, dtype=torch.uint8, device="meta"), match="workspace is on")


def test_linear_refuses(E, P):
    from entropy_coded_weight_amd.linear import linear
    blob = torch.zeros(900, dtype=torch.uint8)
    sc = torch.ones(7, dtype=torch.float32)
    xs, ys = _xy(65, [(4, 256), (3, 512)])
    _rejects(E, linear, P, blob, sc, xs, ys, weights=torch.zeros(2559, dtype=torch.int16),
             stream=0, match="out holds 2559")
    _rejects(E, linear, P, blob, sc, xs, ys, weights=torch.zeros(2560, dtype=torch.uint8),
             stream=0, match="1-byte elements, expected 2")
    bad = [xs[0], torch.zeros(65, 511, dtype=torch.bfloat16)]
    _rejects(E, linear, P, blob, sc, bad, ys, stream=0, match="x\\[1\\] has 511 columns")
    _rejects(E, linear, P, blob, sc[:6], xs, ys, stream=0, match="scales holds 6")
    P.adaptive = True
    _rejects(E, linear, P, blob, sc, xs, ys, stream=0, match="per-tensor tables")
    P.adaptive = False
    P.tensors["kind"][1] = E.KIND_BF16EXP
    _rejects(E, linear, P, blob, sc, xs, ys, stream=0, match="exponent streams")
    # up to 64 rows the call is the fused one, with its checks
    xs, ys = _xy(64, [(4, 256), (3, 512)])
    P.tensors["kind"][1] = E.KIND_INT8
    _rejects(E, linear, P, blob[:899], sc, xs, ys, stream=0, match="compressed holds")


# ---- calls without a plan: the device encoder and the device tile order ----

def _cpu(n, dtype=torch.uint8):
    return torch.zeros(n, dtype=dtype)


@pytest.mark.parametrize("call", [
    lambda E: E.count_symbols_device(_cpu(64)),
    lambda E: E.encode_device(_cpu(4096), 4096, np.full(256, 16, np.uint16), _cpu(1 << 16),
                              _cpu(1, torch.int32)),
    lambda E: E.pack_device(_cpu(1 << 16), 4096, 4096, _cpu(1, torch.int32),
                            _cpu(1, torch.int64), _cpu(1 << 16)),
    lambda E: E.count_symbols_device_batch([(_cpu(64), _cpu(256, torch.int64))]),
    lambda E: E.pack_device_batch([(_cpu(1 << 16), 4096, 4096, _cpu(1, torch.int32),
                                    _cpu(1, torch.int64))], _cpu(1 << 16)),
    lambda E: E.encode_device_batch([(_cpu(4096), 4096, _cpu(256, torch.int16), _cpu(1 << 16),
                                      _cpu(1, torch.int32))]),
    lambda E: E.region_offsets_device(_cpu(4, torch.int32), _cpu(4, torch.int64),
                                      _cpu(1, torch.int64)),
    lambda E: E.count_chunks_device_batch([(_cpu(4096), 4096, _cpu(256, torch.int32))]),
    lambda E: E.build_freq_device(_cpu(256, torch.int64), _cpu(256, torch.int16)),
    lambda E: E.encode_device_adaptive_batch([(_cpu(4096), 4096, _cpu(256, torch.int16),
                                               _cpu(1 << 16), _cpu(1, torch.int32))]),
    lambda E: E.region_offsets_device_adaptive(_cpu(4, torch.int32), _cpu(4, torch.int64),
                                               _cpu(1, torch.int64)),
    lambda E: E.pack_device_adaptive_batch([(_cpu(1 << 16), 4096, 4096, _cpu(1, torch.int32),
                                             _cpu(1, torch.int64), _cpu(256, torch.int16))],
                                           _cpu(1 << 16)),
    lambda E: E.tile_order_device(_cpu(16 * 64), 16, 64, 16),
], ids=["count", "encode", "pack", "count_batch", "pack_batch", "encode_batch", "offsets",
        "count_chunks", "build_freq", "encode_adaptive", "offsets_adaptive", "pack_adaptive",
        "tile_order"])
def test_plan_free_device_calls_refuse_host_tensors(E, call):
    """A host tensor's address handed to a kernel would be dereferenced on
    the GPU: each device call refuses one before reaching the library."""
    _rejects(E, call, E, match="on a GPU is required")


def test_chunk_count_refuses_a_zero_chunk_size(E):
    assert E._n_chunks(4097, 4096) == 2 and E._n_chunks(0, 64) == 0
    _rejects(E, E._n_chunks, 10, 0, match="chunk_symbols 0")
