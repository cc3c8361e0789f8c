"""GPU parity of the on-device encoder (through the C ABI): its containers
must be byte-identical to the oracle's encoder (small tensors) and to the
library's host encoder, which the CPU suite proves byte-identical to the
oracle's (the full 70B-shaped layer). Also: device byte counts against
numpy, decode of a device-encoded container back to the source codes, and
the frequency-0 rejection."""
import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu-encoder] {msg}", flush=True)


@pytest.fixture(scope="module")
def E():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import entropy_coded_weight_amd as E
    E.lib()
    return E


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).ravel().copy()).cuda()


def _dev_specs(specs):
    return [dict(sp, symbols=_dev(sp["symbols"])) for sp in specs]


def _oracle_chunks(c):
    return np.array([(int(r[0]), int(r[1]), int(r[2]), int(r[3]), int(r[4])) for r in c.chunks],
                    dtype=np.uint64).reshape(-1, 5)


def _device_chunks(b):
    ch = b.chunks
    return np.stack([ch["tensor"], ch["n_symbols"], ch["n_words"], ch["byte_offset"],
                     ch["elem_offset"]], axis=1).astype(np.uint64)


def _check_against_oracle(E, specs):
    c = oracle.encode_container(specs)
    b = E.encode_batch_device(_dev_specs(specs))
    blob = b.blob.cpu().numpy()
    assert blob.size == c.blob.size
    assert np.array_equal(blob, c.blob)
    assert np.array_equal(_device_chunks(b), _oracle_chunks(c))
    for t, td in enumerate(c.tensors):
        assert np.array_equal(b.freq[t], td["freq"])
    return b


def test_count_symbols_device(E):
    import torch
    rng = np.random.default_rng(5)
    for n in (0, 1, 15, 16, 17, 4095, 1 << 20, (1 << 20) + 7):
        a = rng.integers(0, 256, n, dtype=np.uint8)
        a[: n // 3] = 7  # a heavy symbol
        got = E.count_symbols_device(_dev(a) if n else torch.zeros(16, dtype=torch.uint8,
                                                                   device="cuda")[:0])
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy().view(np.uint64),
                              np.bincount(a, minlength=256).astype(np.uint64)), n


def test_tiny_laplace_and_e4m3_match_oracle(E):
    _say("tiny laplace 256x256, 4096-symbol chunks")
    _check_against_oracle(E, synth.tiny_int8_laplace())
    _say("e4m3 4096x4096")
    _check_against_oracle(E, synth.e4m3_matrix())


def test_ragged_and_degenerate_tensors_match_oracle(E):
    specs = []
    for seed, (r, c, C) in enumerate([(3, 7, 64), (1, 65, 64), (17, 129, 4096), (5, 4097, 4096),
                                      (33, 1000, 65536), (2, 65536 + 64, 65536)]):
        specs.append(synth.random_int8_tensor(r, c, 1.5 + seed, seed, C))
    one = synth.random_int8_tensor(16, 64, 1.0, 40, 64)
    one["symbols"] = np.full(one["symbols"].shape, 9, np.uint8)  # single symbol: f = 4096
    specs.append(one)
    allb = synth.random_int8_tensor(64, 512, 1.0, 41, 4096)
    allb["symbols"] = synth.random_bytes(64 * 512, 41).view(np.uint8)  # all 256 byte values
    specs.append(allb)
    _say(f"{len(specs)} ragged / degenerate tensors")
    _check_against_oracle(E, specs)


def test_device_container_decodes_to_source(E):
    import torch
    specs = synth.llama2_13b_block(shapes=[("q", 5120, 5120), ("down", 5120, 13824)])
    b = E.encode_batch_device(_dev_specs(specs))
    p = E.plan(b.tensors, b.freq, b.chunks, b.blob.numel())
    out = torch.zeros(b.out_elems, dtype=torch.uint8, device="cuda")
    status = torch.full((len(b.chunks),), -7, dtype=torch.int32, device="cuda")
    E.decode(p, b.blob, out, E.OUT_CODES, None, status)
    torch.cuda.synchronize()
    assert (status.cpu().numpy() == 0).all()
    src = np.concatenate([np.ascontiguousarray(s["symbols"]).view(np.uint8).ravel()
                          for s in specs])
    assert np.array_equal(out.cpu().numpy(), src)


def test_frequency_zero_symbol_is_rejected(E):
    import torch
    sym = np.zeros(64 * 70, np.uint8)
    sym[64 * 65 + 3] = 5          # in chunk 1 (chunks of 4096)
    freq = np.zeros(256, np.uint16)
    freq[0] = 4096                # byte 5 has frequency 0
    d = _dev(sym)
    scratch = torch.empty(int(E.lib().entq_encode_device_scratch_bytes(sym.size, 4096)),
                          dtype=torch.uint8, device="cuda")
    nw = torch.zeros(2, dtype=torch.int32, device="cuda")
    E.encode_device(d, 4096, freq, scratch, nw)
    torch.cuda.synchronize()
    got = nw.cpu().numpy().view(np.uint32)
    assert got[0] == 0 and got[1] == 0xFFFFFFFF
    with pytest.raises(E.EntqError):
        E.encode_device(d, 4096, np.zeros(256, np.uint16), scratch, nw)  # sum != 4096


def test_llama2_70b_layer_matches_host_encoder(E):
    _say("70B-shaped layer 0: device encoder vs host encoder (855.6 M symbols)")
    specs = synth.llama2_70b_layer(0)
    host = E.encode_batch(specs)
    dev = E.encode_batch_device(_dev_specs(specs))
    assert dev.blob.numel() == host.blob.size
    assert np.array_equal(dev.blob.cpu().numpy(), host.blob)
    assert np.array_equal(dev.chunks, host.chunks)
    assert np.array_equal(dev.freq, host.freq)


def test_region_offsets_device(E):
    import torch
    rng = np.random.default_rng(9)
    for k, base in ((1, 0), (1023, 16), (1024, 0), (5001, 4096), (40000, 32)):
        nw = rng.integers(0, 65537, k).astype(np.uint32)
        if k > 3:
            nw[3] = 0xFFFFFFFF  # a rejected chunk takes no bytes
        size = np.where(nw > (1 << 20), 0, (256 + 2 * nw.astype(np.uint64) + 15) // 16 * 16)
        want = base + np.concatenate([[0], np.cumsum(size)[:-1]]).astype(np.uint64)
        nw_d = torch.from_numpy(nw.view(np.int32)).cuda()
        offs = torch.empty(k, dtype=torch.int64, device="cuda")
        end = torch.zeros(1, dtype=torch.int64, device="cuda")
        E.region_offsets_device(nw_d, offs, end, base)
        torch.cuda.synchronize()
        assert np.array_equal(offs.cpu().numpy().view(np.uint64), want), k
        assert int(end.cpu()[0]) == base + int(size.sum()), k


def test_batched_encode_over_sixteen_tensors_matches_oracle(E):
    # 21 tensors: the batched call splits them over two launches
    specs = [synth.random_int8_tensor(3 + t, 64 * (1 + t % 5), 0.8 + 0.2 * t, 100 + t,
                                      (64, 4096, 256)[t % 3]) for t in range(21)]
    _say("21 tensors through the batched encode")
    _check_against_oracle(E, specs)


def test_batched_encode_marks_invalid_device_table(E):
    import torch
    rng = np.random.default_rng(3)
    sym = rng.integers(0, 4, 64 * 300, dtype=np.uint8)
    good = np.zeros(256, np.uint16)
    good[:4] = 1024
    bad = good.copy()
    bad[0] = 1023                           # sums to 4095
    d = _dev(sym)
    scr = [torch.empty(int(E.lib().entq_encode_device_scratch_bytes(sym.size, 4096)),
                       dtype=torch.uint8, device="cuda") for _ in range(2)]
    nws = [torch.zeros(5, dtype=torch.int32, device="cuda") for _ in range(2)]
    fd = torch.from_numpy(np.stack([good, bad]).view(np.int16)).cuda()
    E.encode_device_batch([(d, 4096, fd[0], scr[0], nws[0]), (d, 4096, fd[1], scr[1], nws[1])])
    torch.cuda.synchronize()
    ok = nws[0].cpu().numpy().view(np.uint32)
    assert (ok != 0xFFFFFFFF).all() and (ok > 0).all()
    assert (nws[1].cpu().numpy().view(np.uint32) == 0xFFFFFFFF).all()


# ---- per-chunk tables ------------------------------------------------------

def test_per_chunk_counts_match_numpy(E):
    import torch
    rng = np.random.default_rng(61)
    arrays = [rng.integers(0, 256, n, dtype=np.uint8) for n in (64, 4096 * 3 + 64, 65536 * 2 + 4160)]
    arrays[1][:5000] = 7                                   # a skewed stretch
    Cs = [64, 4096, 65536]
    devs = [_dev(a) for a in arrays]
    outs = [torch.full((-(-a.size // C), 256), -1, dtype=torch.int32, device="cuda")
            for a, C in zip(arrays, Cs)]
    E.count_chunks_device_batch([(d, C, o) for d, C, o in zip(devs, Cs, outs)])
    torch.cuda.synchronize()
    for a, C, o in zip(arrays, Cs, outs):
        want = np.stack([np.bincount(a[e0:e0 + C], minlength=256) for e0 in range(0, a.size, C)])
        np.testing.assert_array_equal(o.cpu().numpy(), want)


def _check_adaptive_against_oracle(E, specs):
    c = oracle.encode_container_adaptive(specs)
    b = E.encode_batch_device_adaptive(_dev_specs(specs))
    blob = b.blob.cpu().numpy()
    assert blob.size == c.blob.size
    assert np.array_equal(blob, c.blob)
    assert np.array_equal(_device_chunks(b), _oracle_chunks(c))
    assert b.freq is None
    return b


def test_per_chunk_tables_match_oracle(E):
    specs = []
    for seed, (r, c, C) in enumerate([(3, 7, 64), (1, 65, 64), (17, 129, 4096), (5, 4097, 4096),
                                      (33, 1000, 65536), (2, 65536 + 64, 65536)]):
        specs.append(synth.random_int8_tensor(r, c, 1.5 + seed, 70 + seed, C))
    one = synth.random_int8_tensor(16, 64, 1.0, 80, 64)
    one["symbols"] = np.full(one["symbols"].shape, 9, np.uint8)       # f = 4096 in every chunk
    allb = synth.random_int8_tensor(64, 512, 1.0, 81, 4096)
    allb["symbols"] = synth.random_bytes(64 * 512, 81).view(np.uint8)  # all 256 byte values
    specs += [one, allb, synth.banded_int8_tensor(48, 2816, 4, 7, 2816 * 4)]
    w = synth.bf16_weights(8, 4096)[0]
    e, _ = oracle.bf16_split(w["bf16"])
    specs.append(dict(kind=oracle.KIND_BF16EXP, rows=8, cols=4096, chunk_symbols=8192, symbols=e))
    _say(f"{len(specs)} tensors with per-chunk tables, device encoder vs oracle")
    _check_adaptive_against_oracle(E, specs)


def test_per_chunk_tables_70b_layer_match_host_and_decode(E):
    import torch
    _say("70B-shaped layer 0 with per-chunk tables: device vs host encoder, then decode")
    specs = synth.llama2_70b_layer(0)
    host = E.encode_batch_adaptive(specs)
    dev = E.encode_batch_device_adaptive(_dev_specs(specs))
    assert dev.blob.numel() == host.blob.size
    assert np.array_equal(dev.blob.cpu().numpy(), host.blob)
    assert np.array_equal(dev.chunks, host.chunks)
    p = E.plan(dev.tensors, None, dev.chunks, dev.blob.numel())
    out = torch.zeros(dev.out_elems, dtype=torch.uint8, device="cuda")
    status = torch.full((len(dev.chunks),), -7, dtype=torch.int32, device="cuda")
    E.decode(p, dev.blob, out, E.OUT_CODES, None, status)
    torch.cuda.synchronize()
    assert (status.cpu().numpy() == 0).all()
    src = np.concatenate([np.ascontiguousarray(s["symbols"]).view(np.uint8).ravel()
                          for s in specs])
    assert np.array_equal(out.cpu().numpy(), src)


def test_per_chunk_encode_marks_invalid_tables(E):
    import torch
    sym = np.zeros(4096 * 3, np.uint8)
    sym[4096 + 10] = 5                       # chunk 1 holds byte 5
    d = _dev(sym)
    freq = np.zeros((3, 256), np.uint16)
    freq[:, 0] = 4096                        # chunk 1's table lacks byte 5
    freq[2, 0] = 4000                        # chunk 2's table sums to 4000
    fd = torch.from_numpy(freq.view(np.int16)).cuda()
    scratch = torch.empty(int(E.lib().entq_encode_device_scratch_bytes(sym.size, 4096)),
                          dtype=torch.uint8, device="cuda")
    nw = torch.zeros(3, dtype=torch.int32, device="cuda")
    E.encode_device_adaptive_batch([(d, 4096, fd, scratch, nw)])
    torch.cuda.synchronize()
    got = nw.cpu().numpy().view(np.uint32)
    assert got[0] == 0 and got[1] == 0xFFFFFFFF and got[2] == 0xFFFFFFFF


def test_device_tables_equal_the_oracle_rule(E):
    """entq_build_freq_device on u32 and u64 counts: the oracle's table for
    every row, trimming, shortfall, one-byte and empty rows included."""
    import torch
    rng = np.random.default_rng(62)
    rows = [np.zeros(256, np.int64), np.eye(256, dtype=np.int64)[200] * 65536,
            np.full(256, 256, np.int64), np.arange(256, dtype=np.int64)]
    for i in range(4000):
        c = rng.integers(0, [2, 50, 5000, 1 << 20][i % 4], 256)
        c[rng.random(256) < rng.random()] = 0
        if i % 3 == 0:
            c[int(rng.integers(0, 256))] += int(rng.integers(1, 1 << 30))
        rows.append(c)
    counts = np.stack(rows)
    want = np.stack([oracle.quantize_freqs(r.astype(np.uint64)) if r.sum()
                     else np.zeros(256, np.uint16) for r in counts])
    for dt, rows_ok in ((torch.int64, slice(None)), (torch.int32, counts.max(axis=1) < 2**31)):
        sel = counts[rows_ok]
        cd = torch.from_numpy(sel.astype(np.int64 if dt == torch.int64 else np.int32)).cuda()
        fd = torch.full((sel.shape[0], 256), -1, dtype=torch.int16, device="cuda")
        E.build_freq_device(cd, fd)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(fd.cpu().numpy().view(np.uint16), want[rows_ok])


def test_device_calls_refuse_short_buffers(E):
    """Buffers a kernel would overrun are refused before the launch (no
    kernel runs in this test): word counts and offsets short of the chunk
    count, a count table short of 256 entries, a per-chunk table array short
    of 256 per chunk, the wrong element types, a buffer on another device."""
    import torch
    cuda = dict(device="cuda")
    sym = torch.zeros(8192, dtype=torch.uint8, **cuda)            # 2 chunks of 4096
    scratch = torch.empty(int(E.lib().entq_encode_device_scratch_bytes(8192, 4096)),
                          dtype=torch.uint8, **cuda)
    freq = np.zeros(256, np.uint16)
    freq[0] = 4096
    nw1 = torch.zeros(1, dtype=torch.int32, **cuda)
    nw2 = torch.zeros(2, dtype=torch.int32, **cuda)
    offs1 = torch.zeros(1, dtype=torch.int64, **cuda)
    blob = torch.zeros(1 << 16, dtype=torch.uint8, **cuda)
    cases = [
        (lambda: E.encode_device(sym, 4096, freq, scratch, nw1), "n_words holds 1"),
        (lambda: E.encode_device(sym, 4096, freq, scratch, nw2.to(torch.int64)), "dtype"),
        (lambda: E.count_symbols_device(sym, torch.zeros(255, dtype=torch.int64, **cuda)),
         "counts holds 255"),
        (lambda: E.pack_device(scratch, 8192, 4096, nw2, offs1, blob), "offsets holds 1"),
        (lambda: E.region_offsets_device(nw2, offs1, torch.zeros(1, dtype=torch.int64, **cuda)),
         "offsets holds 1"),
        (lambda: E.encode_device_adaptive_batch(
            [(sym, 4096, torch.zeros(256, dtype=torch.int16, **cuda), scratch, nw2)]),
         "freq holds 256"),
        (lambda: E.count_chunks_device_batch([(sym, 4096, torch.zeros(256, dtype=torch.int32,
                                                                      **cuda))]),
         "counts holds 256"),
        (lambda: E.build_freq_device(torch.zeros(512, dtype=torch.int64, **cuda),
                                     torch.zeros(256, dtype=torch.int16, **cuda)),
         "freq holds 256"),
        (lambda: E.tile_order_device(sym, 16, 512, 16, out=torch.zeros(8192, dtype=torch.uint8)),
         "on a GPU is required"),
    ]
    for call, match in cases:
        with pytest.raises(E.EntqError, match=match):
            call()
    torch.cuda.synchronize()
