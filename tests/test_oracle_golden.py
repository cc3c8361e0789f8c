"""Regression pin: the oracle reproduces tests/golden/oracle_small_containers.txt
(written by tests/golden/make_golden.py from the oracle alone) and decodes
it back to the stored symbols."""
import hashlib
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "oracle_small_containers.txt")


def _parse():
    cases = []
    cur = None
    for line in open(GOLDEN):
        line = line.rstrip("\n")
        if not line or line.startswith("#"):
            continue
        tag, _, rest = line.partition(" ")
        if tag == "case":
            name, n, C = rest.split()
            cur = dict(name=name, n=int(n), C=int(C), chunks=[])
            cases.append(cur)
        elif tag == "symbols":
            cur["symbols"] = np.frombuffer(bytes.fromhex(rest), np.uint8)
        elif tag == "freq":
            f = np.zeros(256, np.uint16)
            for kv in rest.split():
                s, v = kv.split(":")
                f[int(s)] = int(v)
            cur["freq"] = f
        elif tag == "chunk":
            head, _, words = rest.partition(" | ")
            parts = head.split()
            cur["chunks"].append(dict(n=int(parts[0]), nw=int(parts[1]),
                                      states=[int(v, 16) for v in parts[2:]],
                                      words=[int(v, 16) for v in words.split()]))
        elif tag == "sha256":
            cur["sha256"] = rest
    return cases


def test_golden_containers_reproduce_and_decode():
    cases = _parse()
    assert len(cases) == 3
    for c in cases:
        sym = c["symbols"]
        assert sym.size == c["n"]
        freq = oracle.quantize_freqs(oracle.count_symbols(sym))
        np.testing.assert_array_equal(freq, c["freq"])
        blob, desc = oracle.encode_tensor(sym, c["C"], freq)
        assert hashlib.sha256(blob.tobytes()).hexdigest() == c["sha256"], c["name"]
        assert desc.shape[0] == len(c["chunks"])
        for k, ch in enumerate(c["chunks"]):
            off = int(desc[k, 2])
            assert int(desc[k, 0]) == ch["n"] and int(desc[k, 1]) == ch["nw"]
            assert blob[off:off + 256].view(np.uint32).tolist() == ch["states"]
            assert blob[off + 256:off + 256 + 2 * ch["nw"]].view(np.uint16).tolist() == ch["words"]
        out, st = oracle.decode_tensor(blob, desc, c["freq"], sym.size)
        assert np.all(st == 0) and np.array_equal(out, sym)
