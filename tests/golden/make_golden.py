"""Writes tests/golden/oracle_small_containers.txt from the oracle alone.

The pages print no worked example of the coder, so this fixture is a
regression pin: it freezes what the oracle (already pinned by closed forms,
brute force and an independent Python statement) produces for a few small
seeded inputs, so that any later change to the oracle's arithmetic shows up
as a diff that has to be justified.

Run from the repository root:  python tests/golden/make_golden.py
"""
import hashlib
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small_containers.txt")


def cases():
    yield "laplace_b2_300_C128", synth.int8_codes(
        lambda x: synth.laplace_cdf(x, 2.0), 300, synth.key(1000, 0, 0, 0)).view(np.uint8), 128
    yield "normal_s1_200_C64", synth.int8_codes(
        lambda x: synth.normal_cdf(x, 1.0), 200, synth.key(1000, 1, 0, 0)).view(np.uint8), 64
    yield "bytes_uniform_129_C4096", synth.random_bytes(129, 5), 4096


def main():
    lines = ["# name n C | freq (symbol:f ...) | per chunk: n_symbols n_words states(hex) words(hex) | sha256(blob)"]
    for name, sym, C in cases():
        freq = oracle.quantize_freqs(oracle.count_symbols(sym))
        blob, desc = oracle.encode_tensor(sym, C, freq)
        f = " ".join(f"{s}:{int(freq[s])}" for s in range(256) if freq[s])
        lines.append(f"case {name} {sym.size} {C}")
        lines.append(f"symbols {sym.tobytes().hex()}")
        lines.append(f"freq {f}")
        for k in range(desc.shape[0]):
            off = int(desc[k, 2])
            nw = int(desc[k, 1])
            st = blob[off:off + 256].view(np.uint32)
            w = blob[off + 256:off + 256 + 2 * nw].view(np.uint16)
            lines.append(f"chunk {int(desc[k, 0])} {nw} {' '.join(f'{v:08x}' for v in st)} | "
                         f"{' '.join(f'{v:04x}' for v in w)}")
        lines.append(f"sha256 {hashlib.sha256(blob.tobytes()).hexdigest()}")
    with open(OUT, "w") as fh:
        fh.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
