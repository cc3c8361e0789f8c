"""CPU check of the compiled kernels' resource use (device assembly built
here, no GPU): the 16-wave decode and fused kernels must keep two workgroups
resident per compute unit, which on MI355X takes at most 80 scalar
registers per wave in total and at most half of the CU's 160 KB of LDS per
workgroup. A kernel over either limit still runs and still matches the
oracle, but with one workgroup per CU the second waits, and the decode of a
70B-shaped layer takes far longer; this test catches that at build time."""
import os
import re
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _kernels(source):
    from entropy_coded_weight_amd import build
    with tempfile.TemporaryDirectory() as d:
        txt = open(build.asm(os.path.join(d, "k.s"), source)).read()
    out = {}
    for m in re.finditer(r"\.amdhsa_kernel (\S+)", txt):
        seg = txt[m.end():]
        out[m.group(1)] = dict(
            sgprs=int(re.search(r"; TotalNumSgprs: (\d+)", seg).group(1)),
            vgprs=int(re.search(r"\.amdhsa_next_free_vgpr (\d+)", seg).group(1)),
            lds=int(re.search(r"\.amdhsa_group_segment_fixed_size (\d+)", seg).group(1)))
    return out


@pytest.mark.parametrize("source,kernel", [("entq_decode.hip", "decode_stream"),
                                           ("entq_decode_gemv.hip", "decode_gemv"),
                                           ("entq_decode_tiles.hip", "decode_tile_gemm"),
                                           ("entq_decode_tiles.hip", "decode_tiles_rowmajor"),
                                           ("entq_decode_gemm.hip", "decode_gemm")])
def test_two_workgroups_fit_per_compute_unit(source, kernel):
    ks = {n: v for n, v in _kernels(source).items() if kernel in n}
    assert ks, f"no {kernel} instance in {source}"
    for name, r in ks.items():
        assert r["sgprs"] <= 80, (name, r)
        assert r["lds"] <= 80 * 1024, (name, r)
        if kernel != "decode_gemm":  # (its 64-row split form without packing takes more)
            # 8 waves per SIMD share its 512 vector registers per lane
            assert r["vgprs"] <= 64, (name, r)
