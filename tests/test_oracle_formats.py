"""Pins of the oracle's number formats against what fixes them independently:
torch's CPU casts (run as a black-box library), the IEEE rules for NaN, and
the bf16 field layout checked through torch's bf16 -> fp32 conversion.

Sources: Float8/Int8 base codes dequantised with per-channel scales
(EntQuant summary "Float8@2bits ...", technical part §2); BF16 split into
exponent and sign+mantissa (DFloat11 write-up, "Formato DFloat11")."""
import numpy as np
import pytest
import torch

import oracle


def _torch_bf16_bits(u32: np.ndarray) -> np.ndarray:
    f = torch.from_numpy(u32.view(np.float32).copy())
    return f.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_rne_matches_torch_on_every_rounding_boundary():
    hi = np.arange(1 << 16, dtype=np.uint32)
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1234, 0xC000],
                    dtype=np.uint32)
    u = ((hi[:, None] << 16) | lows[None, :]).ravel()
    nan = ((u & 0x7F800000) == 0x7F800000) & ((u & 0x007FFFFF) != 0)
    u = u[~nan]
    np.testing.assert_array_equal(oracle.bf16_from_f32_bits(u), _torch_bf16_bits(u))


def test_bf16_rne_matches_torch_on_random_patterns():
    rng = np.random.default_rng(1)
    u = rng.integers(0, 1 << 32, size=2_000_000, dtype=np.uint64).astype(np.uint32)
    nan = ((u & 0x7F800000) == 0x7F800000) & ((u & 0x007FFFFF) != 0)
    u = u[~nan]
    np.testing.assert_array_equal(oracle.bf16_from_f32_bits(u), _torch_bf16_bits(u))


def test_bf16_special_values():
    cases = {
        0x00000000: 0x0000, 0x80000000: 0x8000,          # signed zeros
        0x7F800000: 0x7F80, 0xFF800000: 0xFF80,          # infinities
        0x7F7FFFFF: 0x7F80,                              # max finite rounds up to inf
        0x7F7F7FFF: 0x7F7F,                              # just below the midpoint
        0x3F808000: 0x3F80,                              # tie to even (down)
        0x3F818000: 0x3F82,                              # tie to even (up)
        0x00008000: 0x0000, 0x00018000: 0x0002,          # subnormal ties
    }
    for u, want in cases.items():
        assert int(oracle.bf16_from_f32_bits(np.array([u], np.uint32))[0]) == want, hex(u)


def test_bf16_nan_follows_ieee_narrowing():
    # IEEE 754-2008 6.2.3: a NaN converted to a narrower format stays a quiet
    # NaN and keeps its sign and the high-order bits of its payload.
    rng = np.random.default_rng(2)
    mant = rng.integers(1, 1 << 23, size=10000).astype(np.uint32)
    sign = rng.integers(0, 2, size=10000).astype(np.uint32) << 31
    u = sign | 0x7F800000 | mant
    b = oracle.bf16_from_f32_bits(u).astype(np.uint32)
    assert np.all((b & 0x7F80) == 0x7F80)                    # exponent all ones
    assert np.all((b & 0x0040) == 0x0040)                    # quiet bit
    assert np.all((b >> 15) == (u >> 31))                    # sign kept
    assert np.all((b & 0x3F) == ((u >> 16) & 0x3F))          # top payload kept
    # and torch, which canonicalises, agrees that the result is a NaN
    assert torch.isnan(torch.from_numpy(b.astype(np.uint16).view(np.int16))
                       .view(torch.bfloat16).float()).all()


def test_e4m3_decode_all_256_codes_match_torch():
    # every pattern, the two NaN codes included: torch's CPU cast widens a
    # NaN code keeping its sign and putting its mantissa bits at the top of
    # the fp32 payload, as IEEE 754-2008 6.2.3 widens a NaN
    mine = oracle.e4m3_table().view(np.float32)
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan_ref)
    assert nan_ref.sum() == 2 and nan_ref[0x7F] and nan_ref[0xFF]
    np.testing.assert_array_equal(mine.view(np.uint32), ref.view(np.uint32))
    bits = oracle.e4m3_table()
    assert bits[0x7F] >> 31 == 0 and bits[0xFF] >> 31 == 1  # sign kept
    # a few values by the format definition: 448 max, 2^-9 min subnormal, -0
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and bits[0x80] == 0x80000000


def test_int8_value_is_twos_complement():
    for c in range(256):
        v = np.array([oracle.lib().orc_int8_to_f32_bits(c)], np.uint32).view(np.float32)[0]
        assert v == (c if c < 128 else c - 256)


@pytest.mark.parametrize("kind", [oracle.KIND_INT8, oracle.KIND_E4M3])
def test_dequant_matches_torch_fp32_product_then_bf16(kind):
    rng = np.random.default_rng(3 + kind)
    codes = rng.integers(0, 256, size=200_000).astype(np.uint8)
    if kind == oracle.KIND_E4M3:
        codes[(codes & 0x7F) == 0x7F] = 0x7E  # NaN codes are checked separately
    rows, cols = 400, 500
    # scales spanning normal magnitudes plus a few extreme ones
    scales = rng.uniform(1e-3, 1e-2, size=rows).astype(np.float32)
    scales[:4] = np.array([3.0e38, 1e-40, -2.5, 0.0], np.float32)
    got = oracle.dequant_tensor(codes, rows, cols, kind, scales)
    if kind == oracle.KIND_INT8:
        v = torch.from_numpy(codes.view(np.int8).astype(np.float32))
    else:
        v = torch.from_numpy(codes).view(torch.float8_e4m3fn).float()
    p = v.reshape(rows, cols) * torch.from_numpy(scales)[:, None]
    want = p.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).ravel()
    np.testing.assert_array_equal(got, want)


def test_dequant_of_nan_code_composes_the_pinned_steps():
    # value: torch's widening of the NaN code; product: the host's IEEE
    # multiply (a NaN operand comes out as itself, quieted); bf16: the IEEE
    # narrowing (sign and top payload kept, quiet bit set)
    codes = torch.tensor([0x7F, 0xFF], dtype=torch.uint8).view(torch.float8_e4m3fn)
    v = codes.float().numpy().view(np.uint32)
    for scale in (0.5, -0.5, 3.0e38, 0.0, 1e-40, float("inf"), float("-inf")):
        sb = int(np.array([scale], np.float32).view(np.uint32)[0])
        for c, vb in zip((0x7F, 0xFF), v):
            p = int(_np_mul_bits([int(vb)], [sb])[0])
            want = (p >> 16) | 0x0040
            assert oracle.dequant_bf16(c, oracle.KIND_E4M3, scale) == want, (hex(c), scale)
    assert oracle.dequant_bf16(0x7F, oracle.KIND_E4M3, 0.5) >> 15 == 0
    assert oracle.dequant_bf16(0xFF, oracle.KIND_E4M3, 0.5) >> 15 == 1


def _np_mul_bits(a_bits, b_bits):
    a = np.array(a_bits, np.uint32).view(np.float32)
    b = np.array(b_bits, np.uint32).view(np.float32)
    with np.errstate(all="ignore"):
        return (a * b).view(np.uint32)


def test_product_nan_rules_match_ieee_hardware_multiply():
    # numpy's float32 multiply runs the host's IEEE unit: with one NaN
    # operand the result is that operand quieted (payload and sign kept),
    # 0 * inf is the default NaN, everything else is the rounded product.
    rng = np.random.default_rng(9)
    specials = [0x7FC12345, 0xFFA00001, 0x7F800001, 0x7F800000, 0xFF800000, 0x00000000,
                0x80000000, 0x00000001, 0x7F7FFFFF, 0x3F800000, 0xBF800000]
    finite = rng.integers(0, 1 << 32, 2000, dtype=np.uint64).astype(np.uint32)
    finite = finite[((finite >> 23) & 0xFF) != 0xFF]
    pairs = [(a, b) for a in specials for b in specials
             if not (oracle._isnan_bits(a) and oracle._isnan_bits(b))]
    pairs += [(int(a), int(b)) for a, b in zip(finite[:1000], finite[1000:2000])]
    pairs += [(int(a), s) for a in finite[:50] for s in specials]
    a = [p[0] for p in pairs]
    b = [p[1] for p in pairs]
    want = _np_mul_bits(a, b)
    got = np.array([oracle.mul_f32_bits(x, y) for x, y in pairs], np.uint32)
    np.testing.assert_array_equal(got, want)
    assert oracle.mul_f32_bits(0x00000000, 0x7F800000) == 0xFFC00000


def test_product_with_two_nans_keeps_the_codes_nan():
    assert oracle.mul_f32_bits(0xFFC00000, 0x7FC12345) == 0xFFC00000
    assert oracle.mul_f32_bits(0x7FA00000, 0xFFC00001) == 0x7FE00000


def test_bf16_split_merge_round_trip_all_patterns():
    w = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    e, sm = oracle.bf16_split(w)
    np.testing.assert_array_equal(oracle.bf16_merge(e, sm), w)


def test_bf16_exponent_field_is_the_biased_exponent():
    # Through torch's bf16 -> fp32 conversion: a normal bf16 with exponent
    # byte e, sign bit from sm and mantissa sm & 0x7F has value
    # (-1)^s * 2^(e - 127) * (1 + m / 128).
    w = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    e, sm = oracle.bf16_split(w)
    vals = torch.from_numpy(w.view(np.int16)).view(torch.bfloat16).double().numpy()
    normal = (e > 0) & (e < 255)
    s = (sm >> 7).astype(np.float64)
    m = (sm & 0x7F).astype(np.float64)
    want = (-1.0) ** s * np.ldexp(1.0 + m / 128.0, e.astype(np.int64) - 127)
    np.testing.assert_array_equal(vals[normal], want[normal])
