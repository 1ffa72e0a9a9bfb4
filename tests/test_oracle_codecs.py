"""Pins for the oracle's bf16 and E4M3 codecs (CPU only).

The codecs are checked against torch's CPU casts (a library routine), the
format tables in tests/golden/, and a textbook frexp-based rounding written
with exact rationals.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle.codecs import bf16_decode, bf16_encode, e4m3_decode, e4m3_encode
from conftest import hexint, load_golden


def structured_f32(max_biased_exp: int) -> np.ndarray:
    """fp32 patterns that hit every rounding boundary of narrower formats.

    Exponent field 0..max_biased_exp, all 128 values of the top 7 mantissa
    bits, and low 16 bits in {0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF}; both signs.
    """
    exps = np.arange(max_biased_exp + 1, dtype=np.uint32)
    hi = np.arange(128, dtype=np.uint32)
    lo = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    bits = (exps[:, None, None] << 23) | (hi[None, :, None] << 16) | lo[None, None, :]
    bits = bits.reshape(-1)
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    return bits.view(np.float32)


def random_f32(n, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32).view(np.float32)


def torch_e4m3(v):
    return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_bf16(v):
    return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(
        torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------- E4M3

def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))
    assert np.isnan(ours).sum() == 2  # only S.1111.111


def test_e4m3_golden_table():
    g = load_golden("e4m3_ocp_values.json")
    for item in g["decode"]:
        v = e4m3_decode(np.array([hexint(item["code"])], dtype=np.uint8))[0]
        if item["value"] == "nan":
            assert math.isnan(v)
        else:
            assert v == item["value"] and math.copysign(1, v) == math.copysign(1, item["value"])
    for item in g["encode_rne"]:
        code = e4m3_encode(np.array([item["value"]], dtype=np.float32))[0]
        assert code == hexint(item["code"]), item


@pytest.mark.parametrize("source", ["structured", "random"])
def test_e4m3_encode_matches_torch_within_range(source):
    v = structured_f32(136) if source == "structured" else random_f32(1 << 20, 7)
    v = v[~np.isnan(v)]
    # torch's cast overflows to NaN above the 464 midpoint; compare where it saturates.
    inside = np.abs(v.astype(np.float64)) <= 464.0
    ours = e4m3_encode(v[inside])
    ref = torch_e4m3(v[inside])
    assert np.array_equal(ours, ref)
    assert inside.sum() > 100_000 if source == "structured" else inside.sum() > 1000


def test_e4m3_encode_saturates_and_nan():
    v = np.array([464.0, 464.01, 1e6, np.inf, -1e30, -np.inf, np.nan, -np.nan], dtype=np.float32)
    codes = e4m3_encode(v)
    assert list(codes[:4]) == [0x7E] * 4
    assert list(codes[4:6]) == [0xFE] * 2
    assert codes[6] & 0x7F == 0x7F and codes[7] & 0x7F == 0x7F


def textbook_round(v: float, mant_bits: int, emin: int, emax_value) -> Fraction:
    """Nearest-even rounding of |v| to a binary format with `mant_bits` stored
    mantissa bits and minimum normal exponent `emin` (exact rationals)."""
    a = abs(Fraction(v))
    if a == 0:
        return Fraction(0)
    _, e = math.frexp(float(a))          # float(a) has the right binade for these inputs
    e = e - 1                            # a in [2^e, 2^(e+1)) up to rounding of float()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (max(e, emin) - mant_bits)   # spacing
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * q
    return min(r, emax_value) if emax_value is not None else r


def test_e4m3_encode_matches_textbook_rounding():
    rng = np.random.default_rng(3)
    # magnitudes spread over the whole normal and subnormal E4M3 range
    mags = np.exp2(rng.uniform(-14, 8.8, size=4000)).astype(np.float32)
    signs = np.where(rng.random(4000) < 0.5, -1, 1).astype(np.float32)
    v = mags * signs
    codes = e4m3_encode(v)
    vals = e4m3_decode(codes)
    for x, got in zip(v.tolist(), vals.tolist()):
        want = float(textbook_round(x, 3, -6, Fraction(448)))
        assert abs(got) == want, (x, got, want)
        if want != 0:
            assert math.copysign(1, got) == math.copysign(1, x)


# ---------------------------------------------------------------- bf16

def test_bf16_golden_table():
    g = load_golden("bf16_values.json")
    for item in g["decode"]:
        v = float(bf16_decode(np.array([hexint(item["bits"])], dtype=np.uint16))[0])
        want = float(item["value"])
        assert v == want
    for item in g["encode_rne"]:
        bits = bf16_encode(np.array([item["value"]], dtype=np.float64))[0]
        assert bits == hexint(item["bits"]), item


@pytest.mark.parametrize("source", ["structured", "random"])
def test_bf16_encode_matches_torch(source):
    v = structured_f32(255) if source == "structured" else random_f32(1 << 20, 11)
    ours = bf16_encode(v)
    ref = torch_bf16(v)
    nan = np.isnan(v)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all((ours[nan] & 0x7FFF) > 0x7F80)


def test_bf16_decode_roundtrip_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16_decode(codes)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(vals[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    back = bf16_encode(vals[~nan])
    assert np.array_equal(back, codes[~nan])


def test_bf16_encode_from_fp64_rounds_once():
    """fp64 inputs are rounded once (never via fp32), checked with exact rationals."""
    rng = np.random.default_rng(5)
    base = np.exp2(rng.uniform(-130, 127, size=3000))
    # put many values right next to bf16 midpoints, where double rounding would show
    ups = bf16_decode(bf16_encode(base)).astype(np.float64)
    _, e = np.frexp(ups)                                  # ups in [2^(e-1), 2^e)
    spacing = np.exp2(np.maximum(e - 1, -126) - 7)
    mids = ups + spacing / 2                              # exact bf16 midpoints
    near = np.concatenate([base, mids, np.nextafter(mids, 0), np.nextafter(mids, np.inf)])
    near = near * np.where(rng.random(near.size) < 0.5, -1.0, 1.0)
    got = bf16_decode(bf16_encode(near)).astype(np.float64)
    for x, g in zip(near.tolist(), got.tolist()):
        want = float(textbook_round(x, 7, -126, None))
        assert abs(g) == want, (x, g, want)
