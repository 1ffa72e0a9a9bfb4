"""Pins for the oracle's MXFP8 quantisation (OCP MX v1.0, E4M3 elements)."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle.codecs import bf16_decode, e4m3_decode
from oracle.moe import dequant_mxfp8, dispatch_mxfp8, e8m0_decode, layout, quantize_mxfp8_rows
from workloads import bf16_bits_from_f32
from routed import make_workload
from conftest import hexint, load_golden


@pytest.mark.parametrize("block", load_golden("mxfp8_block_hand.json")["blocks"], ids=lambda b: b["name"])
def test_mxfp8_hand_worked_blocks(block):
    x = np.zeros(32, dtype=np.float32)
    x[:len(block["x"])] = np.array(block["x"], dtype=np.float32)
    bits = bf16_bits_from_f32(x[None, :])
    assert np.array_equal(bf16_decode(bits)[0, :len(block["x"])].astype(np.float64),
                          np.array(block["x"], dtype=np.float64))      # inputs are bf16 values
    codes, scales = quantize_mxfp8_rows(bits)
    want = np.zeros(32, dtype=np.uint8)
    want[:len(block["codes"])] = [hexint(c) for c in block["codes"]]
    assert scales.shape == (1, 1) and int(scales[0, 0]) == block["scale_code"]
    assert np.array_equal(codes[0], want)


def test_e8m0_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = e8m0_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def rational_shared_exponent(bits_block):
    """floor(log2 max|v|) - 8 from the bf16 bit fields (integer arithmetic)."""
    best = None
    for b in bits_block:
        b = int(b) & 0x7FFF
        if b == 0:
            continue
        e, m = b >> 7, b & 0x7F
        fl = (e - 127) if e > 0 else (m.bit_length() - 1 - 133)   # subnormal: m * 2^-133
        best = fl if best is None else max(best, fl)
    return None if best is None else max(-127, min(127, best - 8))


def round_e4m3_sat(q: Fraction) -> Fraction:
    a = abs(q)
    if a == 0:
        return Fraction(0)
    if a >= 448:
        return Fraction(448)
    e = math.frexp(float(a))[1] - 1
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    spacing = Fraction(2) ** (max(e, -6) - 3)
    n = a / spacing
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2):
        fl += 1
    return min(fl * spacing, Fraction(448))


def test_mxfp8_exact_rational_brute_force():
    rng = np.random.default_rng(23)
    T, H = 4, 256
    x = (rng.standard_normal((T, H)) * np.exp2(rng.integers(-30, 30, size=(T, H)))).astype(np.float32)
    x[0, :32] = 0.0
    x[1, 32:64] *= 2.0 ** -110         # tiny block: the shared exponent clamps at -127
    x[2, 64:96] = 300.0 + 30 * rng.random(32)   # elements that saturate
    bits = bf16_bits_from_f32(x)
    codes, scales = quantize_mxfp8_rows(bits)
    xs = bf16_decode(bits)
    for t in range(T):
        for blk in range(H // 32):
            sl = slice(32 * blk, 32 * (blk + 1))
            shared = rational_shared_exponent(bits[t, sl])
            if shared is None:
                assert scales[t, blk] == 0
                signs = np.signbit(xs[t, sl])
                assert np.array_equal(codes[t, sl], np.where(signs, 0x80, 0).astype(np.uint8))
                continue
            assert int(scales[t, blk]) == shared + 127
            for h in range(32):
                v = Fraction(float(xs[t, 32 * blk + h]))
                want = round_e4m3_sat(v / Fraction(2) ** shared)
                got = Fraction(float(e4m3_decode(codes[t, 32 * blk + h])))
                assert abs(got) == want and (want == 0 or (got < 0) == (v < 0)), (t, blk, h)


def test_mxfp8_dispatch_and_dequant_bounds():
    wl = make_workload("deepseekv3", tokens=48)
    lay = layout(wl.topk_idx, 256, 8)
    codes, scales = dispatch_mxfp8(wl.x_bits, lay["pos"])
    T, k = wl.topk_idx.shape
    deq = bf16_decode(dequant_mxfp8(codes, scales)).astype(np.float64)
    x = bf16_decode(wl.x_bits).astype(np.float64)
    for t in range(T):
        rows = lay["pos"][t]
        for j in range(1, k):
            assert np.array_equal(codes[rows[j]], codes[rows[0]])
            assert np.array_equal(scales[rows[j]], scales[rows[0]])
        d, xt = deq[rows[0]].reshape(-1, 32), x[t].reshape(-1, 32)
        X = e8m0_decode(scales[rows[0]])[:, None]
        q = np.abs(xt) / X
        normal = (q >= 2.0 ** -6) & (q <= 448)
        # E4M3 rounding (2^-4 relative) plus the bf16 rounding of the dequantised value
        assert np.all(np.abs(d - xt)[normal] <= (2.0 ** -4 + 2.0 ** -8 * 1.07) * np.abs(xt)[normal])
        sat = q > 448                            # [448, 512): clamped to 448
        assert np.all(np.abs(d[sat]) == (448 * X.repeat(32, 1))[sat])
        # the block maximum lands in [256, 512) before clamping
        am = np.max(np.abs(xt), axis=1)
        assert np.all((am / X[:, 0] >= 256) & (am / X[:, 0] < 512))
