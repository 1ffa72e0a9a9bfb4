"""Pins for the oracle's bf16 dispatch, FP8 dispatch, combine and dequant.

Independent checks: hand-worked fixtures, exact-rational brute force of the
FP8 quantiser, the closed-form E4M3 error bound, the amax -> +-448 identity,
torch's CPU FP8/bf16 casts for dequant, combine(dispatch(x)) == x with
identity experts, unpermute / one-hot / power-of-two scaling identities, and
exact-rational evaluation of combine on tiny inputs.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import combine, dequant_fp8, dispatch_bf16, dispatch_fp8, layout
from oracle.codecs import bf16_decode, e4m3_decode
from oracle.moe import quantize_fp8_rows
from workloads import bf16_bits_from_f32, make_expert_outputs
from routed import make_workload
from conftest import combine_tolerance, hexint, load_golden


def small_workload(name, tokens, hidden=None):
    wl = make_workload(name, tokens=tokens, hidden=hidden)
    lay = layout(wl.topk_idx, wl.shape.experts, wl.shape.ranks)
    return wl, lay


# ---------------------------------------------------------------- bf16 dispatch

@pytest.mark.parametrize("name,tokens", [("tiny", 128), ("deepseek16b", 256), ("qwen3_skewed", 300)])
def test_dispatch_bf16_copy_invariant(name, tokens):
    wl, lay = small_workload(name, tokens)
    out = dispatch_bf16(wl.x_bits, lay["pos"])
    T, k = wl.topk_idx.shape
    assert out.shape == (T * k, wl.H)
    for t in range(T):
        for j in range(k):
            assert np.array_equal(out[lay["pos"][t, j]], wl.x_bits[t])
    # every row is the row of the token src_idx names
    assert np.array_equal(out, wl.x_bits[lay["src_idx"]])


# ---------------------------------------------------------------- FP8 dispatch

def golden_block_row(block):
    x = np.zeros(128, dtype=np.float32)
    x[:len(block["x"])] = np.array(block["x"], dtype=np.float32)
    return x


@pytest.mark.parametrize("block", load_golden("fp8_block_hand.json")["blocks"], ids=lambda b: b["name"])
def test_fp8_hand_worked_blocks(block):
    x = golden_block_row(block)
    codes, scales = quantize_fp8_rows(bf16_bits_from_f32(x[None, :]))
    want = np.zeros(128, dtype=np.uint8)
    want[:len(block["codes"])] = [hexint(c) for c in block["codes"]]
    assert scales.shape == (1, 1) and float(scales[0, 0]) == block["scale"]
    assert np.array_equal(codes[0], want)


def rational_round_e4m3(q: Fraction) -> Fraction:
    """Nearest-even E4M3 value of a rational (saturating at 448)."""
    a = abs(q)
    if a == 0:
        return Fraction(0)
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


def f32_div(a: Fraction, b: Fraction) -> Fraction:
    """Correctly rounded fp32 quotient of two fp32 values: the fp64 quotient
    rounded to fp32 (double rounding is harmless for division at 53 >= 2*24+2)."""
    return Fraction(float(np.float32(float(a) / float(b))))


def test_fp8_quantiser_exact_rational_brute_force():
    rng = np.random.default_rng(17)
    # a few tokens with wide dynamic range inside each block
    T, H = 6, 512
    x = (rng.standard_normal((T, H)) * np.exp2(rng.integers(-20, 20, size=(T, H)))).astype(np.float32)
    x[2, :128] = 0.0
    x[2, 5] = -0.0
    x[3, 128:256] *= 2.0 ** -120          # subnormal fp32 scale
    bits = bf16_bits_from_f32(x)
    codes, scales = quantize_fp8_rows(bits)
    xs = bf16_decode(bits)
    for t in range(T):
        for b in range(H // 128):
            blk = [Fraction(float(v)) for v in xs[t, 128 * b:128 * (b + 1)]]
            amax = max(abs(v) for v in blk)
            if amax == 0:
                assert scales[t, b] == 0
                for h, v in enumerate(xs[t, 128 * b:128 * (b + 1)]):
                    assert codes[t, 128 * b + h] == (0x80 if math.copysign(1, v) < 0 else 0)
                continue
            scale = f32_div(amax, Fraction(448))
            assert Fraction(float(scales[t, b])) == scale
            for h, v in enumerate(blk):
                q = f32_div(v, scale)
                want = rational_round_e4m3(q)
                got = Fraction(float(e4m3_decode(codes[t, 128 * b + h])))
                assert abs(got) == want and (want == 0 or (got < 0) == (v < 0)), (t, b, h)


def test_fp8_closed_form_bound_and_amax_identity():
    wl, lay = small_workload("deepseekv3", 64)
    codes, scales = dispatch_fp8(wl.x_bits, lay["pos"])
    T, k = wl.topk_idx.shape
    x = bf16_decode(wl.x_bits).astype(np.float64)
    for t in range(T):
        rows = lay["pos"][t]
        # the k copies are bitwise equal
        for j in range(1, k):
            assert np.array_equal(codes[rows[j]], codes[rows[0]])
            assert np.array_equal(scales[rows[j]].view(np.uint32), scales[rows[0]].view(np.uint32))
        v = e4m3_decode(codes[rows[0]]).reshape(-1, 128)
        s = scales[rows[0]].astype(np.float64)
        xb = x[t].reshape(-1, 128)
        deq = v * s[:, None]
        quot = np.abs(xb) / s[:, None]
        normal = quot >= 2.0 ** -6
        err = np.abs(deq - xb)
        # normal range: half an E4M3 ulp (2^-4 relative) plus the fp32 quotient rounding
        assert np.all(err[normal] <= (2.0 ** -4 + 2.0 ** -22) * np.abs(xb[normal]))
        # subnormal range: half the 2^-9 spacing, in units of the scale
        assert np.all(err[~normal] <= (2.0 ** -10 + 2.0 ** -22) * s[:, None].repeat(128, 1)[~normal])
        # the amax element encodes to +-448 exactly
        am = np.argmax(np.abs(xb), axis=1)
        assert np.all(np.abs(v[np.arange(v.shape[0]), am]) == 448.0)
        assert np.all(s == (np.max(np.abs(xb), axis=1).astype(np.float32) / np.float32(448)))


def test_dequant_matches_torch_casts():
    rng = np.random.default_rng(2)
    codes = rng.integers(0, 256, size=(4, 256), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10       # no NaN codes
    scales = rng.uniform(1e-3, 1.0, size=(4, 2)).astype(np.float32)
    # keep 20 significant bits so that code * scale (4 + 20 bits) is exact in
    # fp32 and torch's fp32 -> bf16 cast sees the exact product
    scales = (scales.view(np.uint32) & np.uint32(0xFFFFFFF0)).view(np.float32)
    ours = dequant_fp8(codes, scales)
    vals = torch.from_numpy(codes).view(torch.float8_e4m3fn).float()
    ref = (vals.view(4, 2, 128) * torch.from_numpy(scales)[:, :, None]).view(4, 256)
    assert torch.equal(ref.double(), torch.from_numpy(codes).view(torch.float8_e4m3fn).double().view(4, 2, 128).mul(
        torch.from_numpy(scales).double()[:, :, None]).view(4, 256))
    ref_bits = ref.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref_bits)


# ---------------------------------------------------------------- combine

@pytest.mark.parametrize("case", load_golden("combine_hand.json")["cases"], ids=lambda c: c["name"])
def test_combine_hand_worked(case):
    y = bf16_bits_from_f32(np.array(case["y"], dtype=np.float32))
    out = combine(y, np.array(case["w"], dtype=np.float32), np.array(case["pos"]))
    assert [int(v) for v in out.reshape(-1)] == [hexint(b) for b in case["out_bits"]]


@pytest.mark.parametrize("name,tokens", [("tiny", 128), ("deepseek16b", 128), ("deepseekv3", 32), ("qwen3_skewed", 128)])
def test_combine_identity_experts_returns_x(name, tokens):
    wl, lay = small_workload(name, tokens)
    x = wl.x_bits.copy()
    x[:, :3] = [0x8000, 0x0000, 0x0001]             # -0, +0 and the smallest subnormal
    y = dispatch_bf16(x, lay["pos"])
    out = combine(y, wl.topk_w, lay["pos"])
    # the weighted sum starts from +0, so -0 comes back as +0; all else bit for bit
    assert np.array_equal(out, np.where(x == 0x8000, np.uint16(0), x))


def test_combine_unpermute_onehot_and_scaling():
    wl, lay = small_workload("deepseek16b", 96, hidden=256)
    T, k = wl.topk_idx.shape
    y = make_expert_outputs(T * k, 256, seed=5)
    # k=1, w=1: exact unpermute of the first slot
    pos1 = lay["pos"][:, :1]
    out = combine(y, np.ones((T, 1), np.float32), pos1)
    assert np.array_equal(out, y[pos1[:, 0]])
    # one-hot weights pick one slot's row exactly
    sel = np.arange(T) % k
    w = np.zeros((T, k), np.float32)
    w[np.arange(T), sel] = 1.0
    out = combine(y, w, lay["pos"])
    assert np.array_equal(out, y[lay["pos"][np.arange(T), sel]])
    # scaling every weight by 2^n scales the result by 2^n exactly
    base = bf16_decode(combine(y, wl.topk_w, lay["pos"]))
    for n in (-3, 5):
        scaled = bf16_decode(combine(y, (wl.topk_w * np.float32(2.0 ** n)), lay["pos"]))
        assert np.array_equal(scaled, base * np.float32(2.0 ** n))


def test_combine_exact_rational_tiny():
    rng = np.random.default_rng(9)
    T, k, H = 5, 3, 16
    y = make_expert_outputs(T * k, H, seed=1)
    w = rng.uniform(-1, 1, size=(T, k)).astype(np.float32)
    pos = rng.permutation(T * k).reshape(T, k)
    pos[1, 2] = -1
    out, mag = combine(y, w, pos, return_magnitude=True)
    yv = bf16_decode(y)
    for t in range(T):
        for h in range(H):
            s = sum((Fraction(float(w[t, j])) * Fraction(float(yv[pos[t, j], h]))
                     for j in range(k) if pos[t, j] >= 0), Fraction(0))
            got = Fraction(float(bf16_decode(out[t, h])))
            # nearest bf16 to the exact sum: check got is a nearest neighbour
            ulp_e = math.frexp(float(abs(s)) or 1.0)[1] - 1
            spacing = Fraction(2) ** (max(ulp_e, -126) - 7)
            assert abs(got - s) <= spacing / 2
            m = sum((abs(Fraction(float(w[t, j])) * Fraction(float(yv[pos[t, j], h])))
                     for j in range(k) if pos[t, j] >= 0), Fraction(0))
            assert abs(Fraction(float(mag[t, h])) - m) <= m * Fraction(1, 2 ** 50)


def test_combine_gate_accepts_fp32_evaluations():
    """An fp32 evaluation in fixed slot order (with or without fused multiply-add)
    passes the gate; a dropped slot or a transposed weight does not."""
    wl, lay = small_workload("deepseekv3", 48, hidden=512)
    T, k = wl.topk_idx.shape
    y = make_expert_outputs(T * k, 512, seed=3)
    ref, mag = combine(y, wl.topk_w, lay["pos"], return_magnitude=True)
    tol = combine_tolerance(ref, mag, k)
    yv = bf16_decode(y)
    refv = bf16_decode(ref).astype(np.float64)

    def fp32_sum(fma, drop=None, w=wl.topk_w):
        acc = np.zeros((T, 512), np.float32)
        for j in range(k):
            if j == drop:
                continue
            term = w[:, j][:, None].astype(np.float64) * yv[lay["pos"][:, j]].astype(np.float64)
            if fma:
                acc = (acc.astype(np.float64) + term).astype(np.float32)
            else:
                acc = (acc + term.astype(np.float32)).astype(np.float32)
        return bf16_decode(bf16_bits_from_f32(acc)).astype(np.float64)

    for fma in (False, True):
        assert np.all(np.abs(fp32_sum(fma) - refv) <= tol)
    assert not np.all(np.abs(fp32_sum(False, drop=k - 1) - refv) <= tol)
    assert not np.all(np.abs(fp32_sum(False, w=wl.topk_w[:, ::-1].copy()) - refv) <= tol)


def test_fp8_round_trip_through_combine():
    wl, lay = small_workload("deepseekv3_fp8", 32)
    codes, scales = dispatch_fp8(wl.x_bits, lay["pos"])
    y = dequant_fp8(codes, scales)
    out = bf16_decode(combine(y, wl.topk_w, lay["pos"])).astype(np.float64)
    x = bf16_decode(wl.x_bits).astype(np.float64)
    s = scales[lay["pos"][:, 0]].astype(np.float64).repeat(128, axis=1)
    bound = 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * s
    # plus bf16 rounding of the dequantised rows and of the output, and the weights' sum
    bound = bound * (1 + 2.0 ** -7) + 2.0 ** -8 * np.abs(x) + 1e-6
    assert np.all(np.abs(out - x) <= bound)
