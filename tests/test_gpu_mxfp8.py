"""GPU parity of MXFP8 dispatch (OCP MX v1.0: E4M3 elements, one E8M0 scale
per 32 channels) against the oracle: codes and scale bytes bit-exact.

Covers the five seeded workloads at full size, hidden sizes whose last
column slice is ragged, and a quantiser sweep: every amax significand against
every bf16 significand of both signs over the binades below it, plus amax
values whose shared exponent clamps at -127, sits on that boundary, or comes
from a bf16 subnormal, and all-zero / negative-zero blocks.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_dispatch_02_amd import Handle
from workloads import CONFIGS, bf16_bits_from_f32
from routed import make_workload
from gpu_util import dev_bf16, dev_i32, host_bits

pytestmark = pytest.mark.gpu

NAMES = [c.name for c in CONFIGS]


def run_mx(h, x_bits, idx, E, R):
    h.layout(dev_i32(idx))
    codes, scales = h.dispatch(dev_bf16(x_bits), mxfp8=True)
    ref = oracle.layout(idx, E, R)
    rc, rs = oracle.dispatch_mxfp8(x_bits, ref["pos"])
    total = int(ref["offsets_e"][-1])
    gc, gs = host_bits(codes)[:total], host_bits(scales)[:total]
    assert gs.dtype == np.uint8 and gs.shape[1] == x_bits.shape[1] // 32
    bad = np.argwhere(gc != rc[:total])
    assert bad.size == 0, f"{len(bad)} code mismatches, first at {bad[:3].tolist()}"
    bad = np.argwhere(gs != rs[:total])
    assert bad.size == 0, f"{len(bad)} scale mismatches, first at {bad[:3].tolist()}"
    return total


@pytest.mark.parametrize("name", NAMES)
def test_dispatch_mxfp8_matches_oracle(name):
    wl = make_workload(name)
    s = wl.shape
    h = Handle(s.tokens, s.hidden, s.topk, s.experts, s.ranks)
    run_mx(h, wl.x_bits, wl.topk_idx, s.experts, s.ranks)


@pytest.mark.parametrize("hidden", [128, 384, 1152, 7168 + 128])
def test_mxfp8_ragged_hidden(hidden):
    """Hidden sizes that leave part of the last 64-lane column slice idle."""
    rng = np.random.default_rng(hidden)
    T, k, E, R = 301, 4, 16, 4
    print(f"[mx ragged] H={hidden}", flush=True)
    x = (rng.standard_normal((T, hidden // 32, 32)) * np.exp2(rng.integers(-20, 20, size=(T, hidden // 32, 1)))
         ).reshape(T, hidden).astype(np.float32)
    x[::7, :32] = 0.0
    x[1::7, 32:64] = -0.0 if hidden > 32 else 0.0
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    idx[rng.random((T, k)) < 0.1] = -1
    run_mx(Handle(T, hidden, k, E, R), bf16_bits_from_f32(x), idx, E, R)


def mx_sweep_blocks():
    """32-channel blocks: channel 0 holds amax, the rest sweep bf16 values.

    amax takes every significand at exponent 0, exponent fields 1..9 (fields
    below 8 clamp the shared exponent at -127, 8 lands on it), bf16
    subnormals and the largest finite bf16; the swept values take every
    significand and both signs over the 22 binades at and below amax's. A
    second set puts amax in every bf16 exponent field with an 11-binade sweep.
    """
    amaxes = [(127 << 7) | m for m in range(128)]
    for e in (1, 2, 7, 8, 9):
        amaxes += [(e << 7) | m for m in (0x00, 0x2A, 0x7F)]
    amaxes += [0x0001, 0x0045, 0x007F, (0xFE << 7) | 0x7F, ((127 + 100) << 7) | 0x35]
    sweeps = [(a, 22) for a in amaxes]
    # every exponent field (every shared exponent a bf16 block can have), narrower sweep
    sweeps += [((e << 7) | 0x55, 11) for e in range(255)]
    blocks = []
    for a, width in sweeps:
        ea = a >> 7
        m = np.arange(128, dtype=np.uint32)
        cand = np.concatenate([(e << 7) | m for e in range(max(ea - width, 0), ea + 1)])
        cand = cand[cand <= a]
        cand = np.concatenate([cand, cand | 0x8000, [0, 0x8000]]).astype(np.uint16)
        for i in range(0, cand.size, 31):
            blk = np.zeros(32, dtype=np.uint16)
            blk[0] = a | (0x8000 if (i // 31) % 2 else 0)     # amax of either sign
            chunk = cand[i:i + 31]
            blk[1:1 + chunk.size] = chunk
            blocks.append(blk)
    blocks.append(np.zeros(32, np.uint16))
    blocks.append(np.full(32, 0x8000, np.uint16))
    return np.stack(blocks)


def test_mxfp8_quantiser_sweep():
    blocks = mx_sweep_blocks()
    H = 7168
    per_row = H // 32
    T = -(-blocks.shape[0] // per_row)
    x = np.zeros((T * per_row, 32), dtype=np.uint16)
    x[:blocks.shape[0]] = blocks
    x = x.reshape(T, H)
    print(f"[mx sweep] {blocks.shape[0]} blocks, T={T}", flush=True)
    rng = np.random.default_rng(9)
    E, R, k = 8, 2, 2
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    run_mx(Handle(T, H, k, E, R), x, idx, E, R)


def test_mxfp8_empty_and_invalid_rows():
    H, k, E, R = 256, 4, 8, 2
    h = Handle(64, H, k, E, R)
    assert run_mx(h, np.zeros((0, H), np.uint16), np.zeros((0, k), np.int32), E, R) == 0
    rng = np.random.default_rng(4)
    idx = np.full((40, k), -1, np.int32)
    idx[::3, 0] = 5
    x = bf16_bits_from_f32(rng.standard_normal((40, H)).astype(np.float32))
    assert run_mx(h, x, idx, E, R) == 14


def test_mxfp8_dequantised_rows_track_the_input():
    """Expert-side view: scale * code is within the E4M3 half-step of x, apart
    from the saturation loss of the block maximum."""
    wl = make_workload("qwen3_skewed", tokens=2048)
    s = wl.shape
    h = Handle(s.tokens, s.hidden, s.topk, s.experts, s.ranks)
    h.layout(dev_i32(wl.topk_idx))
    codes, scales = h.dispatch(dev_bf16(wl.x_bits), mxfp8=True)
    ref = oracle.layout(wl.topk_idx, s.experts, s.ranks)
    gc, gs = host_bits(codes), host_bits(scales)
    toks = np.arange(0, s.tokens, 97)
    rows = ref["pos"][toks, 0]
    deq = oracle.dequant_mxfp8(gc[rows], gs[rows])
    g = oracle.codecs.bf16_decode(deq).astype(np.float64)
    x = oracle.codecs.bf16_decode(wl.x_bits[toks]).astype(np.float64)
    unit = np.exp2(gs[rows].astype(np.float64) - 127).repeat(32, axis=1)
    # E4M3 half-ulp (2^-4 relative) or half its subnormal step (2^-10 * 2^shared),
    # the clamp of quotients in (448, 512) to 448, and the final bf16 rounding
    tol = (2.0 ** -4 * np.abs(x) + 2.0 ** -10 * unit + np.maximum(np.abs(x) - 448.0 * unit, 0.0)
           + 2.0 ** -8 * np.abs(g))
    assert np.all(np.abs(g - x) <= tol)
    torch.cuda.synchronize()
