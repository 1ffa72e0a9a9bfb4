"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle.

Bar: layout arrays, dispatched bf16 rows, FP8 codes and fp32 scales, MXFP8
codes and E8M0 scales are bit-exact; combine is within 1e-2 relative error (plus the fp32 cancellation
term derived in conftest.combine_tolerance). Workloads are the five seeded
shapes at full size, plus edge cases (empty, one token, k=1, one expert per
rank, every slot on one expert, invalid ids, the maximum E and k, 65536
tokens, ragged chunk tails) and an FP8 sweep that covers every bf16
significand against every amax significand over the whole quotient range.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_dispatch_02_amd import Handle, MoeError
from workloads import CONFIGS, make_expert_outputs
from routed import make_workload
from gpu_util import (assert_combine_close, assert_layout_equal, dev_bf16, dev_f32, dev_i32,
                      host_bits, layout_on_gpu)

pytestmark = pytest.mark.gpu

NAMES = [c.name for c in CONFIGS]


def handle(shape, tokens=None, hidden=None):
    return Handle(shape.tokens if tokens is None else tokens,
                  shape.hidden if hidden is None else hidden,
                  shape.topk, shape.experts, shape.ranks)


@pytest.fixture(scope="module", autouse=True)
def gpu_present():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    print(f"\n[gpu] {torch.cuda.get_device_name(0)}", flush=True)


# ---------------------------------------------------------------- layout

@pytest.mark.parametrize("name", NAMES)
def test_layout_matches_oracle(name):
    wl = make_workload(name)
    s = wl.shape
    got = layout_on_gpu(handle(s), wl.topk_idx)
    ref = oracle.layout(wl.topk_idx, s.experts, s.ranks)
    assert_layout_equal(got, ref, s.tokens, s.topk)


EDGE = [
    # name, T, k, E, R, id pattern
    ("empty", 0, 4, 16, 4, "random"),
    ("one_token", 1, 8, 256, 8, "random"),
    ("k1", 3000, 1, 64, 8, "random"),
    ("one_expert_per_rank", 2500, 2, 8, 8, "random"),
    ("every_slot_one_expert", 5000, 1, 128, 8, "const"),
    ("duplicates_one_expert", 700, 4, 16, 4, "const"),
    ("invalid_ids", 1500, 8, 64, 8, "invalid"),
    ("max_experts", 2000, 8, 1024, 8, "random"),
    ("max_topk", 600, 32, 64, 8, "random"),
    ("ragged_tail", 2049, 3, 32, 4, "random"),
    ("single_expert", 300, 1, 1, 1, "random"),
    ("all_invalid", 100, 2, 8, 2, "all_invalid"),
]


def edge_ids(T, k, E, pattern, seed=0):
    rng = np.random.default_rng(seed)
    if pattern == "random":
        return rng.integers(0, E, size=(T, k)).astype(np.int32)
    if pattern == "const":
        return np.full((T, k), E - 1, dtype=np.int32)
    if pattern == "all_invalid":
        return np.full((T, k), -1, dtype=np.int32)
    ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    bad = rng.random((T, k)) < 0.15
    ids[bad] = rng.choice(np.array([-1, E, E + 77, -123456, 2**31 - 1], dtype=np.int64),
                          size=int(bad.sum())).astype(np.int32)
    return ids


def test_combine_subnormal_values():
    """bf16 subnormal rows and products in fp32's subnormal range: combine must
    keep them (no flush to zero), to the oracle's gate; and an identity round
    trip whose every term w * x is an exact fp32 subnormal returns x bit for
    bit (k copies of x / k sum exactly)."""
    rng = np.random.default_rng(77)
    T, H, k, E, R = 300, 512, 8, 64, 8
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    S = T * k
    # y: bf16 subnormals (exponent field 0) and small normals just above them
    mant = rng.integers(1, 128, size=(S, H)).astype(np.uint16)
    sign = (rng.random((S, H)) < 0.5).astype(np.uint16) << 15
    expo = np.where(rng.random((S, H)) < 0.7, 0, rng.integers(1, 4, size=(S, H))).astype(np.uint16)
    y = sign | (expo << 7) | mant
    w = rng.uniform(0.01, 1.0, size=(T, k)).astype(np.float32)
    w[:, 0] = np.float32(2.0 ** -20)   # products far below the smallest bf16 subnormal
    h = Handle(T, H, k, E, R)
    h.layout(dev_i32(idx))
    ref = oracle.layout(idx, E, R)
    got = host_bits(h.combine(dev_bf16(y), dev_f32(w)))
    want, mag = oracle.combine(y, w, ref["pos"], return_magnitude=True)
    _, exact = assert_combine_close(got, want, mag, k)
    assert exact > 0.9, exact
    assert np.any(((got & 0x7F80) == 0) & ((got & 0x7FFF) != 0))   # subnormal results survive
    # identity round trip of subnormal x with weights 1/k: every term exact
    xs = (sign[:T] | mant[:T]).astype(np.uint16)           # bf16 subnormals (mantissa >= 1)
    rows = h.dispatch(dev_bf16(xs))
    back = host_bits(h.combine(rows, dev_f32(np.full((T, k), 1.0 / k, np.float32))))
    torch.cuda.synchronize()
    assert np.array_equal(back, xs)


def test_combine_keeps_negative_zero():
    """A token whose weighted terms all underflow to -0 in fp32 sums to -0 on
    both sides; with a skipped (invalid) last slot the kernel must leave that
    -0 as it is rather than add a zero product (which would give +0)."""
    T, H, k, E, R = 64, 64, 4, 16, 4
    rng = np.random.default_rng(5)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx[:, k - 1] = -1                              # the last slot is skipped
    S = T * k
    y = np.full((S, H), 0x8001, dtype=np.uint16)     # -2^-133, the smallest bf16 subnormal
    w = np.full((T, k), 2.0 ** -20, dtype=np.float32)   # each product -2^-153: below fp32's range
    h = Handle(T, H, k, E, R)
    h.layout(dev_i32(idx))
    ref = oracle.layout(idx, E, R)
    got = host_bits(h.combine(dev_bf16(y), dev_f32(w)))
    want = oracle.combine(y, w, ref["pos"])
    assert np.all(want == 0x8000), "the oracle's sum of negative underflowing terms is -0"
    assert np.array_equal(got, want)


@pytest.mark.parametrize("case", EDGE, ids=lambda c: c[0])
def test_edge_cases_all_ops(case):
    name, T, k, E, R, pattern = case
    print(f"[edge] {name} T={T} k={k} E={E} R={R}", flush=True)
    H = 256
    idx = edge_ids(T, k, E, pattern)
    h = Handle(max(T, 1), H, k, E, R)
    got = layout_on_gpu(h, idx)
    ref = oracle.layout(idx, E, R)
    assert_layout_equal(got, ref, T, k)
    total = int(ref["offsets_e"][-1])

    rng = np.random.default_rng(1)
    x = rng.standard_normal((T, H), dtype=np.float32)
    x[:, :128] *= 0.0                                   # an all-zero FP8 block per token
    if T:
        x[0, 5] = -0.0
    from workloads import bf16_bits_from_f32
    xb = bf16_bits_from_f32(x)
    out = host_bits(h.dispatch(dev_bf16(xb)))
    assert np.array_equal(out[:total], oracle.dispatch_bf16(xb, ref["pos"])[:total])

    codes, scales = h.dispatch(dev_bf16(xb), fp8=True)
    rc, rs = oracle.dispatch_fp8(xb, ref["pos"])
    assert np.array_equal(host_bits(codes)[:total], rc[:total])
    assert np.array_equal(host_bits(scales)[:total].view(np.uint32), rs[:total].view(np.uint32))

    codes, scales = h.dispatch(dev_bf16(xb), mxfp8=True)
    rc, rs = oracle.dispatch_mxfp8(xb, ref["pos"])
    assert np.array_equal(host_bits(codes)[:total], rc[:total])
    assert np.array_equal(host_bits(scales)[:total], rs[:total])

    y = make_expert_outputs(T * k, H, seed=2)
    w = rng.uniform(-1, 1, size=(T, k)).astype(np.float32)
    comb = host_bits(h.combine(dev_bf16(y), dev_f32(w)))
    ref_c, mag = oracle.combine(y, w, ref["pos"], return_magnitude=True)
    assert_combine_close(comb, ref_c, mag, k)


@pytest.mark.parametrize("hidden", [8, 24, 520, 4104, 16384 + 8])
def test_hidden_extremes_bf16(hidden):
    """bf16 dispatch and combine from the smallest row (one 16-byte vector) to
    rows whose last 512-channel slice holds a single vector."""
    print(f"[hidden] bf16 H={hidden}", flush=True)
    T, k, E, R = 700, 4, 32, 4
    rng = np.random.default_rng(hidden)
    idx = edge_ids(T, k, E, "invalid", seed=hidden)
    x = rng.integers(0, 2 ** 16, size=(T, hidden), dtype=np.uint16) & np.uint16(0xBFFF)
    h = Handle(T, hidden, k, E, R)
    got = layout_on_gpu(h, idx)
    ref = oracle.layout(idx, E, R)
    assert_layout_equal(got, ref, T, k)
    total = int(ref["offsets_e"][-1])
    out = host_bits(h.dispatch(dev_bf16(x)))
    assert np.array_equal(out[:total], oracle.dispatch_bf16(x, ref["pos"])[:total])
    y = make_expert_outputs(T * k, hidden, seed=hidden + 1)
    w = rng.uniform(-1, 1, size=(T, k)).astype(np.float32)
    comb = host_bits(h.combine(dev_bf16(y), dev_f32(w)))
    want, mag = oracle.combine(y, w, ref["pos"], return_magnitude=True)
    assert_combine_close(comb, want, mag, k)


@pytest.mark.parametrize("hidden", [128, 16384 + 128])
def test_hidden_extremes_fp8(hidden):
    """FP8 and MXFP8 dispatch at the smallest block-aligned row and a row whose
    last 1024-channel slice holds one 128-channel block."""
    print(f"[hidden] fp8 H={hidden}", flush=True)
    T, k, E, R = 500, 8, 64, 8
    rng = np.random.default_rng(hidden)
    idx = edge_ids(T, k, E, "random", seed=hidden)
    from workloads import bf16_bits_from_f32
    xf = rng.standard_normal((T, hidden)).astype(np.float32) * np.exp2(
        rng.integers(-30, 30, size=(T, hidden // 128, 1))).repeat(128, axis=2).reshape(T, hidden)
    x = bf16_bits_from_f32(xf.astype(np.float32))
    h = Handle(T, hidden, k, E, R)
    h.layout(dev_i32(idx))
    ref = oracle.layout(idx, E, R)
    codes, scales = h.dispatch(dev_bf16(x), fp8=True)
    rc, rs = oracle.dispatch_fp8(x, ref["pos"])
    assert np.array_equal(host_bits(codes), rc)
    assert np.array_equal(host_bits(scales).view(np.uint32), rs.view(np.uint32))
    codes, scales = h.dispatch(dev_bf16(x), mxfp8=True)
    rc, rs = oracle.dispatch_mxfp8(x, ref["pos"])
    assert np.array_equal(host_bits(codes), rc)
    assert np.array_equal(host_bits(scales), rs)


def test_large_token_count_layout():
    T, k, E, R = 65536, 8, 256, 8
    idx = edge_ids(T, k, E, "random", seed=4)
    got = layout_on_gpu(Handle(T, 128, k, E, R), idx)
    ref = oracle.layout(idx, E, R)
    assert_layout_equal(got, ref, T, k)


# Slot counts at the layout's workgroup boundaries: one workgroup with 2, 4 or
# 8 steps of 64 slots per wavefront up to 1024 / 2048 / 4096 slots, then
# workgroups of 1024 slots (a ragged last one included), in one launch up to
# 24 of them and in two (histograms, then placement) from 25 on.
BOUNDARY_SLOTS = (1023, 1024, 1025, 2047, 2048, 2049, 4095, 4096, 4097, 5120, 8191,
                  24575, 24576, 24577)


@pytest.mark.parametrize("slots", BOUNDARY_SLOTS)
def test_layout_at_workgroup_boundaries(slots):
    k = 1 if slots % 8 else 8
    T = slots // k
    for E, R, pattern, seed in ((256, 8, "random", 1), (16, 4, "invalid", 2), (64, 8, "const", 3)):
        print(f"[boundary] slots={T * k} T={T} k={k} E={E} {pattern}", flush=True)
        idx = edge_ids(T, k, E, pattern, seed=seed)
        got = layout_on_gpu(Handle(T, 128, k, E, R), idx)
        assert_layout_equal(got, oracle.layout(idx, E, R), T, k)


def test_layout_reuse_with_fewer_tokens():
    """A handle sized for T_max serves a smaller batch after a larger one."""
    h = Handle(4096, 256, 8, 256, 8)
    for T, seed in ((4096, 1), (1000, 2), (17, 3)):
        idx = edge_ids(T, 8, 256, "random", seed=seed)
        got = layout_on_gpu(h, idx)
        assert_layout_equal(got, oracle.layout(idx, 256, 8), T, 8)


# ---------------------------------------------------------------- dispatch

@pytest.mark.parametrize("name", NAMES)
def test_dispatch_bf16_matches_oracle(name):
    wl = make_workload(name)
    s = wl.shape
    ref = oracle.layout(wl.topk_idx, s.experts, s.ranks)
    h = handle(s)
    h.layout(dev_i32(wl.topk_idx))
    out = host_bits(h.dispatch(dev_bf16(wl.x_bits)))
    want = oracle.dispatch_bf16(wl.x_bits, ref["pos"])
    assert np.array_equal(out, want)


@pytest.mark.parametrize("name", NAMES)
def test_dispatch_fp8_matches_oracle(name):
    wl = make_workload(name)
    s = wl.shape
    ref = oracle.layout(wl.topk_idx, s.experts, s.ranks)
    h = handle(s)
    h.layout(dev_i32(wl.topk_idx))
    codes, scales = h.dispatch(dev_bf16(wl.x_bits), fp8=True)
    rc, rs = oracle.dispatch_fp8(wl.x_bits, ref["pos"])
    assert np.array_equal(host_bits(codes), rc)
    assert np.array_equal(host_bits(scales).view(np.uint32), rs.view(np.uint32))


def fp8_sweep_blocks():
    """128-channel blocks: channel 0 holds amax, the rest sweep bf16 values.

    For every amax significand (128 values, exponent 0) and a few amax values
    at other exponents (large, small, bf16 subnormal), the swept values take
    every significand and both signs over the 22 binades below amax, which
    covers every E4M3 code, every rounding tie and the subnormal E4M3 range.
    """
    amaxes = [(127 << 7) | m for m in range(128)]                    # [1, 2)
    amaxes += [((127 + 100) << 7) | 0x35, ((127 - 60) << 7) | 0x11,
               (1 << 7) | 0x7F, (0 << 7) | 0x45, (0xFE << 7) | 0x7F, (127 << 7) | 0x60]
    blocks = []
    for a in amaxes:
        ea = a >> 7
        cand = []
        for e in range(max(ea - 22, 0), ea + 1):
            m = np.arange(128, dtype=np.uint32)
            cand.append((e << 7) | m)
        cand = np.concatenate(cand).astype(np.uint32)
        cand = cand[cand <= a]
        cand = np.concatenate([cand, cand | 0x8000, [0, 0x8000]]).astype(np.uint16)
        for i in range(0, cand.size, 127):
            chunk = cand[i:i + 127]
            blk = np.zeros(128, dtype=np.uint16)
            blk[0] = a
            blk[1:1 + chunk.size] = chunk
            blocks.append(blk)
    blocks.append(np.zeros(128, np.uint16))
    blocks.append(np.full(128, 0x8000, np.uint16))
    return np.stack(blocks)


def test_fp8_quantiser_sweep():
    blocks = fp8_sweep_blocks()
    H = 7168
    per_row = H // 128
    T = -(-blocks.shape[0] // per_row)
    x = np.zeros((T * per_row, 128), dtype=np.uint16)
    x[:blocks.shape[0]] = blocks
    x = x.reshape(T, H)
    print(f"[fp8 sweep] {blocks.shape[0]} blocks, T={T}", flush=True)
    E, R, k = 8, 2, 2
    idx = edge_ids(T, k, E, "random", seed=9)
    ref = oracle.layout(idx, E, R)
    h = Handle(T, H, k, E, R)
    h.layout(dev_i32(idx))
    codes, scales = h.dispatch(dev_bf16(x), fp8=True)
    rc, rs = oracle.dispatch_fp8(x, ref["pos"])
    gc, gs = host_bits(codes), host_bits(scales)
    mism = np.argwhere(gc != rc)
    assert mism.size == 0, f"{len(mism)} code mismatches, first at {mism[:3].tolist()}"
    assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32))


# ---------------------------------------------------------------- combine

@pytest.mark.parametrize("name", NAMES)
def test_combine_matches_oracle(name):
    wl = make_workload(name)
    s = wl.shape
    ref = oracle.layout(wl.topk_idx, s.experts, s.ranks)
    C = s.tokens * s.topk
    y = make_expert_outputs(C, s.hidden, seed=wl.seed + 1)
    h = handle(s)
    h.layout(dev_i32(wl.topk_idx))
    got = host_bits(h.combine(dev_bf16(y), dev_f32(wl.topk_w)))
    # Every token is compared; the oracle runs over token chunks so that its
    # fp64 intermediates stay small at the largest shape.
    rel, exact = 0.0, []
    chunk = 2048
    for t0 in range(0, s.tokens, chunk):
        toks = np.arange(t0, min(t0 + chunk, s.tokens))
        want, mag = oracle.combine(y, wl.topk_w, ref["pos"], tokens=toks, return_magnitude=True)
        r, e = assert_combine_close(got[toks], want, mag, s.topk)
        rel = max(rel, r)
        exact.append(e * toks.size)
    print(f"[combine {name}] all {s.tokens} tokens: max rel err {rel:.3e}, bitwise-equal fraction "
          f"{sum(exact) / s.tokens:.5f}", flush=True)
    assert rel <= 1e-2


@pytest.mark.parametrize("name", NAMES)
def test_identity_experts_round_trip(name):
    """combine(dispatch(x)) with weights summing to 1 returns x bit for bit,
    except that -0.0 comes back as +0.0 (the weighted sum starts from +0)."""
    wl = make_workload(name)
    s = wl.shape
    h = handle(s)
    h.layout(dev_i32(wl.topk_idx))
    y = h.dispatch(dev_bf16(wl.x_bits))
    got = host_bits(h.combine(y, dev_f32(wl.topk_w)))
    want = np.where(wl.x_bits == 0x8000, np.uint16(0), wl.x_bits)
    assert np.array_equal(got, want)


def test_fp8_pipeline_round_trip():
    """FP8 dispatch -> expert-side dequant (torch, on the GPU) -> combine."""
    wl = make_workload("deepseekv3_fp8")
    s = wl.shape
    ref = oracle.layout(wl.topk_idx, s.experts, s.ranks)
    h = handle(s)
    h.layout(dev_i32(wl.topk_idx))
    codes, scales = h.dispatch(dev_bf16(wl.x_bits), fp8=True)
    deq = (codes.view(torch.float8_e4m3fn).float().view(codes.shape[0], -1, 128)
           * scales[:, :, None]).view(codes.shape[0], -1).to(torch.bfloat16)
    got = host_bits(h.combine(deq, dev_f32(wl.topk_w)))
    rc, rs = oracle.dispatch_fp8(wl.x_bits, ref["pos"])
    # The expert-side dequantisation of every row, in row chunks (its fp64
    # intermediates would otherwise take several GB), then every token.
    C = rc.shape[0]
    y_ref = np.empty(rc.shape, dtype=np.uint16)
    for r0 in range(0, C, 4096):
        y_ref[r0:r0 + 4096] = oracle.dequant_fp8(rc[r0:r0 + 4096], rs[r0:r0 + 4096])
    for t0 in range(0, s.tokens, 1024):
        toks = np.arange(t0, min(t0 + 1024, s.tokens))
        want, mag = oracle.combine(y_ref, wl.topk_w, ref["pos"], tokens=toks, return_magnitude=True)
        # torch's dequant rounds the fp32 product (double rounding vs the oracle's
        # single rounding): allow one more bf16 half-ulp of the inputs in mag
        rel, _ = assert_combine_close(got[toks], want, mag * (1 + 2.0 ** -8), s.topk)
        assert rel <= 1e-2
        x = (wl.x_bits[toks].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        g = (got[toks].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        s_tok = rs[ref["pos"][toks, 0]].astype(np.float64).repeat(128, axis=1)
        assert np.all(np.abs(g - x) <= (2.0 ** -4 + 2.0 ** -7) * np.abs(x) + 2.0 ** -9 * s_tok + 1e-6)


@pytest.mark.parametrize("cap", [1, 7, 64, 300, 511, 512, 700])
def test_workgroup_cap_gives_identical_results(cap):
    """Capping the grid only changes how many items each wavefront loops over.

    The bf16 dispatch changes form at a cap of 512 workgroups (one wavefront
    per item with all k slots below it, the slots spread over a workgroup
    from it on); 600 tokens x 14 slices keep every cap here below the item
    count, so both forms loop."""
    wl = make_workload("deepseekv3", tokens=600)
    s = wl.shape
    h = handle(s)
    x, idx, w = dev_bf16(wl.x_bits), dev_i32(wl.topk_idx), dev_f32(wl.topk_w)
    y = dev_bf16(make_expert_outputs(s.tokens * s.topk, s.hidden, seed=7))
    h.layout(idx)
    ref = [h.dispatch(x).view(torch.int16), *h.dispatch(x, fp8=True), *h.dispatch(x, mxfp8=True),
           h.combine(y, w).view(torch.int16)]
    h.set_max_workgroups(cap)
    got = [h.dispatch(x).view(torch.int16), *h.dispatch(x, fp8=True), *h.dispatch(x, mxfp8=True),
           h.combine(y, w).view(torch.int16)]
    h.set_max_workgroups(0)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    lay = oracle.layout(wl.topk_idx, s.experts, s.ranks)
    assert np.array_equal(host_bits(got[0].view(torch.bfloat16)), oracle.dispatch_bf16(wl.x_bits, lay["pos"]))


# ---------------------------------------------------------------- determinism, streams, errors

def test_bitwise_deterministic_reruns():
    wl = make_workload("deepseekv3")
    s = wl.shape
    h = handle(s)
    x = dev_bf16(wl.x_bits)
    idx = dev_i32(wl.topk_idx)
    w = dev_f32(wl.topk_w)
    y = dev_bf16(make_expert_outputs(s.tokens * s.topk, s.hidden, seed=5))
    first = None
    for _ in range(3):
        h.layout(idx)
        v = {k: t.clone() for k, t in h.view().items()}
        d = h.dispatch(x)
        q, sc = h.dispatch(x, fp8=True)
        mq, ms = h.dispatch(x, mxfp8=True)
        c = h.combine(y, w)
        torch.cuda.synchronize()
        cur = [v["pos"], v["src_idx"], v["counts_e"], d.view(torch.int16), q, sc.view(torch.int32),
               mq, ms, c.view(torch.int16)]
        if first is None:
            first = cur
        else:
            for a, b in zip(first, cur):
                assert torch.equal(a, b)


def test_runs_on_a_side_stream():
    wl = make_workload("deepseek16b")
    s = wl.shape
    h = handle(s)
    x, idx, w = dev_bf16(wl.x_bits), dev_i32(wl.topk_idx), dev_f32(wl.topk_w)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        h.layout(idx)
        y = h.dispatch(x)
        out = h.combine(y, w)
    side.synchronize()
    assert np.array_equal(host_bits(out), np.where(wl.x_bits == 0x8000, np.uint16(0), wl.x_bits))


def test_host_errors_enqueue_nothing():
    wl = make_workload("tiny")
    s = wl.shape
    h = handle(s)
    h.layout(dev_i32(wl.topk_idx))
    x = dev_bf16(wl.x_bits)
    small = torch.empty((s.tokens * s.topk - 1, s.hidden), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(MoeError, match="capacity"):
        h.dispatch(x, out=small)
    h2 = Handle(64, 200, 2, 8, 2)
    h2.layout(dev_i32(np.zeros((4, 2), np.int32)))
    with pytest.raises(MoeError, match="multiple of 128"):
        h2.dispatch(dev_bf16(np.zeros((4, 200), np.uint16)), fp8=True)
    with pytest.raises(MoeError, match="multiple of 128"):
        h2.dispatch(dev_bf16(np.zeros((4, 200), np.uint16)), mxfp8=True)
    with pytest.raises(MoeError, match="capacity"):
        h.combine(small, dev_f32(wl.topk_w))
    torch.cuda.synchronize()


def test_binding_rejects_mis_shaped_tensors():
    """The library sees only pointers; the binding refuses tensors whose shape
    does not match the handle's configuration (which the kernels would read or
    write out of bounds), before any call reaches the GPU."""
    wl = make_workload("tiny")
    s = wl.shape
    T, H, k, E = s.tokens, s.hidden, s.topk, s.experts
    S = T * k
    h = handle(s)
    idx, w, x = dev_i32(wl.topk_idx), dev_f32(wl.topk_w), dev_bf16(wl.x_bits)

    def empty(shape, dtype):
        return torch.empty(shape, dtype=dtype, device="cuda")

    bf, u8, f32, i32 = torch.bfloat16, torch.uint8, torch.float32, torch.int32
    with pytest.raises(ValueError, match="topk_idx"):
        h.layout(empty((T, k + 1), i32))
    with pytest.raises(ValueError, match="topk_idx"):
        h.rank_layout(empty((T, k + 1), i32))
    h.layout(idx)
    h.rank_layout(idx)
    bad = [
        lambda: h.dispatch(empty((T - 1, H), bf)),                       # x: too few tokens
        lambda: h.dispatch(empty((T, H - 8), bf)),                       # x: wrong width
        lambda: h.dispatch(x, out=empty((S, H - 8), bf)),
        lambda: h.dispatch(x, fp8=True, scales=empty((S, H // 128 - 1), f32)),
        lambda: h.dispatch(x, fp8=True, scales=empty((S - 1, H // 128), f32)),
        lambda: h.dispatch(x, mxfp8=True, scales=empty((S, H // 32 - 1), u8)),
        lambda: h.combine(empty((S, H - 8), bf), w),
        lambda: h.combine(empty((S, H), bf), empty((T, k - 1), f32)),
        lambda: h.combine(empty((S, H), bf), empty((T - 1, k), f32)),
        lambda: h.combine(empty((S, H), bf), w, out=empty((T - 1, H), bf)),
        lambda: h.route(empty((T, E - 1), f32)),
        lambda: h.route(empty((T, E), f32), topk_w=empty((T - 1, k), f32)),
        lambda: h.dispatch_ranks(x, idx, empty((T, k - 1), f32)),
        lambda: h.dispatch_ranks(x, idx, w, recv_idx=empty((h.rank_capacity - 1, k), i32)),
        lambda: h.combine_ranks(empty((h.rank_capacity, H), bf), out=empty((T - 1, H), bf)),
        lambda: h.layout_dispatch(empty((T, k - 1), i32), x),
        lambda: h.ll_dispatch(idx, empty((T - 1, H), bf), 8),
        lambda: h.ll_dispatch(idx, x, 8, "fp8", scales=empty((E * 8 - 1, H // 128), f32)),
    ]
    for call in bad:
        with pytest.raises(ValueError):
            call()
    h.ll_dispatch(idx, x, 8)
    with pytest.raises(ValueError, match="w"):
        h.ll_combine(empty((E * 8, H), bf), empty((T - 1, k), f32))
    # nothing above reached the GPU: the handle's layout still gives the oracle's rows
    got = h.dispatch(x)
    torch.cuda.synchronize()
    ref = oracle.layout(wl.topk_idx, E, s.ranks)
    assert np.array_equal(host_bits(got), oracle.dispatch_bf16(wl.x_bits, ref["pos"]))
