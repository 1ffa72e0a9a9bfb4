"""GPU parity of the decode-time (fixed-capacity) dispatch and combine.

Bar: positions, per-expert counts and status bit-exact against
oracle.layout_fixed_capacity; dispatched bf16 rows, FP8 and MXFP8 codes and
scales bit-exact on every row a slot maps to, and no other row written;
combine within the combine tolerance. Covers the DeepSeek-V3 decode shape
(128 tokens, H 7168, top-8 of 256), capacities that drop slots, invalid ids,
the 1024-token limit, empty batches and the workgroup cap.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_dispatch_02_amd import Handle, MoeError
from workloads import bf16_bits_from_f32, make_expert_outputs
from routed import make_workload
from gpu_util import assert_combine_close, dev_bf16, dev_f32, dev_i32, host_bits

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A5A


def ll_case(h, idx, x_bits, C, dtype):
    E = h.num_experts
    rows = E * C
    if dtype == "bf16":
        out = torch.full((rows, h.hidden), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        scales = None
        h.ll_dispatch(dev_i32(idx), dev_bf16(x_bits), C, "bf16", out=out)
    else:
        out = torch.full((rows, h.hidden), 0x5A, dtype=torch.uint8, device="cuda")
        if dtype == "fp8":
            scales = torch.full((rows, h.hidden // 128), 0x5A5A5A5A, dtype=torch.int32,
                                device="cuda").view(torch.float32)
        else:
            scales = torch.full((rows, h.hidden // 32), 0x5A, dtype=torch.uint8, device="cuda")
        h.ll_dispatch(dev_i32(idx), dev_bf16(x_bits), C, dtype, out=out, scales=scales)
    torch.cuda.synchronize()
    v = h.ll_view()
    ref = oracle.layout_fixed_capacity(idx, E, C)
    T = idx.shape[0]
    assert np.array_equal(v["pos"].cpu().numpy().astype(np.int64), ref["pos"]), "pos"
    assert np.array_equal(v["counts"].cpu().numpy(), ref["counts"]), "counts"
    st = v["status"].cpu().numpy().tolist()
    placed = int((ref["pos"] >= 0).sum())
    assert st == [ref["invalid"], placed, T, ref["dropped"]], st
    written = np.zeros(rows, bool)
    written[ref["pos"][ref["pos"] >= 0]] = True
    if dtype == "bf16":
        got = host_bits(out)
        want = oracle.dispatch_bf16(x_bits, ref["pos"], rows=rows)
        assert np.array_equal(got[written], want[written])
        assert np.all(got[~written] == SENTINEL)
    else:
        fn = oracle.dispatch_fp8 if dtype == "fp8" else oracle.dispatch_mxfp8
        rc, rs = fn(x_bits, ref["pos"], rows=rows)
        gc = host_bits(out)
        assert np.array_equal(gc[written], rc[written])
        assert np.all(gc[~written] == 0x5A)
        gs = scales.cpu().numpy()
        if dtype == "fp8":
            assert np.array_equal(gs[written].view(np.uint32), rs[written].view(np.uint32))
            assert np.all(gs[~written].view(np.uint32) == 0x5A5A5A5A)
        else:
            assert np.array_equal(gs[written], rs[written])
            assert np.all(gs[~written] == 0x5A)
    return ref


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "mxfp8"])
@pytest.mark.parametrize("C", [128, 5])
def test_decode_shape(dtype, C):
    """DeepSeek-V3 decode step: 128 tokens, H 7168, top-8 of 256 experts."""
    wl = make_workload("deepseekv3", tokens=128)
    s = wl.shape
    print(f"[ll] deepseekv3 T=128 C={C} {dtype}", flush=True)
    h = Handle(128, s.hidden, s.topk, s.experts, s.ranks)
    ref = ll_case(h, wl.topk_idx, wl.x_bits, C, dtype)
    if C == 128:
        assert ref["dropped"] == 0


@pytest.mark.parametrize("case", [
    ("skewed_drops", 300, 4, 16, 3, "zipf"), ("invalid_ids", 257, 8, 64, 8, "invalid"),
    ("one_expert", 100, 2, 8, 7, "const"), ("k_max", 64, 32, 64, 40, "random"),
    ("max_tokens", 1024, 8, 256, 64, "random"), ("capacity_one", 200, 6, 32, 1, "random"),
    ("single_token", 1, 8, 256, 2, "random"), ("max_experts", 500, 8, 1024, 4, "random"),
], ids=lambda c: c[0])
def test_edge_cases(case):
    name, T, k, E, C, pattern = case
    print(f"[ll edge] {name} T={T} k={k} E={E} C={C}", flush=True)
    rng = np.random.default_rng(T + k + E)
    if pattern == "const":
        idx = np.full((T, k), 3, np.int32)
    elif pattern == "zipf":
        p = np.arange(1, E + 1) ** -1.5
        idx = rng.choice(E, size=(T, k), p=p / p.sum()).astype(np.int32)
    else:
        idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
        if pattern == "invalid":
            bad = rng.random((T, k)) < 0.2
            idx[bad] = rng.choice(np.array([-1, E, -99, 2 ** 31 - 1]), size=int(bad.sum()))
    H = 256
    x = bf16_bits_from_f32(rng.standard_normal((T, H)).astype(np.float32))
    h = Handle(T, H, k, E, 1 if E % 8 else 8)
    for dtype in ("bf16", "fp8", "mxfp8"):
        ref = ll_case(h, idx, x, C, dtype)
    y = make_expert_outputs(E * C, H, seed=4)
    w = rng.uniform(-1, 1, size=(T, k)).astype(np.float32)
    got = host_bits(h.ll_combine(dev_bf16(y), dev_f32(w)))
    want, mag = oracle.combine(y, w, ref["pos"], return_magnitude=True)
    assert_combine_close(got, want, mag, k)


def test_empty_batch_publishes_zero_counts():
    h = Handle(16, 128, 2, 8, 2)
    h.ll_dispatch(dev_i32(np.full((16, 2), 1, np.int32)), dev_bf16(np.zeros((16, 128), np.uint16)), 4)
    h.ll_dispatch(torch.empty((0, 2), dtype=torch.int32, device="cuda"),
                  torch.empty((0, 128), dtype=torch.bfloat16, device="cuda"), 4)
    torch.cuda.synchronize()
    v = h.ll_view()
    assert v["pos"].numel() == 0
    assert v["counts"].cpu().numpy().tolist() == [0] * 8
    assert v["status"].cpu().numpy().tolist() == [0, 0, 0, 0]
    out = h.ll_combine(torch.zeros((32, 128), dtype=torch.bfloat16, device="cuda"),
                       torch.empty((0, 2), dtype=torch.float32, device="cuda"))
    assert out.shape == (0, 128)


def test_matches_standard_slabs_without_drops():
    """With capacity >= every expert's count, expert e's first counts[e] rows equal
    its slab of the standard expert-major buffer."""
    wl = make_workload("deepseek16b", tokens=512)
    s = wl.shape
    h = Handle(512, s.hidden, s.topk, s.experts, s.ranks)
    x, idx = dev_bf16(wl.x_bits), dev_i32(wl.topk_idx)
    h.layout(idx)
    std = h.dispatch(x)
    off = h.view()["offsets_e"].cpu().numpy()
    C = int(np.diff(off).max())
    ll = h.ll_dispatch(idx, x, C)
    torch.cuda.synchronize()
    counts = h.ll_view()["counts"].cpu().numpy()
    assert np.array_equal(counts, np.diff(off))
    for e in range(s.experts):
        n = int(counts[e])
        assert torch.equal(ll[e * C:e * C + n].view(torch.int16),
                           std[int(off[e]):int(off[e]) + n].view(torch.int16)), e


@pytest.mark.parametrize("cap", [1, 5, 50])
def test_workgroup_cap_gives_identical_results(cap):
    wl = make_workload("deepseekv3", tokens=128)
    s = wl.shape
    h = Handle(128, s.hidden, s.topk, s.experts, s.ranks)
    x, idx, w = dev_bf16(wl.x_bits), dev_i32(wl.topk_idx), dev_f32(wl.topk_w)
    y = dev_bf16(make_expert_outputs(s.experts * 16, s.hidden, seed=3))
    rows = s.experts * 16

    def run():
        # zero-filled outputs: rows that no slot maps to are never written
        out = torch.zeros((rows, s.hidden), dtype=torch.bfloat16, device="cuda")
        q = torch.zeros((rows, s.hidden), dtype=torch.uint8, device="cuda")
        qs = torch.zeros((rows, s.hidden // 128), dtype=torch.float32, device="cuda")
        h.ll_dispatch(idx, x, 16, out=out)
        h.ll_dispatch(idx, x, 16, "fp8", out=q, scales=qs)
        v = h.ll_view()
        return [out, q, qs, v["pos"].clone(), v["counts"].clone(), h.ll_combine(y, w)]

    ref = run()
    h.set_max_workgroups(cap)
    got = run()
    h.set_max_workgroups(0)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_host_errors():
    h = Handle(2048, 128, 2, 8, 2)
    x = torch.zeros((1025, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(MoeError, match="MOE_EP_LL_MAX_TOKENS"):
        h.ll_dispatch(torch.zeros((1025, 2), dtype=torch.int32, device="cuda"), x, 4)
    with pytest.raises(MoeError, match="capacity"):
        h.ll_dispatch(torch.zeros((4, 2), dtype=torch.int32, device="cuda"), x[:4], 0)
    torch.cuda.synchronize()
