"""moe_layout_dispatch (layout and dispatch in one launch, small batches)
against the two-call path and the oracle.

Bar: every layout array (pos, src_idx, counts and offsets per expert and per
rank, status) and every dispatched row (bf16, FP8 codes and scales, MXFP8
codes and scales) bit-exact against moe_dispatch_layout + moe_dispatch and
against the oracle; combine after it within the combine tolerance. Covers
both counting modes (below and from 256 tokens), invalid and duplicate ids,
a skewed routing, 1024 experts, top-32, the empty batch and the 1024-token
limit.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_dispatch_02_amd import Handle, MoeError
from workloads import bf16_bits_from_f32, make_expert_outputs
from gpu_util import assert_combine_close, assert_layout_equal, dev_bf16, dev_f32, dev_i32, host_bits

pytestmark = pytest.mark.gpu

CASES = [
    # name, T, k, E, R, H, pattern
    ("decode_v3", 128, 8, 256, 8, 7168, "uniform"),
    ("tiny", 7, 2, 8, 2, 256, "uniform"),
    ("one_token", 1, 8, 64, 8, 1024, "uniform"),
    ("below_shared", 255, 6, 64, 8, 2048, "skewed"),
    ("shared_from", 256, 6, 64, 8, 2048, "skewed"),
    ("invalid_ids", 700, 8, 256, 8, 1024, "invalid"),
    ("duplicates", 300, 4, 16, 4, 512, "duplicates"),
    ("max_experts", 400, 8, 1024, 8, 256, "uniform"),
    ("max_topk", 200, 32, 64, 8, 384, "uniform"),
    ("max_tokens", 1024, 8, 256, 8, 1024, "uniform"),
    ("empty", 0, 4, 16, 4, 256, "uniform"),
]


def ids_for(T, k, E, pattern, rng):
    if pattern == "uniform":
        return rng.integers(0, E, size=(T, k)).astype(np.int32)
    if pattern == "skewed":
        p = np.arange(1, E + 1, dtype=np.float64) ** -1.5
        return rng.choice(E, size=(T, k), p=p / p.sum()).astype(np.int32)
    if pattern == "duplicates":
        return rng.integers(0, max(1, E // 4), size=(T, k)).astype(np.int32)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    bad = rng.random((T, k)) < 0.2
    idx[bad] = rng.choice(np.array([-1, E, 1 << 20, -(1 << 30)]), size=int(bad.sum()))
    return idx


def arrays(h):
    torch.cuda.synchronize()
    return {k: v.cpu().numpy().astype(np.int64) for k, v in h.view().items()}


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_matches_two_call_path_and_oracle(case):
    name, T, k, E, R, H, pattern = case
    print(f"[layout_dispatch] {name} T={T} k={k} E={E} R={R} H={H}", flush=True)
    rng = np.random.default_rng(T * 131 + k)
    idx = ids_for(T, k, E, pattern, rng)
    x = bf16_bits_from_f32(rng.standard_normal((T, H)).astype(np.float32))
    fused, two = Handle(max(T, 1), H, k, E, R), Handle(max(T, 1), H, k, E, R)
    di, dx = dev_i32(idx), dev_bf16(x)
    ref = oracle.layout(idx, E, R)
    n = int(ref["offsets_e"][-1])
    for dtype in ("bf16", "fp8", "mxfp8"):
        got = fused.layout_dispatch(di, dx, dtype)
        two.layout(di)
        if dtype == "bf16":
            want = two.dispatch(dx)
        else:
            want = two.dispatch(dx, fp8=dtype == "fp8", mxfp8=dtype == "mxfp8")
        a, b = arrays(fused), arrays(two)
        for key in ("pos", "src_idx", "counts_e", "offsets_e", "counts_r", "offsets_r"):
            assert np.array_equal(a[key], b[key]), (dtype, key)
        assert np.array_equal(a["status"][:3], b["status"][:3]), dtype
        assert a["status"][3] == 0
        assert_layout_equal(a, ref, T, k)
        if dtype == "bf16":
            assert np.array_equal(host_bits(got)[:n], host_bits(want)[:n])
            assert np.array_equal(host_bits(got)[:n], oracle.dispatch_bf16(x, ref["pos"])[:n])
        else:
            for g, w_ in zip(got, want):
                assert torch.equal(g[:n].view(torch.uint8), w_[:n].view(torch.uint8)), dtype
            rc, rs = (oracle.dispatch_fp8 if dtype == "fp8" else oracle.dispatch_mxfp8)(x, ref["pos"])
            assert np.array_equal(host_bits(got[0])[:n], rc[:n])
    # the layout it leaves behind serves combine
    y = make_expert_outputs(max(T * k, 1), H, seed=T + 5)
    w = rng.uniform(-1, 1, size=(T, k)).astype(np.float32)
    fused.layout_dispatch(di, dx)
    comb = host_bits(fused.combine(dev_bf16(y), dev_f32(w)))
    want_c, mag = oracle.combine(y, w, ref["pos"], return_magnitude=True)
    assert_combine_close(comb, want_c, mag, k)


@pytest.mark.parametrize("cap", [1, 3, 40])
def test_workgroup_cap_gives_identical_results(cap):
    rng = np.random.default_rng(cap)
    T, k, E, R, H = 300, 8, 64, 8, 1024
    idx = dev_i32(rng.integers(0, E, size=(T, k)))
    x = dev_bf16(bf16_bits_from_f32(rng.standard_normal((T, H)).astype(np.float32)))
    h = Handle(T, H, k, E, R)

    def run():
        out = torch.zeros((T * k, H), dtype=torch.bfloat16, device="cuda")
        h.layout_dispatch(idx, x, out=out)
        v = {key: t.clone() for key, t in h.view().items()}
        return [out, v["pos"], v["src_idx"], v["offsets_e"], v["offsets_r"]]

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
        h.layout_dispatch(torch.zeros((1025, 2), dtype=torch.int32, device="cuda"), x)
    torch.cuda.synchronize()
