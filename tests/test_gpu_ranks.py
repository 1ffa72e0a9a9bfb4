"""GPU parity of the rank-deduplicated exchange (one row per (token, rank)).

Bar: rank layout arrays, dispatched rows and receiver metadata bit-exact
against the oracle; the receiver-side expansion (the library's own layout and
dispatch on a rank's rows, with E/R experts) reproduces the standard
expert-major rows of that rank bit for bit; combine of per-rank partials
within the combine tolerance; the end-to-end exchange within tolerance of
the direct combine (it rounds twice: per rank, then the sum).
"""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_dispatch_02_amd import Handle
from workloads import CONFIGS, make_expert_outputs
from routed import make_workload
from gpu_util import assert_combine_close, dev_bf16, dev_f32, dev_i32, host_bits

pytestmark = pytest.mark.gpu

NAMES = [c.name for c in CONFIGS]


def rank_view_np(h):
    torch.cuda.synchronize()
    return {k: v.cpu().numpy().astype(np.int64) for k, v in h.rank_view().items()}


def check_rank_layout(h, idx, E, R):
    T, k = idx.shape
    h.rank_layout(dev_i32(idx))
    got = rank_view_np(h)
    ref = oracle.rank_layout(idx, E, R)
    assert np.array_equal(got["rank_pos"], ref["rank_pos"]), "rank_pos"
    assert np.array_equal(got["counts_r"], ref["counts_r"]), "counts_r"
    assert np.array_equal(got["offsets_r"], ref["offsets_r"]), "offsets_r"
    assert np.array_equal(got["rank_src"], ref["rank_src"]), "rank_src"
    assert got["status"][0] == ref["offsets_r"][-1] and got["status"][1] == T
    # slot_row: the first slot of a token on a rank opens that (token, rank) row
    per = E // R
    want = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        seen = set()
        for j in range(k):
            e = int(idx[t, j])
            if 0 <= e < E and e // per not in seen:
                seen.add(e // per)
                want[t, j] = ref["rank_pos"][t, e // per]
    assert np.array_equal(got["slot_row"], want), "slot_row"
    return ref


@pytest.mark.parametrize("slots", (1024, 1025, 2048, 2049, 4096, 4097, 8191))
def test_rank_layout_at_workgroup_boundaries(slots):
    """Slot counts where the layout changes workgroup shape (one workgroup
    with 2, 4 or 8 steps per wavefront, then workgroups of 1024 slots)."""
    k = 1 if slots % 8 else 8
    T = slots // k
    E, R = 64, 8
    rng = np.random.default_rng(slots)
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    print(f"[rank boundary] slots={T * k} T={T} k={k}", flush=True)
    check_rank_layout(Handle(T, 128, k, E, R), idx, E, R)


@pytest.mark.parametrize("name", NAMES)
def test_rank_layout_and_dispatch_match_oracle(name):
    wl = make_workload(name)
    s = wl.shape
    h = Handle(s.tokens, s.hidden, s.topk, s.experts, s.ranks)
    ref = check_rank_layout(h, wl.topk_idx, s.experts, s.ranks)
    rows, ridx, rw = h.dispatch_ranks(dev_bf16(wl.x_bits), dev_i32(wl.topk_idx), dev_f32(wl.topk_w))
    want_rows, want_idx, want_w = oracle.dispatch_ranks(wl.x_bits, wl.topk_idx, wl.topk_w,
                                                        s.experts, s.ranks, ref)
    n = int(ref["offsets_r"][-1])
    assert np.array_equal(host_bits(rows)[:n], want_rows[:n])
    assert np.array_equal(ridx.cpu().numpy()[:n], want_idx[:n])
    assert np.array_equal(rw.cpu().numpy()[:n].view(np.uint32), want_w[:n].view(np.uint32))


@pytest.mark.parametrize("case", [
    ("k_above_R", 700, 8, 16, 2, "random"), ("R_equals_1", 300, 4, 16, 1, "random"),
    ("R_equals_E", 500, 4, 16, 16, "random"), ("invalid_ids", 900, 8, 64, 8, "invalid"),
    ("duplicates", 400, 4, 8, 4, "const"), ("empty", 0, 4, 16, 4, "random"),
    ("max_topk", 300, 32, 64, 8, "random"), ("ragged", 2049, 3, 32, 4, "random"),
], ids=lambda c: c[0])
def test_rank_edge_cases(case):
    name, T, k, E, R, pattern = case
    print(f"[rank edge] {name} T={T} k={k} E={E} R={R}", flush=True)
    rng = np.random.default_rng(3)
    if pattern == "const":
        idx = np.full((T, k), E - 1, dtype=np.int32)
    else:
        idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
        if pattern == "invalid":
            bad = rng.random((T, k)) < 0.2
            idx[bad] = rng.choice(np.array([-1, E, 2**31 - 1, -77]), size=int(bad.sum()))
    H = 128
    h = Handle(max(T, 1), H, k, E, R)
    ref = check_rank_layout(h, idx, E, R)
    x = rng.integers(0, 2**16, size=(T, H), dtype=np.uint16) & np.uint16(0x7F7F)
    w = rng.uniform(0, 1, size=(T, k)).astype(np.float32)
    rows, ridx, rw = h.dispatch_ranks(dev_bf16(x), dev_i32(idx), dev_f32(w))
    want_rows, want_idx, want_w = oracle.dispatch_ranks(x, idx, w, E, R, ref)
    n = int(ref["offsets_r"][-1])
    assert np.array_equal(host_bits(rows)[:n], want_rows[:n])
    assert np.array_equal(ridx.cpu().numpy()[:n], want_idx[:n])
    assert np.array_equal(rw.cpu().numpy()[:n].view(np.uint32), want_w[:n].view(np.uint32))
    y = make_expert_outputs(max(T * min(k, R), 1), H, seed=5)
    got = host_bits(h.combine_ranks(dev_bf16(y)))
    want, mag = oracle.combine_ranks(y, ref["rank_pos"], return_magnitude=True)
    assert_combine_close(got, want, mag, R)


@pytest.mark.parametrize("name", ["deepseekv3", "qwen3_skewed", "deepseek16b"])
def test_receiver_expansion_matches_standard_slabs(name):
    wl = make_workload(name)
    s = wl.shape
    E, R, k, H = s.experts, s.ranks, s.topk, s.hidden
    per = E // R
    h = Handle(s.tokens, H, k, E, R)
    x, idx, w = dev_bf16(wl.x_bits), dev_i32(wl.topk_idx), dev_f32(wl.topk_w)
    h.layout(idx)
    std = h.dispatch(x)
    std_off = h.view()["offsets_r"].cpu().numpy()
    h.rank_layout(idx)
    rows, ridx, rw = h.dispatch_ranks(x, idx, w)
    off = h.rank_view()["offsets_r"].cpu().numpy()
    for r in range(R):
        a, b = int(off[r]), int(off[r + 1])
        recv = Handle(max(b - a, 1), H, k, per, 1)
        recv.layout(ridx[a:b].contiguous())
        expanded = recv.dispatch(rows[a:b].contiguous())
        n = int(recv.view()["offsets_e"][-1].item())
        assert n == int(std_off[r + 1] - std_off[r])
        assert torch.equal(expanded[:n].view(torch.int16),
                           std[int(std_off[r]):int(std_off[r + 1])].view(torch.int16)), f"rank {r}"


def test_exchange_end_to_end():
    """dispatch_ranks -> per-rank expansion, expert outputs, local weighted
    combine -> combine_ranks, against the direct combine of the same outputs."""
    wl = make_workload("deepseekv3", tokens=1024)
    s = wl.shape
    E, R, k, H = s.experts, s.ranks, s.topk, s.hidden
    per = E // R
    h = Handle(s.tokens, H, k, E, R)
    x, idx, w = dev_bf16(wl.x_bits), dev_i32(wl.topk_idx), dev_f32(wl.topk_w)
    y_std = make_expert_outputs(s.tokens * k, H, seed=9)       # outputs in standard row order
    h.layout(idx)
    std_off = h.view()["offsets_r"].cpu().numpy()
    direct = host_bits(h.combine(dev_bf16(y_std), w))
    h.rank_layout(idx)
    rows, ridx, rw = h.dispatch_ranks(x, idx, w)
    off = h.rank_view()["offsets_r"].cpu().numpy()
    partial = torch.zeros_like(rows)
    for r in range(R):
        a, b = int(off[r]), int(off[r + 1])
        recv = Handle(max(b - a, 1), H, k, per, 1)
        recv.layout(ridx[a:b].contiguous())
        # the receiver's expert outputs, in a buffer sized for the worst case
        n = int(std_off[r + 1] - std_off[r])
        y_local = torch.zeros((recv.capacity, H), dtype=torch.bfloat16, device="cuda")
        y_local[:n] = dev_bf16(y_std[int(std_off[r]):int(std_off[r + 1])])
        partial[a:b] = recv.combine(y_local, rw[a:b].contiguous())
    got = host_bits(h.combine_ranks(partial))
    lay = oracle.layout(wl.topk_idx, E, R)
    ref, mag = oracle.combine(y_std, wl.topk_w, lay["pos"], return_magnitude=True)
    # each per-rank partial is rounded to bf16 before the sum: at most half a
    # bf16 ulp, i.e. 2^-8 relative, of that rank's sum of |w y|; 2^-8 * M in total
    rel, exact = assert_combine_close(got, ref, mag, k, extra=2.0 ** -8 * mag)
    print(f"[exchange] max rel err {rel:.3e}, equal to the oracle {exact:.3f}, "
          f"equal to the direct combine {np.mean(got == direct):.3f}", flush=True)
