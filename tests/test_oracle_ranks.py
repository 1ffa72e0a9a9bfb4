"""Pins for the oracle's rank-deduplicated exchange (CPU only).

Checks: hand-worked fixtures, numpy set operations for which ranks a token
touches, O(T^2) brute force of the rank rows, and the composition invariant
that ties it to the (separately pinned) expert layout: expanding rank r's
rows on the receiver with the expert layout over its local experts gives
exactly the standard dispatch's rows of rank r.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle.codecs import bf16_decode
from workloads import CONFIGS, make_expert_outputs
from routed import make_workload
from conftest import combine_tolerance, load_golden


@pytest.mark.parametrize("case", load_golden("layout_hand.json")["cases"], ids=lambda c: c["name"])
def test_rank_layout_hand_worked(case):
    idx = np.array(case["topk_idx"], dtype=np.int32)
    E, R = case["num_experts"], case["num_ranks"]
    rl = oracle.rank_layout(idx, E, R)
    want = case["rank"]
    for key in ("in_rank", "counts_r", "offsets_r", "rank_pos", "rank_src"):
        assert rl[key].tolist() == want[key], key
    x = np.arange(idx.shape[0] * 8, dtype=np.uint16).reshape(idx.shape[0], 8)
    w = np.arange(idx.size, dtype=np.float32).reshape(idx.shape) + 1
    _, recv_idx, _ = oracle.dispatch_ranks(x, idx, w, E, R, rl)
    assert recv_idx.tolist() == want["recv_idx"]


def test_rank_layout_matches_numpy_sets():
    for shape in CONFIGS:
        wl = make_workload(shape.name, tokens=min(shape.tokens, 1024))
        E, R = shape.experts, shape.ranks
        rl = oracle.rank_layout(wl.topk_idx, E, R)
        T = wl.topk_idx.shape[0]
        in_rank = np.zeros((T, R), dtype=np.int64)
        in_rank[np.repeat(np.arange(T), shape.topk), (wl.topk_idx // (E // R)).reshape(-1)] = 1
        assert np.array_equal(rl["in_rank"], in_rank)
        assert np.array_equal(rl["counts_r"], in_rank.sum(axis=0))
        assert np.array_equal(rl["offsets_r"], np.concatenate([[0], np.cumsum(in_rank.sum(axis=0))]))
        # stable: numpy's stable argsort of (rank, token) pairs
        pairs = np.argwhere(in_rank.T == 1)                  # sorted by rank, then token
        assert np.array_equal(rl["rank_src"][:len(pairs)], pairs[:, 1])
        assert np.all(rl["rank_src"][len(pairs):] == -1)


def test_rank_dedup_saves_rows_at_v3():
    wl = make_workload("deepseekv3")
    rl = oracle.rank_layout(wl.topk_idx, 256, 8)
    rows = int(rl["counts_r"].sum())
    # 8 experts spread over 8 ranks of 32: about 5.3 distinct ranks per token
    assert 5.0 * 4096 < rows < 5.6 * 4096
    assert rows < 0.7 * 4096 * 8


@settings(max_examples=120, deadline=None)
@given(st.data())
def test_rank_layout_brute_force(data):
    R = data.draw(st.integers(1, 4))
    E = R * data.draw(st.integers(1, 4))
    T = data.draw(st.integers(0, 10))
    k = data.draw(st.integers(1, 4))
    ids = data.draw(st.lists(st.integers(-2, E + 1), min_size=T * k, max_size=T * k))
    idx = np.array(ids, dtype=np.int32).reshape(T, k)
    rl = oracle.rank_layout(idx, E, R)
    per = E // R
    member = [[any(0 <= e < E and e // per == r for e in idx[t]) for r in range(R)] for t in range(T)]
    for t in range(T):
        for r in range(R):
            if member[t][r]:
                below = sum(member[u][rr] for u in range(T) for rr in range(R) if rr < r)
                earlier = sum(member[u][r] for u in range(t))
                assert rl["rank_pos"][t, r] == below + earlier
            else:
                assert rl["rank_pos"][t, r] == -1
    assert rl["rank_src"].size == T * min(k, R)


@pytest.mark.parametrize("name", [c.name for c in CONFIGS])
def test_receiver_expansion_equals_standard_rank_slab(name):
    wl = make_workload(name, tokens=256)
    s = wl.shape
    E, R, k = s.experts, s.ranks, s.topk
    per = E // R
    lay = oracle.layout(wl.topk_idx, E, R)
    std = oracle.dispatch_bf16(wl.x_bits, lay["pos"])
    rl = oracle.rank_layout(wl.topk_idx, E, R)
    rows, recv_idx, recv_w = oracle.dispatch_ranks(wl.x_bits, wl.topk_idx, wl.topk_w, E, R, rl)
    for r in range(R):
        a, b = rl["offsets_r"][r], rl["offsets_r"][r + 1]
        local = oracle.layout(recv_idx[a:b], per, 1)
        expanded = oracle.dispatch_bf16(rows[a:b], local["pos"])
        n = int(local["offsets_e"][-1])
        assert np.array_equal(local["counts_e"], lay["counts_e"][r * per:(r + 1) * per])
        assert np.array_equal(expanded[:n], std[lay["offsets_r"][r]:lay["offsets_r"][r + 1]])
        # weights travel with their slots
        assert np.array_equal(recv_w[a:b][recv_idx[a:b] >= 0],
                              wl.topk_w[rl["rank_src"][a:b]][recv_idx[a:b] >= 0])
    # every valid slot is carried exactly once
    assert int((recv_idx >= 0).sum()) == wl.topk_idx.size


def test_combine_ranks_end_to_end():
    wl = make_workload("deepseekv3", tokens=96, hidden=512)
    s = wl.shape
    E, R, k = s.experts, s.ranks, s.topk
    per = E // R
    rl = oracle.rank_layout(wl.topk_idx, E, R)
    rows, recv_idx, recv_w = oracle.dispatch_ranks(wl.x_bits, wl.topk_idx, wl.topk_w, E, R, rl)
    y_std = make_expert_outputs(96 * k, 512, seed=4)
    lay = oracle.layout(wl.topk_idx, E, R)
    ref, mag = oracle.combine(y_std, wl.topk_w, lay["pos"], return_magnitude=True)
    # receivers: expand, take the same expert outputs, reduce locally
    partial = np.zeros((rows.shape[0], 512), dtype=np.uint16)
    for r in range(R):
        a, b = rl["offsets_r"][r], rl["offsets_r"][r + 1]
        local = oracle.layout(recv_idx[a:b], per, 1)
        y_local = y_std[lay["offsets_r"][r]:lay["offsets_r"][r + 1]]
        partial[a:b] = oracle.combine(y_local, recv_w[a:b], local["pos"])
    got = oracle.combine_ranks(partial, rl["rank_pos"])
    gv = bf16_decode(got).astype(np.float64)
    rv = bf16_decode(ref).astype(np.float64)
    # two roundings (per-rank partials, then the sum) instead of one
    assert np.all(np.abs(gv - rv) <= combine_tolerance(ref, mag, k) + 2.0 ** -8 * mag)
    # a single rank reduces to the partial itself
    one = oracle.rank_layout(wl.topk_idx, E, 1)
    assert np.array_equal(oracle.combine_ranks(partial[:96], one["rank_pos"]), partial[:96])
