"""Pins for the oracle's layout (histogram, exclusive scan, stable placement).

Checks: hand-worked fixtures, numpy's stable argsort and bincount/cumsum
(library routines for the same counting sort), O(S^2) brute force on tiny
inputs, and the invariants (counts sum to T*k, pos is a bijection onto the
valid rows, per-expert order is stable by token index).
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import layout
from workloads import CONFIGS
from routed import make_workload
from conftest import load_golden


@pytest.mark.parametrize("case", load_golden("layout_hand.json")["cases"], ids=lambda c: c["name"])
def test_layout_hand_worked(case):
    got = layout(np.array(case["topk_idx"], dtype=np.int32), case["num_experts"], case["num_ranks"])
    for key in ("counts_e", "offsets_e", "counts_r", "offsets_r", "pos", "src_idx"):
        assert got[key].tolist() == case[key], key
    assert got["invalid"] == case["invalid"]


def check_against_stable_argsort(idx, E, R, lay):
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    order = np.argsort(flat, kind="stable")          # rows in expert-major, slot order
    inv = np.empty_like(order)
    inv[order] = np.arange(order.size)
    assert np.array_equal(lay["pos"].reshape(-1), inv)
    assert np.array_equal(lay["src_idx"], order // k)
    counts = np.bincount(flat, minlength=E)
    assert np.array_equal(lay["counts_e"], counts)
    assert np.array_equal(lay["offsets_e"], np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(lay["counts_r"], counts.reshape(R, E // R).sum(axis=1))
    assert np.array_equal(lay["offsets_r"], lay["offsets_e"][::E // R])
    assert lay["counts_e"].sum() == T * k and lay["invalid"] == 0


@pytest.mark.parametrize("shape", CONFIGS, ids=lambda s: s.name)
def test_layout_matches_stable_argsort_on_workloads(shape):
    wl = make_workload(shape.name)
    lay = layout(wl.topk_idx, shape.experts, shape.ranks)
    check_against_stable_argsort(wl.topk_idx, shape.experts, shape.ranks, lay)
    # stability: inside each expert's rows, token index never decreases
    src, off = lay["src_idx"], lay["offsets_e"]
    for e in range(shape.experts):
        seg = src[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) >= 0)


def brute_force(idx, E, R):
    """O(S^2): row of each slot = #valid slots of lower expert + #earlier slots of same expert."""
    T, k = idx.shape
    flat = [int(v) for v in idx.reshape(-1)]
    S = len(flat)
    pos = []
    for s, e in enumerate(flat):
        if not 0 <= e < E:
            pos.append(-1)
            continue
        lower = sum(1 for f in flat if 0 <= f < e)
        earlier = sum(1 for f in flat[:s] if f == e)
        pos.append(lower + earlier)
    src = [-1] * S
    for s, p in enumerate(pos):
        if p >= 0:
            src[p] = s // k
    counts = [sum(1 for f in flat if f == e) for e in range(E)]
    return np.array(pos).reshape(T, k), np.array(src), np.array(counts)


@settings(max_examples=150, deadline=None)
@given(st.data())
def test_layout_brute_force_tiny(data):
    R = data.draw(st.integers(1, 4))
    E = R * data.draw(st.integers(1, 4))
    T = data.draw(st.integers(0, 12))
    k = data.draw(st.integers(1, 4))
    # include invalid ids (-1, E, large) and duplicates
    ids = data.draw(st.lists(st.integers(-2, E + 1), min_size=T * k, max_size=T * k))
    idx = np.array(ids, dtype=np.int32).reshape(T, k)
    lay = layout(idx, E, R)
    pos, src, counts = brute_force(idx, E, R)
    assert np.array_equal(lay["pos"], pos)
    assert np.array_equal(lay["src_idx"], src)
    assert np.array_equal(lay["counts_e"], counts)
    valid = int(((idx >= 0) & (idx < E)).sum())
    assert lay["invalid"] == T * k - valid
    assert lay["offsets_e"][-1] == valid
    # pos is a bijection from valid slots onto rows [0, valid)
    p = lay["pos"].reshape(-1)
    assert sorted(p[p >= 0].tolist()) == list(range(valid))


def test_layout_all_tokens_one_expert_and_empty():
    idx = np.full((50, 1), 3, dtype=np.int32)
    lay = layout(idx, 8, 2)
    assert lay["counts_e"].tolist() == [0, 0, 0, 50, 0, 0, 0, 0]
    assert lay["pos"].reshape(-1).tolist() == list(range(50))
    assert lay["counts_r"].tolist() == [50, 0]
    empty = layout(np.zeros((0, 4), dtype=np.int32), 8, 4)
    assert empty["offsets_e"].tolist() == [0] * 9 and empty["src_idx"].size == 0


def test_layout_rejects_bad_rank_split():
    with pytest.raises(ValueError):
        layout(np.zeros((2, 2), dtype=np.int32), 6, 4)
