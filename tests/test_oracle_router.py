"""Pins for the oracle's router (top-k selection and combine weights)."""
import itertools

import numpy as np
import pytest
import scipy.special

from oracle.router import route
from conftest import load_golden


def as_f32(values):
    return np.array([float(v) for v in values], dtype=np.float32)


@pytest.mark.parametrize("case", load_golden("router_hand.json")["cases"], ids=lambda c: c["name"])
def test_router_hand_worked(case):
    L = as_f32(case["logits"])[None, :]
    idx, w = route(L, case["k"], case["score"])
    assert idx.dtype == np.int32 and w.dtype == np.float32
    assert idx[0].tolist() == case["idx"]
    want = np.array(case["w"], dtype=np.float64)
    # the oracle rounds its fp64 weights once to fp32: within half an fp32 ulp
    assert np.all(np.abs(w[0].astype(np.float64) - want) <= 2.0 ** -24 * want * (1 + 1e-9))


def selection_ok(row, sel):
    """Top-k by value, descending, ties to the lower id (checked without sorting)."""
    k = len(sel)
    if len(set(sel)) != k:
        return False
    vals = [float(row[e]) for e in sel]
    for a in range(k - 1):
        if vals[a] < vals[a + 1] or (vals[a] == vals[a + 1] and sel[a] > sel[a + 1]):
            return False
    chosen = set(sel)
    for e in range(len(row)):
        if e in chosen:
            continue
        v = float(row[e])
        if v > vals[-1] or (v == vals[-1] and e < max(s for s, x in zip(sel, vals) if x == v)):
            return False
    return True


def test_selection_invariants_with_many_ties():
    rng = np.random.default_rng(31)
    T, E = 400, 24
    L = (rng.integers(-3, 4, size=(T, E)) / 2.0).astype(np.float32)
    L[rng.random((T, E)) < 0.1] = np.float32(-0.0)
    for k in (1, 3, 8, 24):
        idx, _ = route(L, k, "softmax")
        for t in range(T):
            assert selection_ok(L[t], idx[t].tolist()), (k, t)


def test_selection_brute_force_tiny():
    """Every logit vector over {-1, -0, +0, 1} for E=4: the selected set has the
    largest sum, the lexicographically smallest ids among such sets, and is
    listed by descending value with ties by ascending id."""
    vals = [-1.0, -0.0, 0.0, 1.0]
    rows = np.array(list(itertools.product(vals, repeat=4)), dtype=np.float32)
    for k in (1, 2, 3):
        idx, _ = route(rows, k, "sigmoid")
        for r, row in enumerate(rows):
            best = max(itertools.combinations(range(4), k),
                       key=lambda c: (sum(float(row[e]) for e in c), [-e for e in c]))
            want = sorted(best, key=lambda e: (-float(row[e]), e))
            assert idx[r].tolist() == want, (row.tolist(), k)


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_weights_match_scipy(score):
    rng = np.random.default_rng(7)
    L = rng.standard_normal((300, 64)).astype(np.float32) * 3
    idx, w = route(L, 8, score)
    sel = np.take_along_axis(L, idx, axis=1).astype(np.float64)
    ref = scipy.special.softmax(sel, axis=1) if score == "softmax" else \
        scipy.special.expit(sel) / scipy.special.expit(sel).sum(axis=1, keepdims=True)
    assert np.all(np.abs(w - ref) <= 2.0 ** -24 * ref + 1e-15)
    assert np.all(np.abs(w.astype(np.float64).sum(axis=1) - 1.0) <= 8 * 2.0 ** -24)
    assert np.all(np.diff(w, axis=1) <= 0)          # descending logits, descending weights


def test_softmax_shift_invariance_and_k1():
    rng = np.random.default_rng(8)
    L = rng.integers(-20, 20, size=(50, 16)).astype(np.float32)
    _, w0 = route(L, 4, "softmax")
    _, w1 = route(L + np.float32(64.0), 4, "softmax")
    assert np.array_equal(w0, w1)
    _, w = route(L, 1, "sigmoid")
    assert np.all(w == 1.0)


def test_router_rejects_bad_arguments():
    with pytest.raises(ValueError):
        route(np.zeros((2, 4), np.float32), 5, "softmax")
    with pytest.raises(ValueError):
        route(np.zeros((2, 4), np.float32), 2, "relu")
