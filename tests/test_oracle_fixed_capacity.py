"""Pins for the oracle's fixed-capacity (decode-time) layout."""
import numpy as np
import pytest

from oracle.moe import dispatch_bf16, layout, layout_fixed_capacity
from conftest import load_golden


@pytest.mark.parametrize("case", load_golden("layout_hand.json")["cases"], ids=lambda c: c["name"])
def test_fixed_capacity_hand_worked(case):
    fc = case["fixed_capacity"]
    got = layout_fixed_capacity(np.array(case["topk_idx"]), case["num_experts"], fc["capacity"])
    assert got["pos"].tolist() == fc["pos"]
    assert got["counts"].tolist() == fc["counts"]
    assert got["dropped"] == fc["dropped"] and got["invalid"] == fc["invalid"]


def random_ids(rng, T, k, E, bad=0.1):
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    m = rng.random((T, k)) < bad
    idx[m] = rng.choice(np.array([-1, E, 99999]), size=int(m.sum()))
    return idx


@pytest.mark.parametrize("C", [1, 3, 17, 10000])
def test_composes_with_the_standard_layout(C):
    """A slot's rank within its expert is its standard row minus the expert's offset."""
    rng = np.random.default_rng(C)
    T, k, E = 300, 4, 16
    idx = random_ids(rng, T, k, E)
    std = layout(idx, E, 4)
    fc = layout_fixed_capacity(idx, E, C)
    e = np.where((idx >= 0) & (idx < E), idx, 0)
    rank = std["pos"] - std["offsets_e"][e]
    want = np.where((std["pos"] >= 0) & (rank < C), e * C + rank, -1)
    assert np.array_equal(fc["pos"], want)
    assert np.array_equal(fc["counts"], np.minimum(std["counts_e"], C))
    assert fc["dropped"] == int(np.maximum(std["counts_e"] - C, 0).sum())
    assert fc["invalid"] == std["invalid"]


def test_brute_force_tiny():
    rng = np.random.default_rng(5)
    T, k, E, C = 12, 3, 4, 4
    idx = random_ids(rng, T, k, E, bad=0.2)
    fc = layout_fixed_capacity(idx, E, C)
    flat = idx.reshape(-1)
    for s, e in enumerate(flat):
        if not 0 <= e < E:
            assert fc["pos"].reshape(-1)[s] == -1
            continue
        r = int(np.sum(flat[:s] == e))
        assert fc["pos"].reshape(-1)[s] == (e * C + r if r < C else -1)


def test_dispatch_into_fixed_regions():
    rng = np.random.default_rng(6)
    T, k, E, C, H = 40, 2, 8, 6, 16
    idx = random_ids(rng, T, k, E)
    x = rng.integers(0, 2 ** 16, size=(T, H), dtype=np.uint16)
    fc = layout_fixed_capacity(idx, E, C)
    out = dispatch_bf16(x, fc["pos"], rows=E * C)
    assert out.shape == (E * C, H)
    for e in range(E):
        n = int(fc["counts"][e])
        toks = [t for t in range(T) for j in range(k) if idx[t, j] == e][:n]
        assert np.array_equal(out[e * C:e * C + n], x[toks])
        assert not out[e * C + n:(e + 1) * C].any()
