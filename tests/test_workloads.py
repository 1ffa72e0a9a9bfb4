"""Checks of the seeded input generators (shapes, determinism, router output)."""
import numpy as np
import pytest

from workloads import CONFIGS, make_expert_outputs, make_workload


@pytest.mark.parametrize("shape", CONFIGS, ids=lambda s: s.name)
def test_workload_shapes_and_router(shape):
    wl = make_workload(shape.name)
    T, H, E, k = shape.tokens, shape.hidden, shape.experts, shape.topk
    assert wl.x_bits.shape == (T, H) and wl.x_bits.dtype == np.uint16
    assert wl.topk_idx.shape == (T, k) and wl.topk_idx.dtype == np.int32
    assert wl.topk_w.shape == (T, k) and wl.topk_w.dtype == np.float32
    assert wl.topk_idx.min() >= 0 and wl.topk_idx.max() < E
    # top-k picks k distinct experts per token
    s = np.sort(wl.topk_idx, axis=1)
    assert np.all(np.diff(s, axis=1) > 0)
    # normalised weights, descending with the router order
    assert np.allclose(wl.topk_w.sum(axis=1), 1.0, atol=1e-6)
    assert np.all(np.diff(wl.topk_w, axis=1) <= 0)
    assert wl.seed == 1000 + CONFIGS.index(shape)


def test_workload_deterministic():
    a = make_workload("deepseek16b", tokens=64)
    b = make_workload("deepseek16b", tokens=64)
    assert np.array_equal(a.x_bits, b.x_bits) and np.array_equal(a.topk_idx, b.topk_idx)
    c = make_workload("deepseek16b", tokens=64, seed=1)
    assert not np.array_equal(a.topk_idx, c.topk_idx)
    assert np.array_equal(make_expert_outputs(8, 16, 3), make_expert_outputs(8, 16, 3))


def test_qwen_workload_is_skewed():
    wl = make_workload("qwen3_skewed")
    counts = np.bincount(wl.topk_idx.reshape(-1), minlength=128)
    # Zipf(1.2) popularity in expert-id order: expert 0 is in almost every token's top-8
    assert counts[0] > 0.9 * wl.T
    per_rank = counts.reshape(8, 16).sum(axis=1)
    assert per_rank[0] > 0.5 * counts.sum()
    assert np.all(np.diff(counts[:8]) < 0)


def test_normal_workload_is_balanced():
    wl = make_workload("deepseekv3")
    counts = np.bincount(wl.topk_idx.reshape(-1), minlength=256)
    assert counts.sum() == 4096 * 8
    assert counts.min() > 60 and counts.max() < 220
