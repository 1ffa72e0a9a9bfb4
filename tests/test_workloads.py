"""Checks of the seeded input generators (shapes, determinism, logit
distributions) and of the routed workloads the tests build from them."""
import numpy as np
import pytest

import workloads
from workloads import CONFIGS, make_expert_outputs
from routed import make_workload


@pytest.mark.parametrize("shape", CONFIGS, ids=lambda s: s.name)
def test_workload_shapes(shape):
    raw = workloads.make_workload(shape.name)
    T, H, E, k = shape.tokens, shape.hidden, shape.experts, shape.topk
    assert raw.x_bits.shape == (T, H) and raw.x_bits.dtype == np.uint16
    assert raw.logits.shape == (T, E) and raw.logits.dtype == np.float32
    assert raw.topk_idx is None and raw.topk_w is None      # the generator does not route
    assert raw.seed == 1000 + CONFIGS.index(shape)
    wl = make_workload(shape.name)
    assert wl.topk_idx.shape == (T, k) and wl.topk_idx.dtype == np.int32
    assert wl.topk_w.shape == (T, k) and wl.topk_w.dtype == np.float32
    assert np.array_equal(wl.x_bits, raw.x_bits) and np.array_equal(wl.logits, raw.logits)


def test_hidden_does_not_change_the_logits():
    a = workloads.make_workload("deepseekv3", tokens=32)
    b = workloads.make_workload("deepseekv3", tokens=32, hidden=128)
    assert np.array_equal(a.logits, b.logits)


def test_workload_deterministic():
    a = workloads.make_workload("deepseek16b", tokens=64)
    b = workloads.make_workload("deepseek16b", tokens=64)
    assert np.array_equal(a.x_bits, b.x_bits) and np.array_equal(a.logits, b.logits)
    c = workloads.make_workload("deepseek16b", tokens=64, seed=1)
    assert not np.array_equal(a.logits, c.logits)
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
