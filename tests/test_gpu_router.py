"""GPU parity of the router kernel (moe_route) against the oracle's router.

Bar: top-k ids bit-exact (the selection compares fp32 logits, no arithmetic);
weights within gpu_util.router_weight_tol (fp32 expf and sums against the
oracle's fp64 weights rounded once). Covers the five workloads, ties and
signed zeros, every expert-count branch of the kernel (<= 64 ... <= 1024),
k = 1 and k = E, extreme logits, and the router feeding the layout.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_dispatch_02_amd import Handle
from workloads import CONFIGS
import workloads
from gpu_util import dev_f32, dev_i32, layout_on_gpu, assert_layout_equal, router_weight_tol

pytestmark = pytest.mark.gpu


def check_route(h, L, k, score):
    idx, w = h.route(dev_f32(L), score)
    torch.cuda.synchronize()
    gi, gw = idx.cpu().numpy(), w.cpu().numpy()
    ri, rw = oracle.route(L, k, score)
    bad = np.argwhere(gi != ri)
    assert bad.size == 0, f"{len(bad)} id mismatches, first {bad[:3].tolist()}"
    tol = router_weight_tol(L, ri, rw)
    err = np.abs(gw.astype(np.float64) - rw)
    assert np.all(err <= tol), f"weight error {float((err / np.maximum(tol, 1e-300)).max()):.3f} x tol"
    ok = rw > 0
    units = float((err[ok] / rw[ok]).max() / 2.0 ** -24) if ok.any() else 0.0
    return gi, gw, units


@pytest.mark.parametrize("shape", CONFIGS, ids=lambda s: s.name)
def test_route_matches_oracle(shape):
    wl = workloads.make_workload(shape.name, hidden=8)
    h = Handle(shape.tokens, 8, shape.topk, shape.experts, shape.ranks)
    _, _, units = check_route(h, wl.logits, shape.topk, shape.weights)
    print(f"[route] {shape.name}: max weight error {units:.1f} x 2^-24 relative", flush=True)


@pytest.mark.parametrize("E,k", [(8, 2), (40, 40 // 2), (64, 8), (100, 6), (128, 8), (256, 8),
                                 (300, 32), (512, 4), (1000, 10), (1024, 32), (32, 32), (16, 1)])
@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_route_expert_counts_and_ties(E, k, score):
    rng = np.random.default_rng(E * 100 + k)
    T = 777
    L = rng.standard_normal((T, E)).astype(np.float32) * 2
    L[::3] = (rng.integers(-4, 4, size=(L[::3].shape)) / 4.0).astype(np.float32)  # many ties
    L[1::5, : E // 2] = np.float32(-0.0)
    L[2::5, : E // 2] = np.float32(0.0)
    R = 4 if E % 4 == 0 else 1
    h = Handle(T, 8, k, E, R)
    check_route(h, L, k, score)


def test_route_extreme_logits():
    T, E, k = 64, 64, 4
    rng = np.random.default_rng(2)
    L = rng.standard_normal((T, E)).astype(np.float32)
    L[0, :4] = [1000.0, 999.0, 998.5, -1000.0]
    L[1] = -1000.0 + rng.random(E).astype(np.float32)
    L[2] = 30.0 * rng.standard_normal(E).astype(np.float32)
    L[3] = np.float32(3.4e38) * np.sign(rng.standard_normal(E)).astype(np.float32)
    h = Handle(T, 8, k, E, 2)
    check_route(h, L, k, "softmax")
    L[3] = 0.0
    L[1] = -40.0 + rng.random(E).astype(np.float32)        # sigmoid scores ~ e^-40, no underflow
    check_route(h, L, k, "sigmoid")


def test_route_empty_and_single_token():
    h = Handle(16, 8, 2, 8, 2)
    idx, w = h.route(torch.empty((0, 8), dtype=torch.float32, device="cuda"))
    assert idx.shape == (0, 2)
    L = np.array([[0.5, -1.0, 2.0, 2.0, 0.0, -0.0, 1.0, 3.0]], np.float32)
    gi, gw, _ = check_route(h, L, 2, "softmax")
    assert gi.tolist() == [[7, 2]]


@pytest.mark.parametrize("name", ["deepseekv3", "qwen3_skewed"])
def test_router_feeds_layout(name):
    """Router and layout on the GPU give the oracle's layout of the oracle's routing."""
    wl = workloads.make_workload(name, hidden=8)
    s = wl.shape
    h = Handle(s.tokens, 8, s.topk, s.experts, s.ranks)
    idx, _ = h.route(dev_f32(wl.logits), s.weights)
    got = layout_on_gpu(h, idx.cpu().numpy())
    ri, _ = oracle.route(wl.logits, s.topk, s.weights)
    assert_layout_equal(got, oracle.layout(ri, s.experts, s.ranks), s.tokens, s.topk)
    h.layout(idx)                                        # straight from the router's output
    torch.cuda.synchronize()
    assert np.array_equal(h.view()["pos"].cpu().numpy(), got["pos"])
