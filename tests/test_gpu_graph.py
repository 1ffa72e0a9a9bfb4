"""The library's calls inside a captured HIP graph (torch.cuda.CUDAGraph).

No call allocates, synchronises or records a memset, so a whole step can be
captured once and replayed. Each test replays several times with new inputs
copied into the captured buffers between replays (eager work and a
synchronisation in between), and checks every replay against the same calls
run eagerly, bit for bit, and one replay against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from combine_moe_dispatch_02_amd import Handle
from workloads import make_expert_outputs
from gpu_util import assert_combine_close, dev_bf16, dev_f32, host_bits

pytestmark = pytest.mark.gpu


def decode_inputs(seed, T=128, H=7168, E=256):
    wl = workloads.make_workload("deepseekv3", seed=seed, tokens=T, hidden=H)
    return wl.logits, wl.x_bits


def test_decode_step_graph_replays():
    T, H, k, E, R, C = 128, 7168, 8, 256, 8, 128
    h = Handle(T, H, k, E, R)
    logits = torch.empty((T, E), dtype=torch.float32, device="cuda")
    x = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    rows = torch.zeros((E * C, H), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

    def step():
        h.route(logits, "sigmoid", topk_idx=idx, topk_w=w)
        h.ll_dispatch(idx, x, C, out=rows)
        h.ll_combine(rows, w, out=out)

    L0, x0 = decode_inputs(11)
    logits.copy_(torch.from_numpy(L0)); x.copy_(dev_bf16(x0))
    step()                                   # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for seed in (21, 22, 23):
        L, xb = decode_inputs(seed)
        logits.copy_(torch.from_numpy(L)); x.copy_(dev_bf16(xb))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [idx.clone(), w.clone(), out.clone()]
        step()                               # the same calls, eagerly
        torch.cuda.synchronize()
        for a, b in zip(got, [idx, w, out]):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), seed
        if seed == 21:
            ri, rw = oracle.route(L, k, "sigmoid")
            assert np.array_equal(got[0].cpu().numpy(), ri)
            # identity experts: combine of the dispatched rows with weights summing to ~1 gives x back
            assert np.array_equal(host_bits(got[2]), np.where(xb == 0x8000, np.uint16(0), xb))


@pytest.mark.parametrize("T", [512, 2048])
def test_standard_step_graph_replays(T):
    """512 tokens: the one-workgroup layout and the per-slot bf16 dispatch;
    2048 tokens (12 layout chunks): the two layout kernels with the block
    lists and the blocked bf16 dispatch."""
    H, k, E, R = 2048, 6, 64, 8
    h = Handle(T, H, k, E, R)
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    x = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T * k, H), dtype=torch.bfloat16, device="cuda")
    d_out = torch.empty((T * k, H), dtype=torch.bfloat16, device="cuda")
    q_out = torch.empty((T * k, H), dtype=torch.uint8, device="cuda")
    q_sc = torch.empty((T * k, H // 128), dtype=torch.float32, device="cuda")
    c_out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")

    def step():
        h.layout(idx)
        h.dispatch(x, out=d_out)
        h.dispatch(x, fp8=True, out=q_out, scales=q_sc)
        h.combine(y, w, out=c_out)

    def load(seed):
        wl = workloads.make_workload("deepseek16b", seed=seed, tokens=T)
        ri, rw = oracle.route(wl.logits, k, "softmax")
        idx.copy_(torch.from_numpy(ri)); w.copy_(torch.from_numpy(rw))
        x.copy_(dev_bf16(wl.x_bits))
        yb = make_expert_outputs(T * k, H, seed=seed + 1)
        y.copy_(dev_bf16(yb))
        return ri, rw, wl.x_bits, yb

    load(1)
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for seed in (5, 6, 7):
        ri, rw, xb, yb = load(seed)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (h.view()["pos"], d_out, q_out, q_sc, c_out)]
        step()
        torch.cuda.synchronize()
        for a, b in zip(got, (h.view()["pos"], d_out, q_out, q_sc, c_out)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), seed
        if seed == 5:
            lay = oracle.layout(ri, E, R)
            assert np.array_equal(got[0].cpu().numpy(), lay["pos"])
            assert np.array_equal(host_bits(got[1]), oracle.dispatch_bf16(xb, lay["pos"]))
            want, mag = oracle.combine(yb, rw, lay["pos"], return_magnitude=True)
            assert_combine_close(host_bits(got[4]), want, mag, k)
