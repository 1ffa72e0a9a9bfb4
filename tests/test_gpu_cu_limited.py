"""Dispatch and combine on compute-unit-limited streams (moe_stream_create_cu_limited)
give the oracle's results; the stream carries the mask moe_cu_mask computes.

The Hybrid-EP news item ("Efficiency Numbers") runs the exchange on a few SMs
so that the rest of the GPU stays free for the experts; the library's
counterpart is a stream limited to n compute units, an equal share of each
of the 8 XCDs. Results must not depend on where the work runs.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from combine_moe_dispatch_02_amd import CuLimitedStream, Handle, _lib, moe_cu_mask
from gpu_util import (assert_combine_close, assert_layout_equal, dev_bf16, dev_f32, dev_i32,
                      host_bits)
from routed import make_workload
from workloads import make_expert_outputs

pytestmark = pytest.mark.gpu


def _stream_mask(raw, words):
    hip = _lib.load()
    fn = hip.hipExtStreamGetCUMask
    fn.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.POINTER(ctypes.c_uint32)]
    fn.restype = ctypes.c_int
    buf = (ctypes.c_uint32 * words)()
    assert fn(ctypes.c_void_p(raw), words, buf) == 0
    return list(buf)


@pytest.mark.parametrize("num_cus", [8, 64])
def test_cu_limited_stream_matches_oracle(num_cus):
    wl = make_workload("deepseek16b")
    s = wl.shape
    total = torch.cuda.get_device_properties(0).multi_processor_count
    print(f"[cu-limited] {num_cus} of {total} compute units, {s.name}", flush=True)
    h = Handle(s.tokens, s.hidden, s.topk, s.experts, s.ranks)
    y_bits = make_expert_outputs(s.tokens * s.topk, s.hidden, seed=wl.seed + 1)
    idx, x, y, w = dev_i32(wl.topk_idx), dev_bf16(wl.x_bits), dev_bf16(y_bits), dev_f32(wl.topk_w)
    # Outputs are allocated on the default stream, before the limited one exists.
    S, H = s.tokens * s.topk, s.hidden
    rows = torch.empty((S, H), dtype=torch.bfloat16, device="cuda")
    codes = torch.empty((S, H), dtype=torch.uint8, device="cuda")
    scales = torch.empty((S, H // 128), dtype=torch.float32, device="cuda")
    comb = torch.empty((s.tokens, H), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    with CuLimitedStream(num_cus) as st:
        want_mask = moe_cu_mask(total, num_cus)
        assert _stream_mask(st.cuda_stream, len(want_mask)) == want_mask
        h.layout(idx)
        h.dispatch(x, out=rows)
        h.dispatch(x, fp8=True, out=codes, scales=scales)
        h.combine(y, w, out=comb)
        st.synchronize()
    view = {k: v.cpu().numpy() for k, v in h.view().items()}
    ref = oracle.layout(wl.topk_idx, s.experts, s.ranks)
    assert_layout_equal(view, ref, s.tokens, s.topk)
    assert np.array_equal(host_bits(rows), oracle.dispatch_bf16(wl.x_bits, ref["pos"]))
    rc, rs = oracle.dispatch_fp8(wl.x_bits, ref["pos"])
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    want, mag = oracle.combine(y_bits, wl.topk_w, ref["pos"], return_magnitude=True)
    rel, _ = assert_combine_close(host_bits(comb), want, mag, s.topk)
    assert rel <= 1e-2


def test_cu_limited_stream_rejects_bad_counts():
    from combine_moe_dispatch_02_amd import MoeError
    with pytest.raises(MoeError, match="multiple of 8"):
        CuLimitedStream(12)
    with pytest.raises(MoeError, match="multiple of 8"):
        CuLimitedStream(100000)
