"""moe_dispatch_layout_noalloc, the layout for callers that cannot allocate
device memory (its per-workgroup histograms live in the library's static
device array), against moe_dispatch_layout on a handle with a workspace:
bit-exact on every output array, on calls in a row that shrink, through
the C ABI."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from combine_moe_dispatch_02_amd import Handle, MoeError, _lib, moe_dispatch_layout_noalloc
from gpu_util import assert_layout_equal, dev_i32
from routed import make_workload

pytestmark = pytest.mark.gpu

KEYS = ("pos", "src_idx", "counts_e", "offsets_e", "counts_r", "offsets_r", "status")


def _noalloc(idx: np.ndarray, E: int, R: int) -> dict:
    T, k = idx.shape
    sizes = {"pos": T * k, "src_idx": T * k, "counts_e": E, "offsets_e": E + 1, "counts_r": R,
             "offsets_r": R + 1, "status": 4}
    # outputs pre-filled with a value no layout writes, so unwritten entries show
    out = {key: torch.full((max(n, 1),), -7, dtype=torch.int32, device="cuda")
           for key, n in sizes.items()}
    moe_dispatch_layout_noalloc(dev_i32(idx), E, R, out["pos"], out["src_idx"], out["counts_e"],
                                out["offsets_e"], out["counts_r"], out["offsets_r"], out["status"])
    torch.cuda.synchronize()
    return {key: out[key].cpu().numpy()[:sizes[key]] for key in KEYS}


def _handle_layout(idx: np.ndarray, E: int, R: int) -> dict:
    T, k = idx.shape
    h = Handle(max(T, 1), 8, k, E, R)
    h.layout(dev_i32(idx))
    torch.cuda.synchronize()
    v = {key: t.cpu().numpy() for key, t in h.view().items()}
    v["pos"] = v["pos"].reshape(-1)
    return v


@pytest.mark.parametrize("order", ["shrinking", "growing"])
def test_noalloc_layout_matches_workspace_layout(order):
    """Calls in a row on one GPU, each compared with the workspace layout
    entry by entry: the DeepSeek-V3-like batch (32 histogram workgroups), a
    smaller one laid out in one launch (6 workgroups, each counting every
    slot; no histograms), and one small enough for a single workgroup."""
    wl = make_workload("deepseekv3")
    rng = np.random.default_rng(3)
    small = np.stack([rng.permutation(64)[:6] for _ in range(1000)]).astype(np.int32)
    tiny = np.stack([rng.permutation(16)[:2] for _ in range(100)]).astype(np.int32)
    cases = [(wl.topk_idx, 256, 8), (small, 64, 8), (tiny, 16, 4)]
    if order == "growing":
        cases = cases[::-1]
    for idx, E, R in cases:
        T, k = idx.shape
        print(f"[noalloc] T={T} k={k} E={E} R={R}", flush=True)
        got = _noalloc(idx, E, R)
        want = _handle_layout(idx, E, R)
        for key in KEYS:
            assert np.array_equal(got[key], want[key][:got[key].size]), key
        assert_layout_equal(got, oracle.layout(idx, E, R), T, k)


def test_noalloc_layout_empty_and_invalid_ids():
    idx = np.full((0, 4), 0, dtype=np.int32)
    got = _noalloc(idx, 32, 4)
    assert np.all(got["counts_e"] == 0) and np.all(got["offsets_e"] == 0)
    assert list(got["status"][:3]) == [0, 0, 0]
    rng = np.random.default_rng(4)
    idx = rng.integers(-3, 40, size=(2000, 4)).astype(np.int32)   # some ids outside [0, 32)
    got = _noalloc(idx, 32, 4)
    assert_layout_equal(got, oracle.layout(idx, 32, 4), 2000, 4)


def test_noalloc_layout_rejects_oversized_batches():
    """A batch whose histograms would not fit the static array is refused on
    the host with a message naming the way out; nothing is enqueued."""
    lib = _lib.load()
    buf = torch.zeros(4096, dtype=torch.int32, device="cuda")
    p = ctypes.c_void_p(buf.data_ptr())
    st = lib.moe_dispatch_layout_noalloc(p, 300000, 8, 256, 8, p, p, p, p, p, p, p, None)
    assert st == _lib.MOE_ERR_UNSUPPORTED
    assert b"moe_dispatch_layout with a workspace" in lib.moe_last_error()
    torch.cuda.synchronize()
    assert torch.all(buf == 0)
    with pytest.raises(MoeError):
        moe_dispatch_layout_noalloc(dev_i32(np.zeros((10, 2), np.int32)), 250, 8, *[buf] * 7)
