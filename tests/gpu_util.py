"""Helpers shared by the GPU tests: host <-> device moves of bit patterns and
the oracle comparisons."""
import numpy as np
import torch

import oracle
from conftest import combine_tolerance


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16).to("cuda")


def host_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")


def layout_on_gpu(h, idx: np.ndarray) -> dict:
    h.layout(dev_i32(idx))
    torch.cuda.synchronize()
    return {k: v.cpu().numpy().astype(np.int64) for k, v in h.view().items()}


def assert_layout_equal(got: dict, ref: dict, T: int, k: int):
    for key in ("counts_e", "offsets_e", "counts_r", "offsets_r"):
        assert np.array_equal(got[key], ref[key]), key
    assert np.array_equal(got["pos"].reshape(T, k), ref["pos"]), "pos"
    assert np.array_equal(got["src_idx"][:T * k], ref["src_idx"]), "src_idx"
    assert got["status"][0] == ref["invalid"]
    assert got["status"][1] == ref["offsets_e"][-1]
    assert got["status"][2] == T


def assert_combine_close(got_bits, ref_bits, mag, k, extra=None):
    """Element-wise gate of conftest.combine_tolerance (plus `extra`, an
    absolute allowance for paths that round more than once)."""
    got = (got_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = (ref_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    tol = combine_tolerance(ref_bits, mag, k)
    if extra is not None:
        tol = tol + extra
    bad = ~(np.abs(got - ref) <= tol)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{bad.sum()} elements outside tolerance; first {tuple(i)}: "
                             f"got {got[tuple(i)]!r} ref {ref[tuple(i)]!r} tol {tol[tuple(i)]!r}")
    big = np.abs(ref) >= 1e-2
    rel = np.abs(got - ref)[big] / np.abs(ref)[big] if big.any() else np.zeros(1)
    return float(rel.max()), float(np.mean(got_bits == ref_bits))


def oracle_layout(idx, E, R):
    return oracle.layout(idx, E, R)
