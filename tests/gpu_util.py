"""Helpers shared by the GPU tests: host <-> device moves of bit patterns and
the oracle comparisons."""
import numpy as np
import torch

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
    exact = float(np.mean(got_bits == ref_bits)) if got_bits.size else 1.0   # empty batch: vacuous
    return float(rel.max()), exact


def router_weight_tol(logits, idx, w_ref):
    """Allowance for fp32 router weights against the oracle's (fp64, rounded once).

    Per weight, relative to w_ref, in units of 2^-24: the logit difference
    l_j - l_max rounds with error up to |l_j - l_max| units of relative error
    in exp (and the same for the largest one in the sum), expf is within one
    fp32 ulp (2 units), the fp32 butterfly sum of at most 32 positive terms
    adds at most 5 levels (5 units), the division and the oracle's rounding one
    unit each; the sigmoid's 1 + e and reciprocal add two. That is at most
    2 + 2 + 5 + 1 + 1 + 2 + 2*D = 13 + 2D units for D = max_j |l_j - l_max|; the
    bound allows 16 + 2D, plus 1e-30 absolute for terms that underflow.
    """
    sel = np.take_along_axis(np.asarray(logits, np.float64), idx.astype(np.int64), axis=1)
    D = np.max(np.abs(sel - sel[:, :1]), axis=1, keepdims=True)
    return 2.0 ** -24 * (16.0 + 2.0 * D) * np.abs(w_ref.astype(np.float64)) + 1e-30
