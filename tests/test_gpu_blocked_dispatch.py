"""bf16 dispatch in its blocked form against the oracle and the per-slot form.

From eight layout chunks of slots on (and while one chunk's tokens hold at
most 3.5 MiB of x), the layout also lists, for each dispatch block of whole
chunks, the block's rows in ascending row order, and the bf16 dispatch copies
x along those lists, one XCD slot per block. The rows must be bit-identical
to the oracle's ("Inside the Nebius + PyTorch DeepSeek V3 recipe", section
"Mixture-of-experts and wide expert parallelism": each token goes to the
experts its router picked) and to the per-slot form, which a workgroup cap
selects; rows past the placed total stay untouched. Cases: exactly eight
chunks and one more, blocks whose edges split a token's slots, a row whose
last slice holds one 16-byte vector, the narrowest row, every slot on one
expert, invalid ids, k = 1 and k = 32, XCD slots that walk two and eight
blocks, 128 layout workgroups (column sums split over threads) feeding blocks
of 16 chunks, the one-launch layout feeding blocks of 2 chunks, a batch
whose x is too large for the early burst and one too large for the blocked
form, a handle reused across sizes that take different forms, and the
one-call layout + dispatch.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_dispatch_02_amd import Handle
from gpu_util import assert_layout_equal, dev_bf16, dev_i32, host_bits, layout_on_gpu

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC1   # a bf16 NaN pattern no dispatched row holds


def ids(T, k, E, pattern, seed):
    rng = np.random.default_rng(seed)
    if pattern == "const":
        return np.full((T, k), E - 1, dtype=np.int32)
    out = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) if k <= E \
        else rng.integers(0, E, size=(T, k)).astype(np.int32)
    if pattern == "invalid":
        bad = rng.random((T, k)) < 0.15
        out[bad] = rng.choice(np.array([-1, E, 2 ** 31 - 1], dtype=np.int64),
                              size=int(bad.sum())).astype(np.int32)
    return out


def bf16_rows(T, H, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(0, 2 ** 16, size=(T, H), dtype=np.uint16) & np.uint16(0xBFFF)


def dispatch_into_sentinel(h, x, rows, H):
    out = torch.full((rows, H), SENTINEL, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    h.dispatch(x, out=out)
    return host_bits(out)


CASES = [
    # name, T, k, E, R, H, id pattern
    ("eight_chunks", 1024, 8, 256, 8, 7168, "random"),
    ("nine_chunks", 1025, 8, 256, 8, 7168, "random"),
    ("blocks_split_tokens", 3000, 6, 64, 8, 2048, "random"),
    ("ragged_last_slice", 1100, 8, 256, 8, 7176, "invalid"),
    ("narrowest_row", 2048, 8, 128, 8, 8, "random"),
    ("one_expert", 4096, 8, 256, 8, 1024, "const"),
    ("k32_invalid", 600, 32, 1024, 8, 1024, "invalid"),
    ("k1", 9000, 1, 64, 8, 512, "random"),
    # 32 chunks of 912 KiB of x: blocks of 2 chunks, two per XCD slot
    ("two_blocks_per_slot", 32768, 1, 64, 8, 456, "random"),
    # 64 chunks of 2 MiB: blocks of 1 chunk, eight per slot; last slice one vector
    ("eight_blocks_per_slot", 65536, 1, 64, 8, 1032, "random"),
    # 128 chunks of 16 KiB: blocks of 16 chunks, the layout's split column sums
    ("split_sums_lists", 16384, 8, 128, 8, 64, "invalid"),
    # 16 chunks, the last one partial: the one-launch layout, blocks of 2 chunks
    ("one_launch_layout_pairs", 2000, 8, 256, 8, 64, "invalid"),
    # x of 161 MB (above 144 MiB): blocked, without the early burst of x
    ("blocked_without_burst", 45000, 1, 64, 8, 1792, "random"),
    # x of 215 MB (above 192 MiB): the per-slot form, though 59 chunks
    ("x_above_blocked_limit", 60000, 1, 64, 8, 1792, "random"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_blocked_dispatch_matches_oracle_and_per_slot_form(case):
    name, T, k, E, R, H, pattern = case
    print(f"[blocked] {name} T={T} k={k} E={E} H={H} {pattern}", flush=True)
    idx = ids(T, k, E, pattern, seed=len(name))
    xb = bf16_rows(T, H, seed=T + H)
    h = Handle(T, H, k, E, R)
    got = layout_on_gpu(h, idx)
    ref = oracle.layout(idx, E, R)
    assert_layout_equal(got, ref, T, k)
    total = int(ref["offsets_e"][-1])
    x = dev_bf16(xb)
    rows = T * k + 5                      # more rows than the capacity: the tail stays untouched
    blocked = dispatch_into_sentinel(h, x, rows, H)
    want = oracle.dispatch_bf16(xb, ref["pos"])
    assert np.array_equal(blocked[:total], want[:total])
    assert np.all(blocked[total:] == SENTINEL)
    h.set_max_workgroups(1 << 20)         # a cap above the item count: the per-slot form, uncapped
    per_slot = dispatch_into_sentinel(h, x, rows, H)
    h.set_max_workgroups(0)
    assert np.array_equal(blocked, per_slot)


def test_handle_reused_across_forms():
    """One handle: a batch in the blocked form, then one below eight chunks
    (per-slot form, its layout writes no lists), then the blocked form again
    with fewer tokens than the first -- each dispatch follows its own layout."""
    T_max, H, k, E, R = 4096, 1024, 8, 256, 8
    h = Handle(T_max, H, k, E, R)
    for T, seed in ((4096, 1), (600, 2), (1500, 3), (4096, 4)):
        print(f"[blocked] reuse T={T}", flush=True)
        idx = ids(T, k, E, "random", seed)
        xb = bf16_rows(T, H, seed)
        h.layout(dev_i32(idx))
        ref = oracle.layout(idx, E, R)
        out = host_bits(h.dispatch(dev_bf16(xb)))
        assert np.array_equal(out, oracle.dispatch_bf16(xb, ref["pos"]))


def test_layout_dispatch_call_uses_lists():
    """moe_layout_dispatch from 640 tokens on runs the layout of
    moe_dispatch_layout (at 1024 tokens x top-8 one launch that also writes the
    lists) and then the dispatch, here in the blocked form."""
    T, H, k, E, R = 1024, 7168, 8, 256, 8
    idx = ids(T, k, E, "invalid", seed=9)
    xb = bf16_rows(T, H, seed=10)
    h = Handle(T, H, k, E, R)
    out = host_bits(h.layout_dispatch(dev_i32(idx), dev_bf16(xb)))
    ref = oracle.layout(idx, E, R)
    total = int(ref["offsets_e"][-1])
    assert np.array_equal(out[:total], oracle.dispatch_bf16(xb, ref["pos"])[:total])
