"""Seeded random configurations through every entry point, against the oracle.

Each case draws T, H, k, E, R, an id pattern (uniform, skewed, duplicates,
invalid ids) and a fixed-capacity C, then checks the layout, bf16 / FP8 /
MXFP8 dispatch, combine, the rank-deduplicated exchange and the decode-time
path to the same bars as the dedicated tests (bit-exact, combine within the
combine tolerance), and reruns the dispatches and combine under a workgroup
cap, which must give the same bits. The draws are fixed by the case seed.
"""
import numpy as np
import pytest

import oracle
from combine_moe_dispatch_02_amd import Handle
from workloads import bf16_bits_from_f32, make_expert_outputs
from gpu_util import (assert_combine_close, assert_layout_equal, dev_bf16, dev_f32, dev_i32,
                      host_bits, layout_on_gpu)

pytestmark = pytest.mark.gpu


def draw_case(seed):
    rng = np.random.default_rng(10_000 + seed)
    R = int(rng.choice([1, 2, 4, 8]))
    E = R * int(rng.choice([1, 2, 3, 8, 16, 32]))
    k = int(rng.integers(1, min(E, 32) + 1))
    T = int(rng.choice([1, 2, 63, 64, 65, 257, 1000, 2049, 3001]))
    H = 128 * int(rng.integers(1, 40))
    pattern = str(rng.choice(["uniform", "skewed", "duplicates", "invalid"]))
    if pattern == "uniform":
        idx = rng.integers(0, E, size=(T, k))
    elif pattern == "skewed":
        p = np.arange(1, E + 1, dtype=np.float64) ** -1.5
        idx = rng.choice(E, size=(T, k), p=p / p.sum())
    elif pattern == "duplicates":
        idx = rng.integers(0, max(1, E // 4), size=(T, k))
    else:
        idx = rng.integers(0, E, size=(T, k))
        bad = rng.random((T, k)) < 0.25
        idx[bad] = rng.choice(np.array([-1, E, 1 << 20, -(1 << 30)]), size=int(bad.sum()))
    x = bf16_bits_from_f32((rng.standard_normal((T, H)) *
                            np.exp2(rng.integers(-8, 8, size=(T, 1)))).astype(np.float32))
    w = rng.uniform(-1, 1, size=(T, k)).astype(np.float32)
    C = int(rng.integers(1, max(2, (T * k) // E + 3)))
    # drawn last, so the draws above are those of the uncapped sweep
    cap = int(rng.choice([1, 3, 17, 100, 511, 512, 700]))
    return dict(T=T, H=H, k=k, E=E, R=R, pattern=pattern, idx=idx.astype(np.int32), x=x, w=w, C=C,
                cap=cap)


@pytest.mark.parametrize("seed", range(30))
def test_random_config(seed):
    c = draw_case(seed)
    T, H, k, E, R, C = c["T"], c["H"], c["k"], c["E"], c["R"], c["C"]
    idx, x, w = c["idx"], c["x"], c["w"]
    print(f"[random {seed}] T={T} H={H} k={k} E={E} R={R} C={C} cap={c['cap']} {c['pattern']}",
          flush=True)
    h = Handle(T, H, k, E, R)
    # standard layout and dispatches
    got = layout_on_gpu(h, idx)
    ref = oracle.layout(idx, E, R)
    assert_layout_equal(got, ref, T, k)
    n = int(ref["offsets_e"][-1])
    dx = dev_bf16(x)
    d16 = host_bits(h.dispatch(dx))
    assert np.array_equal(d16[:n], oracle.dispatch_bf16(x, ref["pos"])[:n])
    q, s = h.dispatch(dx, fp8=True)
    rq, rs = oracle.dispatch_fp8(x, ref["pos"])
    q8, s8 = host_bits(q), host_bits(s)
    assert np.array_equal(q8[:n], rq[:n])
    assert np.array_equal(s8[:n].view(np.uint32), rs[:n].view(np.uint32))
    q, s = h.dispatch(dx, mxfp8=True)
    rq, rs = oracle.dispatch_mxfp8(x, ref["pos"])
    assert np.array_equal(host_bits(q)[:n], rq[:n])
    assert np.array_equal(host_bits(s)[:n], rs[:n])
    # combine of independent expert outputs
    y = make_expert_outputs(T * k, H, seed=seed)
    dy, dw = dev_bf16(y), dev_f32(w)
    comb = host_bits(h.combine(dy, dw))
    want, mag = oracle.combine(y, w, ref["pos"], return_magnitude=True)
    assert_combine_close(comb, want, mag, k)
    # the same calls under a workgroup cap: only the looping changes
    h.set_max_workgroups(c["cap"])
    capped = [host_bits(h.dispatch(dx)), *map(host_bits, h.dispatch(dx, fp8=True)),
              host_bits(h.combine(dy, dw))]
    h.set_max_workgroups(0)
    assert np.array_equal(capped[0][:n], d16[:n])
    assert np.array_equal(capped[1][:n], q8[:n]) and np.array_equal(capped[2][:n], s8[:n])
    assert np.array_equal(capped[3], comb)
    # rank-deduplicated exchange
    h.rank_layout(dev_i32(idx))
    rl = oracle.rank_layout(idx, E, R)
    rows, ridx, rw = h.dispatch_ranks(dx, dev_i32(idx), dev_f32(w))
    want_rows, want_idx, want_w = oracle.dispatch_ranks(x, idx, w, E, R, rl)
    m = int(rl["offsets_r"][-1])
    assert np.array_equal(host_bits(rows)[:m], want_rows[:m])
    assert np.array_equal(ridx.cpu().numpy()[:m], want_idx[:m])
    assert np.array_equal(rw.cpu().numpy()[:m].view(np.uint32), want_w[:m].view(np.uint32))
    part = make_expert_outputs(max(T * min(k, R), 1), H, seed=seed + 1)
    got_r = host_bits(h.combine_ranks(dev_bf16(part)))
    want_r, mag_r = oracle.combine_ranks(part, rl["rank_pos"], return_magnitude=True)
    assert_combine_close(got_r, want_r, mag_r, R)
    # layout and dispatch in one launch, and the decode-time path (token limit 1024)
    if T <= 1024:
        h2 = Handle(T, H, k, E, R)
        fused = h2.layout_dispatch(dev_i32(idx), dx)
        v2 = {key: t.cpu().numpy().astype(np.int64) for key, t in h2.view().items()}
        assert_layout_equal(v2, ref, T, k)
        assert np.array_equal(host_bits(fused)[:n], oracle.dispatch_bf16(x, ref["pos"])[:n])
        out = h.ll_dispatch(dev_i32(idx), dx, C)
        v = h.ll_view()
        fc = oracle.layout_fixed_capacity(idx, E, C)
        assert np.array_equal(v["pos"].cpu().numpy().astype(np.int64), fc["pos"])
        assert np.array_equal(v["counts"].cpu().numpy(), fc["counts"])
        mapped = fc["pos"][fc["pos"] >= 0]
        want_ll = oracle.dispatch_bf16(x, fc["pos"], rows=E * C)
        assert np.array_equal(host_bits(out)[mapped], want_ll[mapped])
        yl = make_expert_outputs(E * C, H, seed=seed + 2)
        got_l = host_bits(h.ll_combine(dev_bf16(yl), dev_f32(w)))
        want_l, mag_l = oracle.combine(yl, w, fc["pos"], return_magnitude=True)
        assert_combine_close(got_l, want_l, mag_l, k)
