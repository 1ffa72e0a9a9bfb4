"""Benchmark: MoE dispatch & combine on one MI355X, HBM GB/s and % of peak.

One step is one pass of the whole path over one batch resident in HBM:
layout (histogram + scan + placement), bf16 dispatch, FP8 dispatch, and
combine of the bf16-dispatched rows (identity experts), on the
DeepSeek-V3-like shape T=4096, H=7168, E=256 in 8 virtual ranks, top-8.

Every op reads its inputs from HBM: the inputs rotate over enough copies
(at least COLD_FOOTPRINT bytes of each, 8x the 256 MB last-level cache) that
none is still cached when it is read again, and the FP8 dispatch reads its
own copies of x, so it does not find the rows the bf16 dispatch just read.
Outputs rotate over at least three sets.

GB/s counts algorithmic bytes (each input read once, each output written
once, index arrays included):
  layout         12*S                      (S = T*k slots: ids in, pos and src_idx out)
  dispatch bf16  2*T*H + 2*S*H + 4*S
  dispatch FP8   2*T*H + S*H + 4*S*(H/128) + 4*S
  combine        2*S*H + 8*S + 2*T*H
Prints one JSON line (rank 0).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, 8 TB/s
LLC_BYTES = 256 << 20    # MI355X last-level (Infinity) cache
COLD_FOOTPRINT = 2 << 30 # bytes each rotating input spans: 8x the last-level cache
METRIC = "dispatch & combine HBM GB/s + % of peak, H=7168 T=4096 E=256 top-8"
WORKLOAD = "deepseekv3"


def op_bytes(T, H, k):
    S = T * k
    return {
        "layout": 12 * S,
        "dispatch_bf16": 2 * T * H + 2 * S * H + 4 * S,
        "dispatch_fp8": 2 * T * H + S * H + 4 * S * (H // 128) + 4 * S,
        "combine": 2 * S * H + 8 * S + 2 * T * H,
    }


def mxfp8_bytes(T, H, k):
    """MXFP8 dispatch (not part of the step): x once, codes + E8M0 bytes per row, pos."""
    S = T * k
    return 2 * T * H + S * H + S * (H // 32) + 4 * S


class HipTimer:
    """A HIP timing event created with hipEventDisableSystemFence.

    A default event (torch.cuda.Event) records with a system-scope release
    and acquire: the GPU writes back and invalidates its caches at every
    record, which costs microseconds and slows the kernel that follows, so
    the op between two such events looks slower than it runs. These events
    only take timestamps on the launch stream. The functions come from the
    HIP runtime the kernels library (and torch) already use, looked up
    through the library's own handle.
    """

    DISABLE_SYSTEM_FENCE = 0x20000000   # hipEventDisableSystemFence
    _hip = None

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            import ctypes
            from combine_moe_dispatch_02_amd import _lib
            hip = _lib.load()
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        import ctypes
        self._ev = ctypes.c_void_p()
        err = self._runtime().hipEventCreateWithFlags(ctypes.byref(self._ev),
                                                     self.DISABLE_SYSTEM_FENCE)
        if err != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {err}")

    def record(self, stream):
        err = self._runtime().hipEventRecord(self._ev, stream.cuda_stream)
        if err != 0:
            raise RuntimeError(f"hipEventRecord failed: {err}")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end` (both recorded and complete)."""
        import ctypes
        ms = ctypes.c_float()
        err = self._runtime().hipEventElapsedTime(ctypes.byref(ms), self._ev, end._ev)
        if err != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {err}")
        return ms.value

    def __del__(self):
        if self._hip is not None and getattr(self, "_ev", None):
            self._hip.hipEventDestroy(self._ev)


_QUEUE_AHEAD_BUF = None


def queue_ahead():
    """Keep the GPU busy (a bounded spin of about 2 ms: torch's own sleep
    kernel) while the host enqueues a timing loop, so that every event
    records back to back on the GPU and no call's time includes host launch
    latency. Without it a small op (a few us) is timed at the host's launch
    rate."""
    import torch
    sleep = getattr(torch.cuda, "_sleep", None)
    if sleep is not None:
        sleep(4_000_000)
        return
    # Without torch's sleep kernel: about 2 ms of plain device writes instead
    # (their dirty lines are written back during the first timed calls, which
    # then read a little slower).
    global _QUEUE_AHEAD_BUF
    if _QUEUE_AHEAD_BUF is None:
        _QUEUE_AHEAD_BUF = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    for i in range(8):
        _QUEUE_AHEAD_BUF.fill_(i)


KERNEL_OF_OP = {"dispatch_bf16": "dispatch_bf16_blocks_kernel",
                "dispatch_fp8": "dispatch_fp8_kernel", "combine": "combine_kernel<true, 8>"}
TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "traffic_deepseekv3.json")


def sources_sha256(paths) -> str:
    """SHA-256 over the named files' bytes, in order (paths from the repository root)."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(root, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(op: str):
    """HBM bytes per launch of op's kernel from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when any source the
    kernel is compiled from has changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)["kernels"][KERNEL_OF_OP[op]]
        if sources_sha256(rec["sources"]) != rec["sources_sha256"]:
            return None
        return int(rec["traffic_bytes"])
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(wl, sample_tokens: int, reps: int = 3):
    """Time the oracle, as committed, on a sample of the same workload.

    The calling thread is pinned to one host CPU and any BLAS/OpenMP pool is
    limited to one thread for the whole measurement, so "cores" is enforced,
    not assumed. Each op runs `reps` times; the per-op median is reported and
    the rate is the sample's algorithmic bytes over the sum of the medians.
    """
    import oracle
    s = wl.shape
    T, H, k = sample_tokens, s.hidden, s.topk
    x = wl.x_bits[:T]
    idx, w = oracle.route(wl.logits[:T], k, s.weights)   # the routing is not timed
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:   # pragma: no cover - the pin below still holds the thread to one CPU
        threadpool_limits = None
    allowed = os.sched_getaffinity(0)
    core = min(allowed)
    secs = {"layout": [], "dispatch_bf16": [], "dispatch_fp8": [], "combine": []}
    os.sched_setaffinity(0, {core})
    try:
        limits = threadpool_limits(limits=1) if threadpool_limits is not None else None
        try:
            cores = len(os.sched_getaffinity(0))
            for _ in range(reps):
                t0 = time.perf_counter()
                lay = oracle.layout(idx, s.experts, s.ranks)
                t1 = time.perf_counter()
                y = oracle.dispatch_bf16(x, lay["pos"])
                t2 = time.perf_counter()
                oracle.dispatch_fp8(x, lay["pos"])
                t3 = time.perf_counter()
                oracle.combine(y, w, lay["pos"])
                t4 = time.perf_counter()
                for key, dt in zip(secs, (t1 - t0, t2 - t1, t3 - t2, t4 - t3)):
                    secs[key].append(dt)
        finally:
            if limits is not None:
                limits.restore_original_limits()
    finally:
        os.sched_setaffinity(0, allowed)
    med = {key: float(np.median(v)) for key, v in secs.items()}
    nbytes = op_bytes(T, H, k)
    total = sum(nbytes.values())
    elapsed = sum(med.values())
    return {
        "value": round(total / elapsed / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
        "sample": f"{T} of {s.tokens} tokens of the {s.name} workload: layout, bf16 dispatch, FP8 "
                  f"dispatch and combine (numpy), each run {reps} times on one pinned host CPU "
                  f"(1 of {len(allowed)} available), per-op median; {elapsed:.2f} s for {total} "
                  "algorithmic bytes",
        "seconds_median": {key: round(v, 4) for key, v in med.items()},
        "GBps_per_op": {key: round(nbytes[key] / med[key] / 1e9, 4) for key in med},
        "host_cpus": os.cpu_count(),
    }


def copies_for(nbytes: int, minimum: int = 3) -> int:
    """How many copies of an nbytes buffer span COLD_FOOTPRINT (at least `minimum`)."""
    return max(minimum, -(-COLD_FOOTPRINT // max(1, nbytes)))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sustained-iters", type=int, default=30,
                    help="per-op timings, each op back to back over the rotating buffers")
    ap.add_argument("--cpu-sample-tokens", type=int, default=4096)
    ap.add_argument("--workgroup-sweep", type=int, default=1,
                    help="1: also report GB/s against a cap on the payload kernels' workgroups")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--instrument-every", type=int, default=5,
                    help="record per-op HIP events in every N-th timed step (1: every step)")
    ap.add_argument("--skip", default="",
                    help="comma list of report sections to leave out: rank, decode (router and "
                         "decode-time path), sweep, others (the other full-size workloads), "
                         "context (warm-x, evicted-x, in-order and copy/fill figures), cus "
                         "(compute-unit-limited streams, with a concurrent GEMM)")
    args = ap.parse_args()

    skip = {x for x in args.skip.split(",") if x}
    if not skip <= {"rank", "decode", "sweep", "others", "context", "cus"}:
        ap.error(f"--skip takes rank, decode, sweep, others, context, cus; got {args.skip}")
    if args.steps < 1:
        ap.error("--steps must be at least 1")
    if "sweep" in skip:
        args.workgroup_sweep = 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the expert-parallel work; --gpus {args.gpus} "
              "is not supported (the inter-GPU exchange is not part of this library)", file=sys.stderr)
        sys.exit(2)

    import torch
    from combine_moe_dispatch_02_amd import Handle
    from workloads import make_workload

    wl = make_workload(WORKLOAD)
    s = wl.shape
    T, H, k, E, R = s.tokens, s.hidden, s.topk, s.experts, s.ranks
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    h = Handle(T, H, k, E, R, device=dev)
    # Router outputs from the library's router kernel (untimed set-up).
    logits = torch.from_numpy(wl.logits).to(dev)
    topk_idx, topk_w = h.route(logits, s.weights)
    torch.cuda.synchronize()

    S = T * k
    x_dev = torch.from_numpy(wl.x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    x_bytes = 2 * T * H
    # Inputs rotate over copies spanning COLD_FOOTPRINT each; the FP8 dispatch
    # has copies of its own. Outputs rotate over three sets (combine's input,
    # the bf16 dispatch's output, over as many as span COLD_FOOTPRINT).
    n_x = copies_for(x_bytes)
    n_d = copies_for(2 * S * H)
    bufs = {
        "xb": [x_dev.clone() for _ in range(n_x)],
        "xq": [x_dev.clone() for _ in range(n_x)],
        "idx": [topk_idx.clone() for _ in range(3)],
        "w": [topk_w.clone() for _ in range(3)],
        "d_out": [torch.empty((S, H), dtype=torch.bfloat16, device=dev) for _ in range(n_d)],
        "q_out": [torch.empty((S, H), dtype=torch.uint8, device=dev) for _ in range(3)],
        "q_scales": [torch.empty((S, H // 128), dtype=torch.float32, device=dev) for _ in range(3)],
        "c_out": [torch.empty((T, H), dtype=torch.bfloat16, device=dev) for _ in range(3)],
    }

    def B(key, i):
        lst = bufs[key]
        return lst[i % len(lst)]

    ops = ("layout", "dispatch_bf16", "dispatch_fp8", "combine")

    def run_op(name, i):
        if name == "layout":
            h.layout(B("idx", i))
        elif name == "dispatch_bf16":
            h.dispatch(B("xb", i), out=B("d_out", i))
        elif name == "dispatch_fp8":
            h.dispatch(B("xq", i), fp8=True, out=B("q_out", i), scales=B("q_scales", i))
        else:
            h.combine(B("d_out", i), B("w", i), out=B("c_out", i))

    stream = torch.cuda.current_stream(dev)
    # Every expert-row set holds dispatched rows before anything reads it.
    h.layout(bufs["idx"][0])
    for i in range(n_d):
        h.dispatch(B("xb", i), out=B("d_out", i))
    for i in range(args.warmup):
        for name in ops:
            run_op(name, i)
    torch.cuda.synchronize()

    # Timed region: exactly K steps. Every `instrument_every`-th step (steps
    # every-1, 2*every-1, ...; the last step if K < every) records HIP events
    # (HipTimer: timestamps without cache maintenance) on the launch stream at
    # every op boundary (op i spans events i and i+1 of that step); the per-op
    # times and the roofline come from those steps. Step 0 is never among
    # them: it starts on an idle GPU, where an event would also time the
    # host's launch latency. The other steps run without events, so the wall
    # time per step carries as little timing overhead as possible.
    every = max(1, args.instrument_every)
    instrumented = [i for i in range(args.steps) if i % every == every - 1] or [args.steps - 1]
    ev = {i: [HipTimer() for _ in range(len(ops) + 1)] for i in instrumented}
    base = args.warmup
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        marks = ev.get(i)
        if marks is None:
            for name in ops:
                run_op(name, base + i)
            continue
        marks[0].record(stream)
        for j, name in enumerate(ops):
            run_op(name, base + i)
            marks[j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    nbytes = op_bytes(T, H, k)
    step_bytes = sum(nbytes.values())
    per_op = {}
    for j, name in enumerate(ops):
        us = np.array([ev[i][j].elapsed_time(ev[i][j + 1]) * 1e3 for i in instrumented])
        per_op[name] = {"bytes": nbytes[name], "us_mean": round(float(us.mean()), 2),
                        "us_median": round(float(np.median(us)), 2),
                        "GBps": round(nbytes[name] / (us.mean() * 1e-6) / 1e9, 1),
                        "frac_of_peak": round(nbytes[name] / (us.mean() * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}

    def sustained_us(fn, iters, first=0, stats=False):
        """Median us of fn(i), i = first, first+1, ..., over back-to-back calls
        (3 untimed first) on torch's current stream, with the GPU queued ahead
        of the loop."""
        cur = torch.cuda.current_stream(dev)
        evs = [(HipTimer(), HipTimer()) for _ in range(iters)]
        queue_ahead()
        for i in range(3 + iters):
            if i >= 3:
                evs[i - 3][0].record(cur)
            fn(first + i)
            if i >= 3:
                evs[i - 3][1].record(cur)
        torch.cuda.synchronize()
        us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
        if not stats:
            return round(float(np.median(us)), 2)
        return {"us_median": round(float(np.median(us)), 2),
                "us_p10": round(float(np.percentile(us, 10)), 2),
                "us_p90": round(float(np.percentile(us, 90)), 2)}


    def per_slot_form(handle, fn, nbytes_op):
        """The bf16 dispatch in its per-slot form (a workgroup cap above the item
        count selects it, uncapped) and, right after it under the same
        conditions, in the form the handle picks by default (blocked where that
        applies): a same-box, back-to-back comparison."""
        handle.set_max_workgroups(1 << 20)
        try:
            us = sustained_us(fn, args.sustained_iters)
        finally:
            handle.set_max_workgroups(0)
        us_default = sustained_us(fn, args.sustained_iters)
        return {"us_median": us, **rate(nbytes_op, us),
                "default_form_us_median": us_default}
    def rate(nb, us):
        return {"GBps": round(nb / (us * 1e-6) / 1e9, 1),
                "frac_of_peak": round(nb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}

    # Sustained per-op timings: each op alone, back to back over the same
    # rotating buffers (inputs from HBM). Every call finds the previous
    # call's dirty lines in the last-level cache and leaves as many behind, so
    # each call pays for its own writes reaching HBM.
    sustained = {}
    context = {}
    if args.sustained_iters > 0:
        for name in ops:
            st = sustained_us(lambda i, n=name: run_op(n, i), args.sustained_iters, stats=True)
            st.update(rate(nbytes[name], st["us_median"]))
            sustained[name] = st
        # MXFP8 dispatch (32-channel blocks, E8M0 scales), same method.
        mx_scales = [torch.empty((S, H // 32), dtype=torch.uint8, device=dev) for _ in range(3)]
        mx = mxfp8_bytes(T, H, k)
        us = sustained_us(lambda i: h.dispatch(B("xq", i), mxfp8=True, out=B("q_out", i),
                                               scales=mx_scales[i % 3]), args.sustained_iters)
        sustained["dispatch_mxfp8"] = {"bytes": mx, "us_median": us, **rate(mx, us)}
        del mx_scales

    if args.sustained_iters > 0 and "context" not in skip:
        # Context 1: the two dispatches reading one copy of x over and over, so
        # that x (2*T*H bytes) stays in the last-level cache -- as when the op
        # before dispatch has just written it. Not the headline.
        warm = {}
        for name, fn in (("dispatch_bf16", lambda i: h.dispatch(bufs["xb"][0], out=B("d_out", i))),
                         ("dispatch_fp8", lambda i: h.dispatch(bufs["xb"][0], fp8=True,
                                                               out=B("q_out", i),
                                                               scales=B("q_scales", i)))):
            us = sustained_us(fn, args.sustained_iters)
            warm[name] = {"us_median": us, **rate(nbytes[name], us)}
        context["x_cache_resident"] = warm
        # Context 2: a cross-check of the cold-input method -- every timed call
        # follows a 1 GiB read sweep (a reduction; no dirty lines) and then the
        # layout of the same ids (as in a step, where the layout's outputs are
        # fresh when the dispatch reads them; the sweep alone would evict them
        # too), both outside its events.
        sweep_src = torch.zeros(1 << 28, dtype=torch.float32, device=dev)
        sink = torch.zeros((), dtype=torch.float32, device=dev)
        evicted = {}
        for name in ("dispatch_bf16", "dispatch_fp8"):
            evs = [(HipTimer(), HipTimer()) for _ in range(args.sustained_iters)]
            for i in range(3 + args.sustained_iters):
                sink.copy_(sweep_src.amax())
                h.layout(bufs["idx"][0])
                if i >= 3:
                    evs[i - 3][0].record(stream)
                run_op(name, i)
                if i >= 3:
                    evs[i - 3][1].record(stream)
            torch.cuda.synchronize()
            us = float(np.median([a.elapsed_time(b) * 1e3 for a, b in evs]))
            evicted[name] = {"us_median": round(us, 2), **rate(nbytes[name], us)}
        context["x_evicted_by_sweep"] = evicted
        del sweep_src, sink
        # Context 3: torch's device-to-device copy of the bf16 dispatch's byte
        # count (half read, half written) and a plain write (fill) of the bf16
        # dispatch's output size, same method.
        half = nbytes["dispatch_bf16"] // 2
        wbytes = S * H * 2
        cbufs = [torch.empty(max(wbytes, 2 * half), dtype=torch.uint8, device=dev) for _ in range(3)]
        for label, moved, fn in (("copy_same_bytes", 2 * half,
                                  lambda b: b[half:2 * half].copy_(b[:half])),
                                 ("write_same_bytes", wbytes, lambda b: b[:wbytes].fill_(7))):
            us = sustained_us(lambda i, f=fn: f(cbufs[i % 3]), args.sustained_iters)
            context[label] = {"bytes": moved, "us_median": us,
                              "GBps": round(moved / (us * 1e-6) / 1e9, 1)}
        del cbufs
        # Context 4, same kernels and method: the bf16 and FP8 dispatches with
        # their destination rows in token order. When every slot of token t goes to
        # expert t*k / (T*k/E) (repeated ids are independent slots), the layout
        # puts slot (t, j) at row t*k + j: the same bytes as the workload's
        # routing, with the row writes sequential instead of spread over the E
        # expert regions at once. Not a figure of the workload.
        if S % E == 0 and (S // E) % k == 0:
            rows_per_expert = S // E
            seq_idx = (torch.arange(T, device=dev, dtype=torch.int32) * k // rows_per_expert)
            seq_idx = seq_idx.view(T, 1).expand(T, k).contiguous()
            h.layout(seq_idx)
            in_order = bool(torch.equal(h.view()["pos"].flatten(),
                                        torch.arange(S, device=dev, dtype=torch.int32)))
            us = sustained_us(lambda i: h.dispatch(B("xb", i), out=B("d_out", i)),
                              args.sustained_iters)
            context["dispatch_bf16_rows_in_order"] = {
                "us_median": us, **rate(nbytes["dispatch_bf16"], us),
                "positions_in_order": in_order,
                "routing": "every slot of token t on expert t*k/(T*k/E), not the workload's"}
            # the FP8 dispatch under the same in-order layout (its own x copies)
            us8 = sustained_us(lambda i: h.dispatch(B("xq", i), fp8=True, out=B("q_out", i),
                                                    scales=B("q_scales", i)),
                               args.sustained_iters)
            context["dispatch_fp8_rows_in_order"] = {
                "us_median": us8, **rate(nbytes["dispatch_fp8"], us8),
                "positions_in_order": in_order,
                "routing": "every slot of token t on expert t*k/(T*k/E), not the workload's"}
            h.layout(bufs["idx"][0])
        # Context 5, same method and inputs: the bf16 dispatch in its per-slot
        # form (a workgroup cap above the item count selects it, uncapped), for
        # a same-box comparison with the blocked form the step uses.
        context["dispatch_bf16_per_slot_form"] = per_slot_form(
            h, lambda i: h.dispatch(B("xb", i), out=B("d_out", i)), nbytes["dispatch_bf16"])

    # Rank-deduplicated exchange (one row per (token, rank)), sustained method.
    exchange = {}
    if args.sustained_iters > 0 and "rank" not in skip:
        h.rank_layout(bufs["idx"][0])
        torch.cuda.synchronize()
        rows = int(h.rank_view()["status"][0].item())
        cap = h.rank_capacity
        rb = [{"out": torch.empty((cap, H), dtype=torch.bfloat16, device=dev),
               "idx": torch.empty((cap, k), dtype=torch.int32, device=dev),
               "w": torch.empty((cap, k), dtype=torch.float32, device=dev)}
              for _ in range(copies_for(2 * cap * H))]
        RB = lambda i: rb[i % len(rb)]   # noqa: E731
        xb = {"rank_layout": 4 * S + 4 * S + 4 * T * R + 4 * rows,
              "dispatch_ranks": 2 * T * H + 2 * rows * H + 8 * rows * k + 12 * S,
              "combine_ranks": 2 * rows * H + 2 * T * H + 4 * T * R}
        calls = {"rank_layout": lambda i: h.rank_layout(B("idx", i)),
                 "dispatch_ranks": lambda i: h.dispatch_ranks(B("xb", i), B("idx", i), B("w", i),
                                                              out=RB(i)["out"],
                                                              recv_idx=RB(i)["idx"],
                                                              recv_w=RB(i)["w"]),
                 "combine_ranks": lambda i: h.combine_ranks(RB(i)["out"], out=B("c_out", i))}
        for i in range(len(rb)):
            calls["dispatch_ranks"](i)
        for name, fn in calls.items():
            us = sustained_us(fn, args.sustained_iters)
            exchange[name] = {"bytes": xb[name], "us_median": us,
                              "GBps": round(xb[name] / (us * 1e-6) / 1e9, 1)}
        exchange["rows"] = rows
        exchange["rows_without_dedup"] = S
        del rb

    # Bandwidth against the number of workgroups (4 wavefronts each) the payload
    # kernels may use (moe_set_max_workgroups), sustained method, 256 CUs.
    sweep = {}
    if args.workgroup_sweep:
        for capw in (16, 32, 64, 128, 256, 512, 1024, 0):
            h.set_max_workgroups(capw)
            row = {}
            for name in ("dispatch_bf16", "dispatch_fp8", "combine"):
                us = sustained_us(lambda i, n=name: run_op(n, i), 5)
                row[name] = round(nbytes[name] / (us * 1e-6) / 1e9, 1)
            sweep["uncapped" if capw == 0 else str(capw)] = row
        h.set_max_workgroups(0)

    # Compute-unit-limited streams: each payload op on n compute units (an
    # equal share of every XCD, moe_stream_create_cu_limited), then the bf16
    # dispatch and combine on n units concurrently with a bf16 GEMM
    # (8192 x 8192 x 8192, torch) on a stream limited to the other 256 - n.
    cu_limited = {}

    def measure_cu_limited():
        from combine_moe_dispatch_02_amd import CuLimitedStream
        total_cus = torch.cuda.get_device_properties(dev).multi_processor_count
        by_cus = {}
        for n in (8, 16, 32, 64, 128, total_cus):
            with CuLimitedStream(n, dev):
                row = {}
                for name in ("dispatch_bf16", "dispatch_fp8", "combine"):
                    us = sustained_us(lambda i, nm=name: run_op(nm, i), 5 if n < 64 else 10)
                    row[name] = round(nbytes[name] / (us * 1e-6) / 1e9, 1)
            by_cus[str(n)] = row
        cu_limited["GBps_by_cus"] = by_cus
        gm = 8192
        ga = torch.randn((gm, gm), dtype=torch.bfloat16, device=dev)
        gb = torch.randn((gm, gm), dtype=torch.bfloat16, device=dev)
        gc = torch.empty((gm, gm), dtype=torch.bfloat16, device=dev)
        gflop = 2.0 * gm ** 3

        def gemm(i):
            torch.mm(ga, gb, out=gc)

        def loop_us(fn, st, n):
            """Elapsed us of n back-to-back calls of fn on stream st (HIP events)."""
            e = (HipTimer(), HipTimer())
            with torch.cuda.stream(st):
                e[0].record(st)
                for i in range(n):
                    fn(i)
                e[1].record(st)
            torch.cuda.synchronize()
            return e[0].elapsed_time(e[1]) * 1e3

        def under_load(inner, st_in, n_in, outer, st_out, n_out):
            """us of n_in calls of `inner` on st_in while `outer` runs on
            st_out the whole time: the outer loop is enqueued first and the
            inner stream spins ~1 ms before its loop, so every inner call has
            outer work beside it. Returns (inner us, whether the outer loop's
            events bracket the inner loop's)."""
            eo = (HipTimer(), HipTimer())
            ei = (HipTimer(), HipTimer())
            with torch.cuda.stream(st_out):
                eo[0].record(st_out)
                for i in range(n_out):
                    outer(i)
                eo[1].record(st_out)
            with torch.cuda.stream(st_in):
                sleep = getattr(torch.cuda, "_sleep", None)
                if sleep is not None:
                    sleep(2_000_000)
                ei[0].record(st_in)
                for i in range(n_in):
                    inner(i)
                ei[1].record(st_in)
            torch.cuda.synchronize()
            covered = eo[0].elapsed_time(ei[0]) > 0 and ei[1].elapsed_time(eo[1]) > 0
            return ei[0].elapsed_time(ei[1]) * 1e3, covered

        # the GEMM alone on every compute unit, for reference
        for i in range(3):
            gemm(i)
        t_all = loop_us(gemm, stream, 20) / 20
        cu_limited["gemm_tflops_all_cus"] = round(gflop / (t_all * 1e-6) / 1e12, 1)
        overlap = {}
        for n in (32, 64):
            for op in ("dispatch_bf16", "combine"):
                dsx = CuLimitedStream(n, dev)
                gsx = CuLimitedStream(total_cus - n, dev)
                try:
                    fn = (lambda i, o=op: run_op(o, i))
                    loop_us(fn, dsx.stream, 3)
                    loop_us(gemm, gsx.stream, 3)
                    t_d = loop_us(fn, dsx.stream, 10) / 10
                    t_g = loop_us(gemm, gsx.stream, 10) / 10
                    # each side measured over ~8 ms of its own calls while the
                    # other runs over ~6x that (a slowed inner loop still fits)
                    nd, ng = max(5, int(8000 / t_d)), max(3, int(8000 / t_g))
                    us_d, cov_d = under_load(fn, dsx.stream, nd, gemm, gsx.stream,
                                             max(5, int(48000 / t_g)))
                    us_g, cov_g = under_load(gemm, gsx.stream, ng, fn, dsx.stream,
                                             max(10, int(48000 / t_d)))
                    # the same with the exchange's grid capped at 4 workgroups
                    # of 4 wavefronts per unit, whose wavefronts loop over the
                    # items: few workgroup launches instead of one per item
                    h.set_max_workgroups(4 * n)
                    t_l = loop_us(fn, dsx.stream, 10) / 10
                    nl = max(5, int(8000 / t_l))
                    us_l, cov_l = under_load(fn, dsx.stream, nl, gemm, gsx.stream,
                                             max(5, int(48000 / t_g)))
                    overlap[f"{op}_on_{n}_cus"] = {
                        "alone_GBps": round(nbytes[op] / (t_d * 1e-6) / 1e9, 1),
                        "beside_gemm_GBps": round(nd * nbytes[op] / (us_d * 1e-6) / 1e9, 1),
                        "gemm_cus": total_cus - n,
                        "gemm_alone_tflops": round(gflop / (t_g * 1e-6) / 1e12, 1),
                        "gemm_beside_exchange_tflops": round(ng * gflop / (us_g * 1e-6) / 1e12, 1),
                        "looping_grid": {
                            "alone_GBps": round(nbytes[op] / (t_l * 1e-6) / 1e9, 1),
                            "beside_gemm_GBps": round(nl * nbytes[op] / (us_l * 1e-6) / 1e9, 1)},
                        "calls_measured": [nd, ng, nl],
                        "fully_overlapped": bool(cov_d and cov_g and cov_l)}
                finally:
                    h.set_max_workgroups(0)
                    dsx.close()
                    gsx.close()
        cu_limited["with_gemm"] = overlap
        del ga, gb, gc

    if args.sustained_iters > 0 and "cus" not in skip:
        # A box whose runtime refuses CU-masked streams still reports the rest.
        from combine_moe_dispatch_02_amd import MoeError
        try:
            measure_cu_limited()
        except (MoeError, RuntimeError) as e:
            torch.cuda.synchronize()
            cu_limited["error"] = f"{type(e).__name__}: {e}"

    # Router at the prefill shape, and the decode-time path at 128 tokens
    # (fixed per-expert capacity 128: no slot can be dropped).
    router, decode = {}, {}
    if args.sustained_iters > 0 and "decode" not in skip:
        rbytes = 4 * T * E + 8 * T * k
        lg = [logits.clone() for _ in range(copies_for(4 * T * E))]
        us = sustained_us(lambda i: h.route(lg[i % len(lg)], s.weights, topk_idx=B("idx", i),
                                            topk_w=B("w", i)), args.sustained_iters)
        router = {"tokens": T, "experts": E, "topk": k, "score": s.weights, "bytes": rbytes,
                  "us_median": us, "GBps": round(rbytes / (us * 1e-6) / 1e9, 1)}
        Td, C = 128, 128
        hd = Handle(Td, H, k, E, R, device=dev)
        dsets = []
        for i in range(3):
            di, dw = hd.route(logits[:Td].contiguous(), s.weights)
            dsets.append({"idx": di, "w": dw, "x": B("xb", i)[:Td].contiguous(),
                          "lg": logits[:Td].clone(),
                          "out": torch.empty((E * C, H), dtype=torch.bfloat16, device=dev),
                          "q": torch.empty((E * C, H), dtype=torch.uint8, device=dev),
                          "qs": torch.empty((E * C, H // 128), dtype=torch.float32, device=dev),
                          "std": torch.empty((Td * k, H), dtype=torch.bfloat16, device=dev),
                          "c": torch.empty((Td, H), dtype=torch.bfloat16, device=dev)})
        D = lambda i: dsets[i % len(dsets)]   # noqa: E731
        torch.cuda.synchronize()
        decode["tokens"], decode["capacity"] = Td, C
        decode["route_us"] = sustained_us(
            lambda i: hd.route(D(i)["lg"], s.weights, topk_idx=D(i)["idx"], topk_w=D(i)["w"]),
            args.sustained_iters)
        decode["ll_dispatch_bf16_us"] = sustained_us(
            lambda i: hd.ll_dispatch(D(i)["idx"], D(i)["x"], C, out=D(i)["out"]), args.sustained_iters)
        decode["ll_dispatch_fp8_us"] = sustained_us(
            lambda i: hd.ll_dispatch(D(i)["idx"], D(i)["x"], C, "fp8", out=D(i)["q"], scales=D(i)["qs"]),
            args.sustained_iters)
        decode["ll_combine_us"] = sustained_us(
            lambda i: hd.ll_combine(D(i)["out"], D(i)["w"], out=D(i)["c"]), args.sustained_iters)

        def std_path(i):
            hd.layout(D(i)["idx"])
            hd.dispatch(D(i)["x"], out=D(i)["std"])
        decode["layout_plus_dispatch_bf16_us"] = sustained_us(std_path, args.sustained_iters)
        decode["combine_us"] = sustained_us(
            lambda i: hd.combine(D(i)["std"], D(i)["w"], out=D(i)["c"]), args.sustained_iters)
        decode["payload_bytes_bf16"] = 2 * Td * H + 2 * Td * k * H

        # The whole decode step (router -> decode-time dispatch -> combine of the
        # dispatched rows): eagerly, replayed as one captured HIP graph per
        # step, and as one graph holding ten steps (per-step figure), which
        # separates the graph launch's own cost from the kernels'.
        g0 = dsets[0]

        def decode_step():
            hd.route(g0["lg"], s.weights, topk_idx=g0["idx"], topk_w=g0["w"])
            hd.ll_dispatch(g0["idx"], g0["x"], C, out=g0["out"])
            hd.ll_combine(g0["out"], g0["w"], out=g0["c"])
        decode_step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            decode_step()
        graph10 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph10):
            for _ in range(10):
                decode_step()
        torch.cuda.synchronize()
        decode["step_eager_us"] = sustained_us(lambda i: decode_step(), args.sustained_iters)
        decode["step_graph_us"] = sustained_us(lambda i: graph.replay(), args.sustained_iters)
        decode["step_in_10_step_graph_us"] = round(
            sustained_us(lambda i: graph10.replay(), max(5, args.sustained_iters // 3)) / 10, 2)
        del graph, graph10, dsets, hd

        # Decode-time dispatch (fixed capacity = T, nothing dropped) and the
        # one-launch packed layout + dispatch against the two calls, over batch
        # sizes (bf16).
        scaling = {}
        for Tn in (32, 128, 512, 1024):
            hn = Handle(Tn, H, k, E, R, device=dev)
            ni, _ = hn.route(logits[:Tn].contiguous(), s.weights)
            nx = bufs["xb"][0][:Tn].contiguous()
            n_ll = torch.empty((E * Tn, H), dtype=torch.bfloat16, device=dev)
            n_std = torch.empty((Tn * k, H), dtype=torch.bfloat16, device=dev)

            def n_standard(i):
                hn.layout(ni)
                hn.dispatch(nx, out=n_std)
            scaling[str(Tn)] = {
                "ll_dispatch_bf16_us": sustained_us(lambda i: hn.ll_dispatch(ni, nx, Tn, out=n_ll),
                                                    args.sustained_iters),
                "layout_dispatch_bf16_us": sustained_us(
                    lambda i: hn.layout_dispatch(ni, nx, out=n_std), args.sustained_iters),
                "layout_plus_dispatch_bf16_us": sustained_us(n_standard, args.sustained_iters)}
            del hn, n_ll, n_std
        decode["by_tokens"] = scaling

    # The other full-size workloads (not the headline): sustained per-op
    # rates with inputs from HBM (the same rotation rule), routing by the
    # router kernel; plus the two dispatches reading one cached copy of x.
    others = {}
    if args.sustained_iters > 0 and "others" not in skip:
        for name in ("deepseek16b", "qwen3_skewed"):
            wo = make_workload(name)
            so = wo.shape
            To, Ho, ko = so.tokens, so.hidden, so.topk
            So = To * ko
            ho = Handle(To, Ho, ko, so.experts, so.ranks, device=dev)
            oi, ow = ho.route(torch.from_numpy(wo.logits).to(dev), so.weights)
            xo = torch.from_numpy(wo.x_bits.view(np.int16)).view(torch.bfloat16).to(dev)
            ob_ = {"x": [xo.clone() for _ in range(copies_for(2 * To * Ho))],
                   "idx": [oi.clone() for _ in range(3)], "w": [ow.clone() for _ in range(3)],
                   "d": [torch.empty((So, Ho), dtype=torch.bfloat16, device=dev)
                         for _ in range(copies_for(2 * So * Ho))],
                   "q": [torch.empty((So, Ho), dtype=torch.uint8, device=dev) for _ in range(3)],
                   "qs": [torch.empty((So, Ho // 128), dtype=torch.float32, device=dev)
                          for _ in range(3)],
                   "c": [torch.empty((To, Ho), dtype=torch.bfloat16, device=dev) for _ in range(3)]}
            del xo
            O = lambda key, i: ob_[key][i % len(ob_[key])]   # noqa: E731
            nb = op_bytes(To, Ho, ko)
            calls = {"layout": lambda i: ho.layout(O("idx", i)),
                     "dispatch_bf16": lambda i: ho.dispatch(O("x", i), out=O("d", i)),
                     "dispatch_fp8": lambda i: ho.dispatch(O("x", i), fp8=True, out=O("q", i),
                                                           scales=O("qs", i)),
                     "combine": lambda i: ho.combine(O("d", i), O("w", i), out=O("c", i))}
            ho.layout(ob_["idx"][0])
            for i in range(len(ob_["d"])):   # every expert-row set holds dispatched rows
                calls["dispatch_bf16"](i)
            row = {"tokens": To, "hidden": Ho, "experts": so.experts, "topk": ko,
                   "x_copies": len(ob_["x"]), "expert_row_sets": len(ob_["d"])}
            for op, fn in calls.items():
                us = sustained_us(fn, args.sustained_iters)
                row[op] = {"us_median": us, **rate(nb[op], us)}
            warm = {}
            for op, fn in (("dispatch_bf16", lambda i: ho.dispatch(ob_["x"][0], out=O("d", i))),
                           ("dispatch_fp8", lambda i: ho.dispatch(ob_["x"][0], fp8=True,
                                                                  out=O("q", i), scales=O("qs", i)))):
                us = sustained_us(fn, args.sustained_iters)
                warm[op] = {"us_median": us, **rate(nb[op], us)}
            row["x_cache_resident"] = warm
            row["dispatch_bf16_per_slot_form"] = per_slot_form(ho, calls["dispatch_bf16"],
                                                               nb["dispatch_bf16"])
            others[name] = row
            del ob_, ho
        torch.cuda.synchronize()

    dominant = max(("dispatch_bf16", "dispatch_fp8", "combine"), key=lambda n: per_op[n]["us_mean"])
    achieved = per_op[dominant]["GBps"]
    traffic = measured_traffic(dominant)
    result = {
        "metric": METRIC,
        "value": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{WORKLOAD}: T={T} H={H} E={E} in R={R} virtual ranks, top-{k}; "
                               "layout + bf16 dispatch + FP8 dispatch + bf16 combine, every input "
                               "read from HBM",
                   "tokens": T, "hidden": H, "experts": E, "virtual_ranks": R, "topk": k,
                   "x_copies_per_dispatch": n_x, "expert_row_sets": n_d},
        "frac_of_peak": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_source": (f"{os.path.relpath(TRAFFIC_FILE, os.path.dirname(os.path.abspath(__file__)))}"
                                        f" [{KERNEL_OF_OP[dominant]}]: rocprofv3 FETCH_SIZE + "
                                        "WRITE_SIZE per launch, copy-calibrated, taken from "
                                        "the same kernel sources (hash-checked)")
                     if traffic is not None else
                     "none: a source of the kernel changed since the counters were taken"},
        "ops": per_op,
        "instrumented_steps": len(instrumented),
        "sustained": sustained,
        "context": context,
        "workgroup_sweep_GBps": sweep,
        "cu_limited": cu_limited,
        "rank_exchange": exchange,
        "router": router,
        "decode": decode,
        "other_workloads": others,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample_tokens)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
