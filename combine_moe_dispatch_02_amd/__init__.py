"""MoE expert-parallel token dispatch and combine for one MI355X (gfx950).

A thin binding over the C ABI of libmoe_ep.so (include/moe_ep.h): every step
runs in the library's HIP kernels; this module only checks tensor
dtypes/devices, passes raw pointers and torch's current HIP stream, and turns
status codes into exceptions. PyTorch provides device memory and streams.

Functions carry the C names (moe_dispatch_layout, moe_dispatch, moe_combine,
...). ``Handle`` bundles them with a workspace tensor for convenience.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (MOE_DTYPE_BF16, MOE_DTYPE_FP8_E4M3, MOE_DTYPE_MXFP8_E4M3, MOE_MX_BLOCK,
                   MOE_EP_FP8_BLOCK, MOE_EP_LL_MAX_TOKENS, MOE_EP_MAX_EXPERTS,
                   MOE_EP_MAX_TOPK, MOE_EP_STATUS_WORDS, MOE_EP_XCDS, MOE_SCORE_SIGMOID,
                   MOE_SCORE_SOFTMAX,
                   MoeConfig, MoeError, MoeLayoutView, MoeLlView, MoeRankLayoutView)

__all__ = ["Handle", "MoeError", "MoeConfig", "moe_workspace_bytes", "moe_handle_create",
           "moe_handle_destroy", "moe_dispatch_layout", "moe_dispatch_layout_noalloc",
           "moe_layout_view", "moe_dispatch",
           "moe_combine", "moe_rank_layout", "moe_rank_layout_view", "moe_dispatch_ranks",
           "moe_combine_ranks", "moe_set_max_workgroups", "moe_route", "moe_layout_dispatch",
           "moe_ll_dispatch",
           "moe_ll_view", "moe_ll_combine", "moe_status_string", "moe_last_error",
           "moe_cu_mask", "moe_stream_create_cu_limited", "moe_stream_destroy", "CuLimitedStream",
           "MOE_EP_XCDS",
           "MOE_DTYPE_BF16", "MOE_DTYPE_MXFP8_E4M3", "MOE_SCORE_SOFTMAX", "MOE_SCORE_SIGMOID",
           "MOE_EP_LL_MAX_TOKENS",
           "MOE_DTYPE_FP8_E4M3", "MOE_EP_MAX_EXPERTS", "MOE_EP_MAX_TOPK", "MOE_EP_FP8_BLOCK"]


def _config(max_tokens, hidden, topk, num_experts, num_ranks) -> MoeConfig:
    return MoeConfig(int(max_tokens), int(hidden), int(topk), int(num_experts), int(num_ranks))


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def _ptr(t: torch.Tensor | None, dtype, name: str, device=None) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the handle's workspace on {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


# Configuration of every handle this module created, so that the calls below
# can check tensor shapes against it: the library sees only pointers, and a
# tensor smaller than the configuration implies would be read or written out
# of bounds on the GPU.
_CONFIGS: dict[int, MoeConfig] = {}


def _matrix(t: torch.Tensor | None, name: str, cols: int, min_rows: int = 0) -> None:
    if t is None:
        return
    if t.dim() != 2 or t.shape[1] != cols:
        raise ValueError(f"{name} must be a [rows, {cols}] matrix, got shape {tuple(t.shape)}")
    if t.shape[0] < min_rows:
        raise ValueError(f"{name} has {t.shape[0]} rows; this call uses {min_rows}")


def _tokens(h: int, view_fn, view_type) -> int | None:
    """num_tokens of the handle's current layout of that kind, or None if it has none."""
    v = view_type()
    if view_fn(ctypes.c_void_p(h), ctypes.byref(v)) != _lib.MOE_OK:
        return None
    return int(v.num_tokens)


def _check_payload(cfg: MoeConfig, tokens: int | None, x, dtype, out, scales) -> None:
    _matrix(x, "x", cfg.hidden, tokens or 0)
    _matrix(out, "out", cfg.hidden)
    if out is None:
        return
    # a hidden size the quantised dtypes do not support is the library's error to report
    if dtype == MOE_DTYPE_FP8_E4M3 and cfg.hidden % MOE_EP_FP8_BLOCK == 0:
        _matrix(scales, "scales", cfg.hidden // MOE_EP_FP8_BLOCK, out.shape[0])
    elif dtype == MOE_DTYPE_MXFP8_E4M3 and cfg.hidden % MOE_EP_FP8_BLOCK == 0:
        _matrix(scales, "scales", cfg.hidden // MOE_MX_BLOCK, out.shape[0])


def moe_workspace_bytes(max_tokens, hidden, topk, num_experts, num_ranks) -> int:
    lib = _lib.load()
    cfg = _config(max_tokens, hidden, topk, num_experts, num_ranks)
    n = lib.moe_workspace_bytes(ctypes.byref(cfg))
    if n == 0:
        raise MoeError(_lib.MOE_ERR_UNSUPPORTED, lib.moe_last_error().decode())
    return int(n)


def moe_handle_create(max_tokens, hidden, topk, num_experts, num_ranks,
                      workspace_ptr: int, workspace_bytes: int) -> int:
    lib = _lib.load()
    cfg = _config(max_tokens, hidden, topk, num_experts, num_ranks)
    h = ctypes.c_void_p()
    _lib.check(lib.moe_handle_create(ctypes.byref(cfg), ctypes.c_void_p(workspace_ptr),
                                     workspace_bytes, ctypes.byref(h)))
    _CONFIGS[int(h.value)] = cfg
    return int(h.value)


def moe_handle_destroy(h: int) -> None:
    _CONFIGS.pop(int(h or 0), None)
    _lib.load().moe_handle_destroy(ctypes.c_void_p(h))


def moe_dispatch_layout(h: int, topk_idx: torch.Tensor, stream=None) -> None:
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [num_tokens, topk]")
    p = _ptr(topk_idx, torch.int32, "topk_idx")
    cfg = _CONFIGS.get(h)
    if cfg is not None:
        _matrix(topk_idx, "topk_idx", cfg.topk)
    _lib.check(_lib.load().moe_dispatch_layout(ctypes.c_void_p(h), ctypes.c_void_p(p),
                                               topk_idx.shape[0], _stream(stream, topk_idx.device)))


def moe_dispatch_layout_noalloc(topk_idx: torch.Tensor, num_experts: int, num_ranks: int,
                                pos: torch.Tensor, src_idx: torch.Tensor, counts_e: torch.Tensor,
                                offsets_e: torch.Tensor, counts_r: torch.Tensor,
                                offsets_r: torch.Tensor, status: torch.Tensor, stream=None) -> None:
    """The layout into caller-owned int32 tensors, with no handle, workspace or
    allocation (its histograms live in the library's static device array)."""
    T, k = (int(topk_idx.shape[0]), int(topk_idx.shape[1])) if topk_idx.dim() == 2 else (-1, -1)
    if T < 0:
        raise ValueError(f"topk_idx must be [num_tokens, topk], got shape {tuple(topk_idx.shape)}")
    dev = topk_idx.device
    want = {"pos": (pos, T * k), "src_idx": (src_idx, T * k), "counts_e": (counts_e, num_experts),
            "offsets_e": (offsets_e, num_experts + 1), "counts_r": (counts_r, num_ranks),
            "offsets_r": (offsets_r, num_ranks + 1), "status": (status, MOE_EP_STATUS_WORDS)}
    ptrs = {}
    for name, (t, n) in want.items():
        ptrs[name] = _ptr(t, torch.int32, name, dev)
        if t.numel() < n:
            raise ValueError(f"{name} has {t.numel()} entries; this call writes {n}")
    pi = _ptr(topk_idx, torch.int32, "topk_idx", dev)
    _lib.check(_lib.load().moe_dispatch_layout_noalloc(
        ctypes.c_void_p(pi), T, k, int(num_experts), int(num_ranks),
        *(ctypes.c_void_p(ptrs[n]) for n in want), _stream(stream, dev)))


def moe_layout_view(h: int) -> MoeLayoutView:
    v = MoeLayoutView()
    _lib.check(_lib.load().moe_layout_view(ctypes.c_void_p(h), ctypes.byref(v)))
    return v


def _payload_ptrs(x, dtype, out, scales):
    px = _ptr(x, torch.bfloat16, "x")
    po = _ptr(out, torch.bfloat16 if dtype == MOE_DTYPE_BF16 else torch.uint8, "out")
    ps = None
    if dtype == MOE_DTYPE_FP8_E4M3:
        ps = _ptr(scales, torch.float32, "scales")
    elif dtype == MOE_DTYPE_MXFP8_E4M3:
        ps = _ptr(scales, torch.uint8, "scales")
    return px, po, ps


def moe_dispatch(h: int, x: torch.Tensor, dtype: int, out: torch.Tensor,
                 scales: torch.Tensor | None = None, stream=None) -> None:
    px, po, ps = _payload_ptrs(x, dtype, out, scales)
    cfg = _CONFIGS.get(h)
    if cfg is not None:
        lib = _lib.load()
        _check_payload(cfg, _tokens(h, lib.moe_layout_view, MoeLayoutView), x, dtype, out, scales)
    _lib.check(_lib.load().moe_dispatch(ctypes.c_void_p(h), ctypes.c_void_p(px), int(dtype),
                                        ctypes.c_void_p(po), ctypes.c_void_p(ps),
                                        out.shape[0], _stream(stream, x.device)))


def moe_combine(h: int, y: torch.Tensor, w: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    py = _ptr(y, torch.bfloat16, "y")
    pw = _ptr(w, torch.float32, "w")
    po = _ptr(out, torch.bfloat16, "out")
    cfg = _CONFIGS.get(h)
    if cfg is not None:
        tokens = _tokens(h, _lib.load().moe_layout_view, MoeLayoutView) or 0
        _matrix(y, "y", cfg.hidden)
        _matrix(w, "w", cfg.topk, tokens)
        _matrix(out, "out", cfg.hidden, tokens)
    _lib.check(_lib.load().moe_combine(ctypes.c_void_p(h), ctypes.c_void_p(py), y.shape[0],
                                       ctypes.c_void_p(pw), ctypes.c_void_p(po),
                                       _stream(stream, y.device)))


def moe_rank_layout(h: int, topk_idx: torch.Tensor, stream=None) -> None:
    if topk_idx.dim() != 2:
        raise ValueError("topk_idx must be [num_tokens, topk]")
    p = _ptr(topk_idx, torch.int32, "topk_idx")
    cfg = _CONFIGS.get(h)
    if cfg is not None:
        _matrix(topk_idx, "topk_idx", cfg.topk)
    _lib.check(_lib.load().moe_rank_layout(ctypes.c_void_p(h), ctypes.c_void_p(p),
                                           topk_idx.shape[0], _stream(stream, topk_idx.device)))


def moe_rank_layout_view(h: int) -> MoeRankLayoutView:
    v = MoeRankLayoutView()
    _lib.check(_lib.load().moe_rank_layout_view(ctypes.c_void_p(h), ctypes.byref(v)))
    return v


def moe_dispatch_ranks(h: int, x: torch.Tensor, topk_idx: torch.Tensor, w: torch.Tensor,
                       out: torch.Tensor, recv_idx: torch.Tensor, recv_w: torch.Tensor,
                       stream=None) -> None:
    args = [_ptr(x, torch.bfloat16, "x"), _ptr(topk_idx, torch.int32, "topk_idx"),
            _ptr(w, torch.float32, "w"), _ptr(out, torch.bfloat16, "out"),
            _ptr(recv_idx, torch.int32, "recv_idx"), _ptr(recv_w, torch.float32, "recv_w")]
    cfg = _CONFIGS.get(h)
    if cfg is not None:
        tokens = _tokens(h, _lib.load().moe_rank_layout_view, MoeRankLayoutView) or 0
        _matrix(x, "x", cfg.hidden, tokens)
        _matrix(topk_idx, "topk_idx", cfg.topk, tokens)
        _matrix(w, "w", cfg.topk, tokens)
        _matrix(out, "out", cfg.hidden)
        _matrix(recv_idx, "recv_idx", cfg.topk, out.shape[0])
        _matrix(recv_w, "recv_w", cfg.topk, out.shape[0])
    _lib.check(_lib.load().moe_dispatch_ranks(ctypes.c_void_p(h), *[ctypes.c_void_p(a) for a in args],
                                              out.shape[0], _stream(stream, x.device)))


def moe_combine_ranks(h: int, y: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    py = _ptr(y, torch.bfloat16, "y")
    po = _ptr(out, torch.bfloat16, "out")
    cfg = _CONFIGS.get(h)
    if cfg is not None:
        tokens = _tokens(h, _lib.load().moe_rank_layout_view, MoeRankLayoutView) or 0
        _matrix(y, "y", cfg.hidden)
        _matrix(out, "out", cfg.hidden, tokens)
    _lib.check(_lib.load().moe_combine_ranks(ctypes.c_void_p(h), ctypes.c_void_p(py), y.shape[0],
                                             ctypes.c_void_p(po), _stream(stream, y.device)))


def moe_set_max_workgroups(h: int, max_workgroups: int) -> None:
    _lib.check(_lib.load().moe_set_max_workgroups(ctypes.c_void_p(h), int(max_workgroups)))


def moe_route(h: int, logits: torch.Tensor, score: int, topk_idx: torch.Tensor,
              topk_w: torch.Tensor, stream=None) -> None:
    pl = _ptr(logits, torch.float32, "logits")
    pi = _ptr(topk_idx, torch.int32, "topk_idx")
    pw = _ptr(topk_w, torch.float32, "topk_w")
    cfg = _CONFIGS.get(h)
    if cfg is not None:
        _matrix(logits, "logits", cfg.num_experts)
        _matrix(topk_idx, "topk_idx", cfg.topk, logits.shape[0])
        _matrix(topk_w, "topk_w", cfg.topk, logits.shape[0])
    _lib.check(_lib.load().moe_route(ctypes.c_void_p(h), ctypes.c_void_p(pl), int(logits.shape[0]),
                                     int(score), ctypes.c_void_p(pi), ctypes.c_void_p(pw),
                                     _stream(stream, logits.device)))


def moe_layout_dispatch(h: int, topk_idx: torch.Tensor, x: torch.Tensor, dtype: int,
                        out: torch.Tensor, scales: torch.Tensor | None, stream=None) -> None:
    pi = _ptr(topk_idx, torch.int32, "topk_idx")
    px, po, ps = _payload_ptrs(x, dtype, out, scales)
    cfg = _CONFIGS.get(h)
    if cfg is not None:
        _matrix(topk_idx, "topk_idx", cfg.topk)
        _check_payload(cfg, topk_idx.shape[0], x, dtype, out, scales)
    _lib.check(_lib.load().moe_layout_dispatch(
        ctypes.c_void_p(h), ctypes.c_void_p(pi), int(topk_idx.shape[0]), ctypes.c_void_p(px),
        int(dtype), ctypes.c_void_p(po), ctypes.c_void_p(ps), out.shape[0],
        _stream(stream, x.device)))


def moe_ll_dispatch(h: int, topk_idx: torch.Tensor, capacity: int, x: torch.Tensor, dtype: int,
                    out: torch.Tensor, scales: torch.Tensor | None, stream=None) -> None:
    pi = _ptr(topk_idx, torch.int32, "topk_idx")
    px, po, ps = _payload_ptrs(x, dtype, out, scales)
    cfg = _CONFIGS.get(h)
    if cfg is not None:
        _matrix(topk_idx, "topk_idx", cfg.topk)
        _check_payload(cfg, topk_idx.shape[0], x, dtype, out, scales)
    _lib.check(_lib.load().moe_ll_dispatch(
        ctypes.c_void_p(h), ctypes.c_void_p(pi), int(topk_idx.shape[0]), int(capacity),
        ctypes.c_void_p(px), int(dtype), ctypes.c_void_p(po), ctypes.c_void_p(ps), out.shape[0],
        _stream(stream, x.device)))


def moe_ll_view(h: int) -> MoeLlView:
    v = MoeLlView()
    _lib.check(_lib.load().moe_ll_view(ctypes.c_void_p(h), ctypes.byref(v)))
    return v


def moe_ll_combine(h: int, y: torch.Tensor, w: torch.Tensor, out: torch.Tensor,
                   stream=None) -> None:
    py = _ptr(y, torch.bfloat16, "y")
    pw = _ptr(w, torch.float32, "w")
    po = _ptr(out, torch.bfloat16, "out")
    cfg = _CONFIGS.get(h)
    if cfg is not None:
        tokens = _tokens(h, _lib.load().moe_ll_view, MoeLlView) or 0
        _matrix(y, "y", cfg.hidden)
        _matrix(w, "w", cfg.topk, tokens)
        _matrix(out, "out", cfg.hidden, tokens)
    _lib.check(_lib.load().moe_ll_combine(ctypes.c_void_p(h), ctypes.c_void_p(py), y.shape[0],
                                          ctypes.c_void_p(pw), ctypes.c_void_p(po),
                                          _stream(stream, y.device)))


def moe_cu_mask(total_cus: int, num_cus: int) -> list[int]:
    """The compute-unit mask moe_stream_create_cu_limited uses: num_cus of
    total_cus units, an equal share of every XCD (host only)."""
    words = (int(total_cus) + 31) // 32
    mask = (ctypes.c_uint32 * max(words, 1))()
    _lib.check(_lib.load().moe_cu_mask(int(total_cus), int(num_cus), mask, words))
    return list(mask)[:words]


def moe_stream_create_cu_limited(num_cus: int) -> int:
    """A raw hipStream_t (int) on the current device limited to num_cus compute units."""
    s = ctypes.c_void_p()
    _lib.check(_lib.load().moe_stream_create_cu_limited(int(num_cus), ctypes.byref(s)))
    return int(s.value)


def moe_stream_destroy(stream: int) -> None:
    _lib.check(_lib.load().moe_stream_destroy(ctypes.c_void_p(int(stream))))


class CuLimitedStream:
    """A stream whose kernels may use only num_cus compute units (an equal
    share of every XCD), as a torch stream: ``with CuLimitedStream(64) as s:``
    makes it torch's current stream, so the Handle calls and torch ops inside
    run on those units. The stream is synchronised and destroyed on exit (or
    by close())."""

    def __init__(self, num_cus: int, device=None):
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None \
            else torch.device(device)
        with torch.cuda.device(self.device):
            self._raw = moe_stream_create_cu_limited(num_cus)
        self.num_cus = int(num_cus)
        self.stream = torch.cuda.ExternalStream(self._raw, device=self.device)
        self._ctx = None

    def __enter__(self):
        self._ctx = torch.cuda.stream(self.stream)
        self._ctx.__enter__()
        return self.stream

    def __exit__(self, *exc):
        self._ctx.__exit__(*exc)
        self._ctx = None
        self.close()
        return False

    def close(self):
        if self._raw:
            self.stream.synchronize()
            moe_stream_destroy(self._raw)
            self._raw = 0

    def __del__(self):
        try:
            self.close()
        except Exception:   # interpreter shutdown: the runtime may be gone
            pass


def moe_status_string(status: int) -> str:
    return _lib.load().moe_status_string(int(status)).decode()


def moe_last_error() -> str:
    return _lib.load().moe_last_error().decode()


class Handle:
    """A handle plus its caller-owned workspace tensor.

    layout(topk_idx) -> dispatch(x[, fp8]) -> [experts] -> combine(y, w).
    """

    def __init__(self, max_tokens, hidden, topk, num_experts, num_ranks, device="cuda"):
        self.max_tokens, self.hidden, self.topk = int(max_tokens), int(hidden), int(topk)
        self.num_experts, self.num_ranks = int(num_experts), int(num_ranks)
        nbytes = moe_workspace_bytes(max_tokens, hidden, topk, num_experts, num_ranks)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.device = self.workspace.device
        self.h = moe_handle_create(max_tokens, hidden, topk, num_experts, num_ranks,
                                   self.workspace.data_ptr(), nbytes)
        self._destroy = _lib.load().moe_handle_destroy   # kept for use at interpreter exit
        self._configs = _CONFIGS                         # likewise
        self.num_tokens = None
        self.rank_num_tokens = None
        self.ll_num_tokens = None

    def __del__(self):
        h = getattr(self, "h", None)
        if h:
            self._configs.pop(h, None)
            self._destroy(ctypes.c_void_p(h))
            self.h = None

    def layout(self, topk_idx: torch.Tensor, stream=None) -> None:
        _ptr(topk_idx, torch.int32, "topk_idx", self.device)
        moe_dispatch_layout(self.h, topk_idx, stream)
        self.num_tokens = int(topk_idx.shape[0])

    # ---- rank-deduplicated exchange
    def rank_layout(self, topk_idx: torch.Tensor, stream=None) -> None:
        _ptr(topk_idx, torch.int32, "topk_idx", self.device)
        moe_rank_layout(self.h, topk_idx, stream)
        self.rank_num_tokens = int(topk_idx.shape[0])

    @property
    def rank_capacity(self) -> int:
        return self.rank_num_tokens * min(self.topk, self.num_ranks)

    def dispatch_ranks(self, x, topk_idx, w, out=None, recv_idx=None, recv_w=None, stream=None):
        """One bf16 row per (token, rank) + receiver metadata (local ids, weights)."""
        rows = self.rank_capacity
        if out is None:
            out = torch.empty((rows, self.hidden), dtype=torch.bfloat16, device=self.device)
        if recv_idx is None:
            recv_idx = torch.empty((rows, self.topk), dtype=torch.int32, device=self.device)
        if recv_w is None:
            recv_w = torch.empty((rows, self.topk), dtype=torch.float32, device=self.device)
        moe_dispatch_ranks(self.h, x, topk_idx, w, out, recv_idx, recv_w, stream)
        return out, recv_idx, recv_w

    def combine_ranks(self, y, out=None, stream=None) -> torch.Tensor:
        if out is None:
            out = torch.empty((self.rank_num_tokens, self.hidden), dtype=torch.bfloat16,
                              device=self.device)
        moe_combine_ranks(self.h, y, out, stream)
        return out

    def rank_view(self) -> dict:
        """The last rank layout's arrays as int32 tensors (views into the workspace)."""
        v = moe_rank_layout_view(self.h)
        base = self.workspace.data_ptr()

        def arr(ptr, n):
            off = ptr - base
            return self.workspace[off:off + 4 * n].view(torch.int32)

        R, T, cap = self.num_ranks, v.num_tokens, v.capacity
        return {"rank_pos": arr(v.rank_pos, T * R).view(T, R),
                "slot_row": arr(v.slot_row, T * self.topk).view(T, self.topk),
                "rank_src": arr(v.src_idx, cap), "counts_r": arr(v.counts_r, R),
                "offsets_r": arr(v.offsets_r, R + 1), "status": arr(v.status, MOE_EP_STATUS_WORDS)}

    # ---- router
    def route(self, logits: torch.Tensor, score: str = "softmax", topk_idx=None, topk_w=None,
              stream=None):
        """fp32 logits [T, E] -> (topk_idx int32 [T, k], topk_w fp32 [T, k])."""
        _ptr(logits, torch.float32, "logits", self.device)
        code = {"softmax": MOE_SCORE_SOFTMAX, "sigmoid": MOE_SCORE_SIGMOID}[score]
        T = int(logits.shape[0])
        if topk_idx is None:
            topk_idx = torch.empty((T, self.topk), dtype=torch.int32, device=self.device)
        if topk_w is None:
            topk_w = torch.empty((T, self.topk), dtype=torch.float32, device=self.device)
        moe_route(self.h, logits, code, topk_idx, topk_w, stream)
        return topk_idx, topk_w

    # ---- layout and dispatch in one launch (small batches)
    def layout_dispatch(self, topk_idx: torch.Tensor, x: torch.Tensor, dtype: str = "bf16",
                        out=None, scales=None, stream=None):
        """layout() + dispatch() in one launch: rows [T*k, H] bf16, or (codes, scales)."""
        _ptr(topk_idx, torch.int32, "topk_idx", self.device)
        _ptr(x, torch.bfloat16, "x", self.device)
        code = {"bf16": MOE_DTYPE_BF16, "fp8": MOE_DTYPE_FP8_E4M3,
                "mxfp8": MOE_DTYPE_MXFP8_E4M3}[dtype]
        rows = int(topk_idx.shape[0]) * self.topk
        if out is None:
            out = torch.empty((rows, self.hidden),
                              dtype=torch.bfloat16 if code == MOE_DTYPE_BF16 else torch.uint8,
                              device=self.device)
        if scales is None and code == MOE_DTYPE_FP8_E4M3:
            scales = torch.empty((rows, self.hidden // MOE_EP_FP8_BLOCK), dtype=torch.float32,
                                 device=self.device)
        if scales is None and code == MOE_DTYPE_MXFP8_E4M3:
            scales = torch.empty((rows, self.hidden // MOE_MX_BLOCK), dtype=torch.uint8,
                                 device=self.device)
        moe_layout_dispatch(self.h, topk_idx, x, code, out, scales, stream)
        self.num_tokens = int(topk_idx.shape[0])
        return out if code == MOE_DTYPE_BF16 else (out, scales)

    # ---- decode-time (fixed-capacity) dispatch and combine
    def ll_dispatch(self, topk_idx: torch.Tensor, x: torch.Tensor, capacity: int,
                    dtype: str = "bf16", out=None, scales=None, stream=None):
        """Rows [E * capacity, H]: bf16, or (codes, scales) for "fp8" / "mxfp8"."""
        _ptr(topk_idx, torch.int32, "topk_idx", self.device)
        _ptr(x, torch.bfloat16, "x", self.device)
        code = {"bf16": MOE_DTYPE_BF16, "fp8": MOE_DTYPE_FP8_E4M3,
                "mxfp8": MOE_DTYPE_MXFP8_E4M3}[dtype]
        rows = self.num_experts * int(capacity)
        if out is None:
            out = torch.empty((rows, self.hidden),
                              dtype=torch.bfloat16 if code == MOE_DTYPE_BF16 else torch.uint8,
                              device=self.device)
        if scales is None and code == MOE_DTYPE_FP8_E4M3:
            scales = torch.empty((rows, self.hidden // MOE_EP_FP8_BLOCK), dtype=torch.float32,
                                 device=self.device)
        if scales is None and code == MOE_DTYPE_MXFP8_E4M3:
            scales = torch.empty((rows, self.hidden // MOE_MX_BLOCK), dtype=torch.uint8,
                                 device=self.device)
        moe_ll_dispatch(self.h, topk_idx, capacity, x, code, out, scales, stream)
        self.ll_num_tokens = int(topk_idx.shape[0])
        return out if code == MOE_DTYPE_BF16 else (out, scales)

    def ll_view(self) -> dict:
        """Positions [T, k], counts [E] and status [4] of the last ll_dispatch."""
        v = moe_ll_view(self.h)
        base = self.workspace.data_ptr()

        def arr(ptr, n):
            off = ptr - base
            return self.workspace[off:off + 4 * n].view(torch.int32)

        T = v.num_tokens
        return {"pos": arr(v.pos, T * self.topk).view(T, self.topk),
                "counts": arr(v.counts, self.num_experts), "status": arr(v.status, 4),
                "capacity": v.capacity, "rows": v.rows}

    def ll_combine(self, y: torch.Tensor, w: torch.Tensor, out=None, stream=None) -> torch.Tensor:
        _ptr(y, torch.bfloat16, "y", self.device)
        if out is None:
            out = torch.empty((self.ll_num_tokens, self.hidden), dtype=torch.bfloat16,
                              device=self.device)
        moe_ll_combine(self.h, y, w, out, stream)
        return out

    def set_max_workgroups(self, n: int) -> None:
        """Cap dispatch/combine at n workgroups (0: no cap)."""
        moe_set_max_workgroups(self.h, n)

    @property
    def capacity(self) -> int:
        return self.num_tokens * self.topk

    def dispatch(self, x: torch.Tensor, fp8: bool = False, out=None, scales=None, stream=None,
                 mxfp8: bool = False):
        """bf16 rows -> [capacity, H] bf16; (uint8 codes, fp32 scales [., H/128]) with
        fp8; (uint8 codes, uint8 E8M0 scales [., H/32]) with mxfp8."""
        _ptr(x, torch.bfloat16, "x", self.device)
        rows = self.capacity
        if mxfp8:
            if out is None:
                out = torch.empty((rows, self.hidden), dtype=torch.uint8, device=self.device)
            if scales is None:
                scales = torch.empty((rows, self.hidden // MOE_MX_BLOCK), dtype=torch.uint8,
                                     device=self.device)
            moe_dispatch(self.h, x, MOE_DTYPE_MXFP8_E4M3, out, scales, stream)
            return out, scales
        if fp8:
            if out is None:
                out = torch.empty((rows, self.hidden), dtype=torch.uint8, device=self.device)
            if scales is None:
                scales = torch.empty((rows, self.hidden // MOE_EP_FP8_BLOCK), dtype=torch.float32,
                                     device=self.device)
            moe_dispatch(self.h, x, MOE_DTYPE_FP8_E4M3, out, scales, stream)
            return out, scales
        if out is None:
            out = torch.empty((rows, self.hidden), dtype=torch.bfloat16, device=self.device)
        moe_dispatch(self.h, x, MOE_DTYPE_BF16, out, None, stream)
        return out

    def combine(self, y: torch.Tensor, w: torch.Tensor, out=None, stream=None) -> torch.Tensor:
        _ptr(y, torch.bfloat16, "y", self.device)
        if out is None:
            out = torch.empty((self.num_tokens, self.hidden), dtype=torch.bfloat16,
                              device=self.device)
        moe_combine(self.h, y, w, out, stream)
        return out

    def view(self) -> dict:
        """The last layout's arrays as int32 tensors (views into the workspace)."""
        v = moe_layout_view(self.h)
        base = self.workspace.data_ptr()

        def arr(ptr, n):
            off = ptr - base
            return self.workspace[off:off + 4 * n].view(torch.int32)

        E, R, T, cap = self.num_experts, self.num_ranks, v.num_tokens, v.capacity
        return {"pos": arr(v.pos, cap).view(T, self.topk), "src_idx": arr(v.src_idx, cap),
                "counts_e": arr(v.counts_e, E), "offsets_e": arr(v.offsets_e, E + 1),
                "counts_r": arr(v.counts_r, R), "offsets_r": arr(v.offsets_r, R + 1),
                "status": arr(v.status, MOE_EP_STATUS_WORDS)}
