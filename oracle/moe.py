"""Plain CPU definitions of MoE token dispatch and combine (test infrastructure only).

What the pages say the two operators do:
  * "Inside the Nebius + PyTorch DeepSeek V3 recipe", section "Mixture-of-experts
    and wide expert parallelism": every MoE layer has a dispatch phase that
    sends each token to the experts the router picked for it, and a combine
    phase that brings the expert outputs back to the tokens' original
    positions.
  * Hybrid-EP news item, sections "Technical Structure" and "Availability and
    Integration": the two operators are dispatch and combine, and buffers are
    preallocated for the worst case because routing is dynamic.
  * "MoE / Hybrid-EP Validation", "Communication path comparison" and "FP8
    dispatch restriction": dispatch may carry FP8 payloads; the measured shape
    is hidden 7168, 4096 tokens per rank, top-8, EP=8.

The pages fix no formula, buffer layout or ordering, so this module writes out
the plainest reading (each reading is listed in the design notes):
  * Layout: a stable counting sort of the T*k (token, slot) pairs by expert id.
    Position = start of the expert's region + number of earlier pairs (token
    order, then slot order) routed to the same expert. Experts are split into
    R virtual ranks contiguously, so rank r's rows are one contiguous slab.
    Ids outside [0, E) are skipped: no row, pos = -1, counted as invalid.
  * Capacity is the worst case, T*k rows; rows past the valid total keep
    src_idx = -1.
  * bf16 dispatch copies each token row, bit for bit, to each of its k rows.
  * FP8 dispatch quantises each token once, per block of 128 channels:
    amax = max |x|, scale = amax / 448 in fp32 (correctly rounded), and each
    code = E4M3 nearest-even of the fp32 quotient x / scale; a block with
    amax = 0 gets scale 0 and signed-zero codes. Codes and the scale are
    written to every destination row of the token.
  * Combine: out[t] = bf16( sum_j w[t,j] * y[pos[t,j]] ), the sum taken over
    valid slots. The oracle forms it in fp64 (each product is exact there) and
    rounds once to bf16.
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_decode, bf16_encode, e4m3_decode, e4m3_encode

__all__ = ["layout", "layout_fixed_capacity", "dispatch_bf16", "dispatch_fp8", "combine",
           "dequant_fp8",
           "rank_layout", "dispatch_ranks", "combine_ranks", "quantize_mxfp8_rows",
           "dispatch_mxfp8", "dequant_mxfp8", "e8m0_decode", "FP8_BLOCK", "FP8_MAX", "MX_BLOCK"]

FP8_BLOCK = 128
FP8_MAX = np.float32(448.0)
MX_BLOCK = 32
E4M3_EMAX = 8          # exponent of E4M3's largest normal value, 448 = 1.75 * 2^8


def layout(topk_idx, num_experts: int, num_ranks: int) -> dict:
    """Histogram, exclusive scan and stable placement of the routed slots.

    Returns int64 numpy arrays:
      counts_e [E], offsets_e [E+1], counts_r [R], offsets_r [R+1],
      pos [T, k] (row of slot (t, j), or -1), src_idx [T*k] (token of each row,
      -1 past the valid total), and the int ``invalid`` (slots with ids outside
      [0, E)).
    """
    idx = np.asarray(topk_idx)
    T, k = idx.shape
    E, R = int(num_experts), int(num_ranks)
    if E <= 0 or R <= 0 or E % R != 0:
        raise ValueError("num_experts must be a positive multiple of num_ranks")
    rows = idx.tolist()

    # Histogram over all slots.
    counts_e = [0] * E
    for t in range(T):
        for j in range(k):
            e = rows[t][j]
            if 0 <= e < E:
                counts_e[e] += 1

    # Exclusive scan over experts; ranks own contiguous groups of E/R experts.
    offsets_e = [0] * (E + 1)
    for e in range(E):
        offsets_e[e + 1] = offsets_e[e] + counts_e[e]
    per = E // R
    counts_r = [sum(counts_e[r * per:(r + 1) * per]) for r in range(R)]
    offsets_r = [offsets_e[r * per] for r in range(R)] + [offsets_e[E]]

    # Stable placement: walk slots in (token, slot) order, one cursor per expert.
    cursor = offsets_e[:E]
    pos = [[-1] * k for _ in range(T)]
    src_idx = [-1] * (T * k)
    for t in range(T):
        for j in range(k):
            e = rows[t][j]
            if 0 <= e < E:
                p = cursor[e]
                cursor[e] = p + 1
                pos[t][j] = p
                src_idx[p] = t

    as64 = lambda a: np.asarray(a, dtype=np.int64)  # noqa: E731
    return {
        "counts_e": as64(counts_e), "offsets_e": as64(offsets_e),
        "counts_r": as64(counts_r), "offsets_r": as64(offsets_r),
        "pos": as64(pos).reshape(T, k), "src_idx": as64(src_idx),
        "invalid": T * k - offsets_e[E],
    }


def layout_fixed_capacity(topk_idx, num_experts: int, capacity: int) -> dict:
    """Placement into fixed per-expert regions (the decode-time layout).

    DeepEP's low-latency kernel family, the decode path of "Inside the Nebius
    + PyTorch DeepSeek V3 recipe", section "DeepEP", receives into buffers
    whose shape does not depend on the routing. Reading: expert e owns rows
    [e*C, (e+1)*C); within it, slots keep the stable (token, slot) order of
    the standard layout; a slot whose rank within its expert is C or more is
    dropped (pos = -1, counted). Ids outside [0, E) are skipped as invalid.

    Returns pos int64 [T, k], counts int64 [E] (rows received, at most C),
    and the ints ``dropped`` and ``invalid``.
    """
    idx = np.asarray(topk_idx)
    T, k = idx.shape
    E, C = int(num_experts), int(capacity)
    if E <= 0 or C <= 0:
        raise ValueError("num_experts and capacity must be positive")
    rows = idx.tolist()
    seen = [0] * E                 # slots routed to each expert so far
    pos = [[-1] * k for _ in range(T)]
    dropped = invalid = 0
    for t in range(T):
        for j in range(k):
            e = rows[t][j]
            if not 0 <= e < E:
                invalid += 1
                continue
            r = seen[e]
            seen[e] = r + 1
            if r < C:
                pos[t][j] = e * C + r
            else:
                dropped += 1
    return {"pos": np.asarray(pos, dtype=np.int64).reshape(T, k),
            "counts": np.minimum(np.asarray(seen, dtype=np.int64), C),
            "dropped": dropped, "invalid": invalid}


def _scatter_rows(rows_per_token: np.ndarray, pos: np.ndarray, capacity: int, fill):
    """out[pos[t, j]] = rows_per_token[t] for every valid slot; other rows = fill."""
    T, k = pos.shape
    out = np.full((capacity,) + rows_per_token.shape[1:], fill, dtype=rows_per_token.dtype)
    flat = pos.reshape(-1)
    tok = np.repeat(np.arange(T), k)
    ok = flat >= 0
    out[flat[ok]] = rows_per_token[tok[ok]]
    return out


def dispatch_bf16(x_bits, pos, rows=None) -> np.ndarray:
    """Copy token rows (bf16 bit patterns, uint16 [T, H]) to their rows
    (``rows`` rows in all, T*k by default)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    pos = np.asarray(pos)
    T, k = pos.shape
    return _scatter_rows(x_bits, pos, T * k if rows is None else rows, 0)


def quantize_fp8_rows(x_bits):
    """Per-token FP8 E4M3 quantisation with one fp32 scale per 128 channels.

    Returns (codes uint8 [T, H], scales float32 [T, H/128]).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, H = x_bits.shape
    if H % FP8_BLOCK != 0:
        raise ValueError("hidden must be a multiple of 128 for FP8 dispatch")
    xf = bf16_decode(x_bits).reshape(T, H // FP8_BLOCK, FP8_BLOCK)    # exact fp32
    amax = np.max(np.abs(xf), axis=2)                                    # fp32, exact
    nonzero = amax > 0
    with np.errstate(divide="ignore", invalid="ignore"):
        scale = np.where(nonzero, amax / FP8_MAX, np.float32(0.0)).astype(np.float32)
        quot = (xf / scale[:, :, None]).astype(np.float32)               # fp32 division
    quot = np.where(nonzero[:, :, None], quot, xf)                       # amax = 0: keep +-0
    codes = e4m3_encode(quot).reshape(T, H)
    return codes, scale


def dispatch_fp8(x_bits, pos, rows=None):
    """FP8 dispatch: quantise each token once, write codes + scales to its rows.

    Returns (codes uint8 [rows, H], scales float32 [rows, H/128]), rows = T*k
    by default; rows that no slot maps to hold zeros.
    """
    pos = np.asarray(pos)
    T, k = pos.shape
    n = T * k if rows is None else rows
    codes, scale = quantize_fp8_rows(x_bits)
    return (_scatter_rows(codes, pos, n, 0),
            _scatter_rows(scale, pos, n, np.float32(0.0)))


def combine(y_bits, w, pos, tokens=None, return_magnitude: bool = False):
    """Top-k weighted gather back to token order.

    out[t, h] = bf16( sum over valid j of w[t, j] * y[pos[t, j], h] ), with the
    sum formed in fp64 and rounded to bf16 once. ``tokens`` restricts the
    evaluation to those token indices (rows of the result follow its order).
    With ``return_magnitude`` also returns sum_j |w[t,j] * y[pos[t,j], h]| (fp64),
    the scale that bounds cancellation in any fp32 evaluation of the same sum.
    """
    y_bits = np.asarray(y_bits, dtype=np.uint16)
    w = np.asarray(w, dtype=np.float32)
    pos = np.asarray(pos)
    T, k = pos.shape
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    H = y_bits.shape[1]
    acc = np.zeros((toks.shape[0], H), dtype=np.float64)
    mag = np.zeros_like(acc)
    for j in range(k):
        p = pos[toks, j]
        ok = p >= 0
        rows = bf16_decode(y_bits[np.where(ok, p, 0)]).astype(np.float64)
        term = w[toks, j].astype(np.float64)[:, None] * rows
        term[~ok] = 0.0
        acc += term
        mag += np.abs(term)
    out = bf16_encode(acc)
    return (out, mag) if return_magnitude else out


def dequant_fp8(codes, scales) -> np.ndarray:
    """Expert-side dequantisation used by the tests: bf16(code value * scale)."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.float32)
    C, H = codes.shape
    vals = e4m3_decode(codes).reshape(C, H // FP8_BLOCK, FP8_BLOCK)
    prod = vals * scales.astype(np.float64)[:, :, None]                # exact in fp64
    return bf16_encode(prod.reshape(C, H))


# ---------------------------------------------------------------------------
# Rank-deduplicated exchange: one row per (token, destination rank).
#
# What an expert-parallel exchange carries ("Inside the Nebius + PyTorch
# DeepSeek V3 recipe", section "Mixture-of-experts and wide expert
# parallelism": each rank holds a subset of the experts, dispatch sends
# tokens to the ranks holding their experts): a token routed to several
# experts of one rank travels to that rank once. Readings (the pages give no
# formula): ranks own contiguous experts; a rank's rows are its tokens in
# token order; each row carries the token's k slots re-expressed for the
# receiver -- the local expert id (e - r*E/R) where the slot's expert lives
# on rank r, else -1 -- and the slot weights (0 where not local); combine
# adds the per-rank partial rows in ascending rank order and rounds once.


def rank_layout(topk_idx, num_experts: int, num_ranks: int) -> dict:
    """Which ranks each token goes to, and the rank-major row of each pair.

    Returns int64 arrays: in_rank [T, R] (0/1), counts_r [R], offsets_r
    [R+1], rank_pos [T, R] (row, or -1), rank_src [T*min(k, R)] (token of
    each row, -1 past the valid total).
    """
    idx = np.asarray(topk_idx)
    T, k = idx.shape
    E, R = int(num_experts), int(num_ranks)
    if E <= 0 or R <= 0 or E % R != 0:
        raise ValueError("num_experts must be a positive multiple of num_ranks")
    per = E // R
    rows = idx.tolist()
    in_rank = [[0] * R for _ in range(T)]
    for t in range(T):
        for j in range(k):
            e = rows[t][j]
            if 0 <= e < E:
                in_rank[t][e // per] = 1
    counts = [sum(in_rank[t][r] for t in range(T)) for r in range(R)]
    offsets = [0] * (R + 1)
    for r in range(R):
        offsets[r + 1] = offsets[r] + counts[r]
    cursor = offsets[:R]
    rank_pos = [[-1] * R for _ in range(T)]
    rank_src = [-1] * (T * min(k, R))
    for t in range(T):
        for r in range(R):
            if in_rank[t][r]:
                p = cursor[r]
                cursor[r] = p + 1
                rank_pos[t][r] = p
                rank_src[p] = t
    as64 = lambda a: np.asarray(a, dtype=np.int64)  # noqa: E731
    return {"in_rank": as64(in_rank).reshape(T, R), "counts_r": as64(counts),
            "offsets_r": as64(offsets), "rank_pos": as64(rank_pos).reshape(T, R),
            "rank_src": as64(rank_src)}


def dispatch_ranks(x_bits, topk_idx, topk_w, num_experts: int, num_ranks: int, rl: dict):
    """Rank-deduplicated bf16 dispatch with the receiver's routing metadata.

    Returns (rows uint16 [T*min(k,R), H], recv_idx int64 [same rows, k],
    recv_w float32 [same rows, k]); unused rows are zero / -1 / 0.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    idx = np.asarray(topk_idx)
    w = np.asarray(topk_w, dtype=np.float32)
    T, k = idx.shape
    E, R = int(num_experts), int(num_ranks)
    per = E // R
    cap = T * min(k, R)
    out = np.zeros((cap, x_bits.shape[1]), dtype=np.uint16)
    recv_idx = np.full((cap, k), -1, dtype=np.int64)
    recv_w = np.zeros((cap, k), dtype=np.float32)
    for t in range(T):
        for r in range(R):
            p = int(rl["rank_pos"][t, r])
            if p < 0:
                continue
            out[p] = x_bits[t]
            for j in range(k):
                e = int(idx[t, j])
                if 0 <= e < E and e // per == r:
                    recv_idx[p, j] = e - r * per
                    recv_w[p, j] = w[t, j]
    return out, recv_idx, recv_w


def combine_ranks(partial_bits, rank_pos, tokens=None, return_magnitude: bool = False):
    """out[t] = bf16( sum over ranks r in ascending order of partial[rank_pos[t, r]] ),
    summed in fp64 and rounded once; tokens with no rank get zeros. With
    ``return_magnitude`` also returns sum_r |partial[rank_pos[t, r]]|."""
    partial_bits = np.asarray(partial_bits, dtype=np.uint16)
    rank_pos = np.asarray(rank_pos)
    T, R = rank_pos.shape
    toks = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    acc = np.zeros((toks.shape[0], partial_bits.shape[1]), dtype=np.float64)
    mag = np.zeros_like(acc)
    for r in range(R):
        p = rank_pos[toks, r]
        ok = p >= 0
        rows = bf16_decode(partial_bits[np.where(ok, p, 0)]).astype(np.float64)
        rows[~ok] = 0.0
        acc += rows
        mag += np.abs(rows)
    out = bf16_encode(acc)
    return (out, mag) if return_magnitude else out


# ---------------------------------------------------------------------------
# MXFP8 dispatch: OCP Microscaling (MX) v1.0 format with E4M3 elements.
#
# The Hybrid-EP news item ("Efficiency Numbers") reports its Qwen3 run in
# MXFP8. The MX format (OCP Microscaling Formats specification v1.0): blocks
# of 32 elements share one E8M0 scale (an 8-bit power-of-two exponent, bias
# 127, no sign or mantissa); its conversion rule takes the shared exponent
# floor(log2(max |V|)) - emax_elem (emax_elem = 8 for E4M3), divides each
# element by 2^shared (exact: a power of two) and rounds it to the element
# format to nearest-even, clamping magnitudes above the largest normal (448).
# Readings (the pages give none): the shared exponent is clamped to E8M0's
# finite range [-127, 127]; an all-zero block gets code 0 (2^-127) and
# signed-zero elements.


def e8m0_decode(codes) -> np.ndarray:
    """E8M0 scale codes -> float64 powers of two (0xFF is NaN)."""
    c = np.asarray(codes).astype(np.int64)
    v = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, v)


def quantize_mxfp8_rows(x_bits):
    """Per-token MXFP8 quantisation: (codes uint8 [T, H], scales uint8 [T, H/32])."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, H = x_bits.shape
    if H % MX_BLOCK != 0:
        raise ValueError("hidden must be a multiple of 32 for MXFP8 dispatch")
    xf = bf16_decode(x_bits).astype(np.float64).reshape(T, H // MX_BLOCK, MX_BLOCK)
    amax = np.max(np.abs(xf), axis=2)
    nonzero = amax > 0
    _, e = np.frexp(np.where(nonzero, amax, 1.0))        # amax = m * 2^e, m in [0.5, 1)
    shared = np.clip(e - 1 - E4M3_EMAX, -127, 127)
    shared = np.where(nonzero, shared, -127)
    q = xf / np.ldexp(1.0, shared)[:, :, None]           # exact: division by 2^shared
    q = np.clip(q, -448.0, 448.0)
    codes = e4m3_encode(q).reshape(T, H)
    return codes, (shared + 127).astype(np.uint8)


def dispatch_mxfp8(x_bits, pos, rows=None):
    """MXFP8 dispatch: quantise each token once, write codes + E8M0 scales to its
    rows (T*k rows by default)."""
    pos = np.asarray(pos)
    T, k = pos.shape
    n = T * k if rows is None else rows
    codes, scale = quantize_mxfp8_rows(x_bits)
    return (_scatter_rows(codes, pos, n, 0), _scatter_rows(scale, pos, n, 0))


def dequant_mxfp8(codes, scales) -> np.ndarray:
    """bf16(code value * 2^(scale - 127)) (exact product, one rounding)."""
    codes = np.asarray(codes, dtype=np.uint8)
    C, H = codes.shape
    vals = e4m3_decode(codes).reshape(C, H // MX_BLOCK, MX_BLOCK)
    prod = vals * e8m0_decode(scales)[:, :, None]
    return bf16_encode(prod.reshape(C, H))
