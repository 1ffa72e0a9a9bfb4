"""Seeded synthetic inputs for MoE token dispatch / combine.

This module only draws inputs. It holds none of the dispatch or combine
arithmetic and is shared by the oracle tests, the HIP parity tests and the
benchmark. Everything here runs on the CPU with numpy; the one rounding step
(fp32 -> bf16 for the activations) uses torch's CPU cast, a library routine
that neither the oracle nor the HIP path uses.

Workload shapes follow the pages:
  * "MoE / Hybrid-EP Validation" (awslabs accelerated-compute tutorials),
    table "Communication path comparison (measured reference)": one rank of
    an EP=8 group at hidden 7168, 4096 tokens per rank, top-8.
  * "Inside the Nebius + PyTorch DeepSeek V3 recipe", section
    "Mixture-of-experts and wide expert parallelism": DeepSeek V3 routes each
    token to 8 of 256 experts; the benchmark section names DeepSeek-16B
    (64 experts).
  * The cryptojournalpost Hybrid-EP news item, section "Efficiency Numbers":
    a Qwen3-235B run, used here for the skewed, larger-T configuration.

The generator draws router logits, not routing decisions: the top-k
selection and its weights are part of the method (the library has a router
kernel, the oracle a router definition), so callers route the logits
themselves -- the tests through the oracle, the benchmark through the
library. Each shape names its weighting ("softmax", or "sigmoid" scores
divided by their sum for the DeepSeek-V3-like shapes).
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = ["Workload", "CONFIGS", "make_workload", "make_expert_outputs", "bf16_bits_from_f32"]


@dataclasses.dataclass(frozen=True)
class Shape:
    name: str
    tokens: int        # T, tokens on this rank
    hidden: int        # H
    experts: int       # E
    ranks: int         # R, virtual EP ranks (experts are split contiguously)
    topk: int          # k
    logits: str        # "uniform", "normal" or "zipf"
    weights: str       # "softmax" or "sigmoid"
    fp8: bool = False  # FP8 dispatch workload


# Index i of CONFIGS is the workload's position in the workload list; the seed
# of workload i is 1000 + i.
CONFIGS = (
    Shape("tiny", 128, 256, 8, 2, 2, "uniform", "softmax"),
    Shape("deepseek16b", 4096, 2048, 64, 8, 6, "normal", "softmax"),
    Shape("deepseekv3", 4096, 7168, 256, 8, 8, "normal", "sigmoid"),
    Shape("deepseekv3_fp8", 4096, 7168, 256, 8, 8, "normal", "sigmoid", fp8=True),
    Shape("qwen3_skewed", 16384, 4096, 128, 8, 8, "zipf", "softmax"),
)
CONFIG_BY_NAME = {c.name: c for c in CONFIGS}
ZIPF_S = 1.2


@dataclasses.dataclass
class Workload:
    shape: Shape
    seed: int
    x_bits: np.ndarray               # uint16 [T, H], bf16 bit patterns
    logits: np.ndarray               # float32 [T, E], router logits
    topk_idx: np.ndarray | None = None   # int32 [T, k], filled in by the caller's router
    topk_w: np.ndarray | None = None     # float32 [T, k]

    @property
    def T(self):
        return self.shape.tokens

    @property
    def H(self):
        return self.shape.hidden


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even) via torch's CPU cast; uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _logits(rng, shape: Shape) -> np.ndarray:
    T, E = shape.tokens, shape.experts
    if shape.logits == "uniform":
        return rng.random((T, E), dtype=np.float32)
    if shape.logits == "normal":
        return rng.standard_normal((T, E), dtype=np.float32)
    if shape.logits == "zipf":
        # Popularity p_e proportional to (e+1)^-s in expert-id order (the most
        # skewed placement: the popular experts all sit on virtual rank 0),
        # plus N(0,1) noise on the logits.
        p = (np.arange(1, E + 1, dtype=np.float64) ** -ZIPF_S)
        p /= p.sum()
        base = np.log(p).astype(np.float32)
        return (base[None, :] + rng.standard_normal((T, E), dtype=np.float32)).astype(np.float32)
    raise ValueError(shape.logits)


def make_workload(name_or_index, seed: int | None = None, tokens: int | None = None,
                  hidden: int | None = None) -> Workload:
    """Draw one workload. Draw order: router logits [T,E], then x [T,H]."""
    if isinstance(name_or_index, int):
        shape = CONFIGS[name_or_index]
        index = name_or_index
    else:
        shape = CONFIG_BY_NAME[name_or_index]
        index = CONFIGS.index(shape)
    if tokens is not None or hidden is not None:
        shape = dataclasses.replace(shape, tokens=shape.tokens if tokens is None else tokens,
                                    hidden=shape.hidden if hidden is None else hidden)
    if seed is None:
        seed = 1000 + index
    rng = np.random.default_rng(seed)
    logits = _logits(rng, shape)
    x = rng.standard_normal((shape.tokens, shape.hidden), dtype=np.float32)
    return Workload(shape, seed, bf16_bits_from_f32(x), logits)


def make_expert_outputs(rows: int, hidden: int, seed: int) -> np.ndarray:
    """Independent N(0,1) bf16 rows standing in for expert outputs [rows, H]."""
    rng = np.random.default_rng(seed)
    y = rng.standard_normal((rows, hidden), dtype=np.float32)
    return bf16_bits_from_f32(y)
