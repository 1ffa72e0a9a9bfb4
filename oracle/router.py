"""Router: top-k expert selection and combine weights (test infrastructure only).

What the pages say: each token activates a small subset, the top-k, of the
experts ("Inside the Nebius + PyTorch DeepSeek V3 recipe", section
"Mixture-of-experts and wide expert parallelism"; DeepSeek V3 picks 8 of 256,
Hybrid-EP news item, opening section). The pages give no scoring or tie rule;
the readings written out here are:
  * selection: the k largest logits of the token, in descending order; equal
    logits go to the lower expert id (a stable descending sort; -0 and +0
    are equal);
  * weights over the k selected experts, computed in fp64 and rounded once to
    fp32:
      "softmax": w_j = exp(l_j) / sum_i exp(l_i);
      "sigmoid": w_j = s_j / sum_i s_i with s = 1 / (1 + exp(-l)), the
      DeepSeek-V3-style gate with no extra scaling factor.
"""
from __future__ import annotations

import numpy as np

__all__ = ["route", "SCORES"]

SCORES = ("softmax", "sigmoid")


def route(logits, k: int, score: str):
    """logits float32 [T, E] -> (topk_idx int32 [T, k], topk_w float32 [T, k])."""
    if score not in SCORES:
        raise ValueError(f"score must be one of {SCORES}")
    L = np.asarray(logits, dtype=np.float32)
    T, E = L.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= number of experts")
    # Stable sort of the negated logits: descending values, lower id first on ties.
    order = np.argsort(-L, axis=1, kind="stable")[:, :k]
    sel = np.take_along_axis(L, order, axis=1).astype(np.float64)
    if score == "softmax":
        z = np.exp(sel - sel[:, :1])          # exp(l_j - l_max): the same ratio, no overflow
    else:
        z = 1.0 / (1.0 + np.exp(-sel))
    w = z / z.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)
