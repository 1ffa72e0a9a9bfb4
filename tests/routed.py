"""Seeded workloads with their routing, for the tests: logits and activations
come from the generator, top-k ids and weights from the oracle's router."""
import dataclasses
import functools

import oracle
import workloads


@functools.lru_cache(maxsize=16)
def _routing(name_or_index, seed, tokens):
    wl = workloads.make_workload(name_or_index, seed=seed, tokens=tokens, hidden=8)
    return oracle.route(wl.logits, wl.shape.topk, wl.shape.weights)


def make_workload(name_or_index, seed=None, tokens=None, hidden=None):
    wl = workloads.make_workload(name_or_index, seed=seed, tokens=tokens, hidden=hidden)
    idx, w = _routing(name_or_index, seed, tokens)
    return dataclasses.replace(wl, topk_idx=idx.copy(), topk_w=w.copy())
