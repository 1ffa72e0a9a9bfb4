"""CPU oracle for MoE expert-parallel token dispatch and combine.

TEST INFRASTRUCTURE ONLY. This package is the slow, plainly written reference
that the HIP kernels are checked against. Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import it; the library's own path
never does, and it shares no code, tables or helpers with the HIP sources.

Contents:
  * ``codecs``  -- bf16 and OCP FP8 E4M3 encoders/decoders written from the
    formats' definitions (nearest representable value, ties to even).
  * ``moe``     -- layout (histogram, exclusive scan, stable placement),
    bf16 dispatch, FP8 dispatch with per-128-channel scales, combine, the
    expert-side FP8 dequantisation used by the tests, and the
    rank-deduplicated exchange (rank layout, dispatch with receiver
    metadata, combine of per-rank partial rows), and MXFP8 dispatch (OCP MX
    v1.0: 32-element blocks, E8M0 power-of-two scales, E4M3 elements), and
    the fixed-capacity (decode-time) layout.
  * ``router``  -- top-k expert selection and softmax / sigmoid weights.

Every function is pinned by ``tests/test_oracle_*.py`` against library
routines, closed forms, invariants, brute force on tiny inputs and the
hand-worked fixtures under ``tests/golden/``.
"""
from . import codecs, moe, router  # noqa: F401
from .moe import (layout, dispatch_bf16, dispatch_fp8, combine, dequant_fp8,  # noqa: F401
                  rank_layout, dispatch_ranks, combine_ranks, dispatch_mxfp8, dequant_mxfp8,
                  layout_fixed_capacity)
from .router import route  # noqa: F401
