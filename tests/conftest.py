import json
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def hexint(s):
    return int(s, 16)


def combine_tolerance(ref_bits, mag, k):
    """Gate used by the GPU parity tests: |got - ref| <= 1e-2 |ref| + 2 (k+1) 2^-24 M + 2^-133.

    1e-2 is the required relative error. The second term bounds what any fp32
    recursive summation of k products can lose to cancellation (M = sum |w y|),
    doubled to cover the final rounding of both sides; the last term covers
    bf16 subnormal spacing.
    """
    ref = (np.asarray(ref_bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return 1e-2 * np.abs(ref) + 2 * (k + 1) * 2.0 ** -24 * mag + 2.0 ** -133
