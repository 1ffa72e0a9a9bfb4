"""Host-side pins of the blocked bf16 dispatch's sizing (CPU only).

tests/host/block_rule_check.cpp includes the library's internal header and
checks, without any GPU call: the multiply-high division the kernel uses
against integer division (every divisor up to 4096 and large ones, on
small, random, boundary and near-multiple numerators below 2^31); and, over
a sweep of T, k and hidden, that the chosen block is a power of two of at
most chunks / 8 chunks and 4 MiB of x, that an XCD slot's x stays within
the prefetch limit, that the lists fit the workspace, that a block's slots
span at most bs / k + 2 tokens, and that the kernel's item indices stay
below 2^31; plus the choice at the three measured shapes.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _hipcc():
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.skipif(_hipcc() is None, reason="needs hipcc")
def test_block_rule_and_fast_division(tmp_path):
    exe = str(tmp_path / "block_rule_check")
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O2", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "combine_moe_dispatch_02_amd", "csrc"),
           os.path.join(HERE, "host", "block_rule_check.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "block rule ok" in res.stdout
