"""Compile tests/hip/e4m3_sweep.hip (hipcc, gfx950) into libe4m3_sweep.so next to
the source. It includes the library's E4M3 conversion header, so that the
exhaustive conversion test runs the dispatch kernels' own code."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "e4m3_sweep.hip")
LIB = os.path.join(HERE, "libe4m3_sweep.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out: str = LIB) -> str:
    cmd = [os.path.join(ROCM, "bin", "hipcc"), "--offload-arch=gfx950", "-O3", "-std=c++17",
           "-fPIC", "-shared", "-Wall",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "combine_moe_dispatch_02_amd", "csrc"), "-x", "hip", SRC,
           "-o", out + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1] if len(sys.argv) > 1 else LIB))
