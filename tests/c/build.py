"""Compile tests/c/abi_roundtrip.c as plain C (gcc -x c) against include/moe_ep.h
and the in-tree libmoe_ep.so; the binary lands next to the source."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_roundtrip.c")
BIN = os.path.join(HERE, "abi_roundtrip")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out: str = BIN) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-x", "c",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           SRC, "-L", os.path.join(ROOT, "combine_moe_dispatch_02_amd"), "-lmoe_ep",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../combine_moe_dispatch_02_amd", f"-Wl,-rpath,{ROCM}/lib", "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"gcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    return out


if __name__ == "__main__":
    print(build(sys.argv[1] if len(sys.argv) > 1 else BIN))
