"""Host check of the FP8 kernels' quotient x / scale (csrc/e4m3.h
e4m3_quotient, Markstein's correction from a rounded reciprocal) against the
host's IEEE division; the exhaustive comparison over every bf16 (amax, x)
pair runs on the GPU (tests/test_gpu_e4m3_sweep.py).

tests/host/quotient_check.cpp includes the header the kernels use and is
built for the host with hipcc (its device pass compiles the same function
for gfx950, unused)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.skipif(_hipcc() is None, reason="needs hipcc")
def test_fp8_quotient_matches_ieee_division(tmp_path):
    exe = str(tmp_path / "quotient_check")
    cmd = [_hipcc(), "--offload-arch=gfx950", "-O2", "-std=c++17",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "combine_moe_dispatch_02_amd", "csrc"),
           os.path.join(HERE, "host", "quotient_check.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
