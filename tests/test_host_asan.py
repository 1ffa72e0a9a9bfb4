"""The C ABI's host code under AddressSanitizer (CPU only; no kernel is launched).

Builds the library with its host pass instrumented (the GPU code as usual)
into a temporary directory, then runs tests/asan/host_checks.py in a child
Python with the ASan runtime preloaded: configuration and argument checks,
repeated handle creation and destruction, every CU-mask count, and the
no-allocation layout's size checks. Any heap or stack error ASan finds
aborts the child and fails the test. (Leak detection is off: the Python
interpreter itself keeps allocations alive at exit.)
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

from combine_moe_dispatch_02_amd import build as lib_build

HERE = os.path.dirname(os.path.abspath(__file__))


def _asan_runtime():
    cands = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return cands[-1] if cands else None


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc")
def test_host_code_under_address_sanitizer(tmp_path):
    rt = _asan_runtime()
    if rt is None:
        pytest.skip("no clang ASan runtime under /opt/rocm/llvm")
    so = lib_build.build(out=str(tmp_path / "libmoe_ep_asan.so"), host_asan=True)
    syms = subprocess.run(["nm", "-D", so], capture_output=True, text=True).stdout
    assert "__asan_report" in syms, "the host code was not instrumented"
    env = dict(os.environ, LD_PRELOAD=rt,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0:verify_asan_link_order=0")
    res = subprocess.run([sys.executable, os.path.join(HERE, "asan", "host_checks.py"), so],
                         capture_output=True, text=True, timeout=300, env=env)
    print(res.stdout[-2000:], res.stderr[-4000:])
    assert "AddressSanitizer" not in res.stderr
    assert res.returncode == 0
    assert "asan host checks ok" in res.stdout
