"""The plain-C program tests/c/abi_roundtrip.c, built by __graft_entry__.build(),
run on the GPU: layout, dispatch and combine through the C ABI alone."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "abi_roundtrip")


def test_c_abi_roundtrip():
    if not os.path.exists(BIN):   # normally built by __graft_entry__.build(); gcc only, no GPU
        import importlib.util
        spec = importlib.util.spec_from_file_location("moe_c_abi_build",
                                                      os.path.join(os.path.dirname(BIN), "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build(BIN)
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, res.stderr
    assert "abi_roundtrip ok" in res.stdout
