"""Exhaustive GPU check of the fp32 -> E4M3 conversion of the FP8 and MXFP8
dispatch kernels (clamp to +-448, then the gfx950 conversion instruction,
round to nearest even), over every finite fp32 bit pattern; and of the FP8
kernels' quotient x / scale, over every (amax, x) pair of bf16 values.

The FP8 dispatch quantises x / scale in fp32 and converts that quotient
("MoE / Hybrid-EP Validation", "FP8 dispatch restriction": dispatch carries
FP8). The parity tests cover the quotients real activations produce; this
test covers the conversion step itself for every fp32 input it could be
handed. tests/hip/e4m3_sweep.hip runs the kernels' own conversion code
(csrc/e4m3.h) over the patterns; the reference is torch's CPU
float8_e4m3fn cast of the value clamped to +-448 (torch's cast alone turns
magnitudes above 464 into NaN, the oracle's encoder saturates), which the
CPU tests pin to the oracle's encoder (tests/test_oracle_codecs.py); a
sample of every chunk is also compared with the oracle's encoder directly.
"""
import ctypes
import os
import time

import numpy as np
import pytest
import torch

from oracle.codecs import e4m3_encode

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "hip", "libe4m3_sweep.so")
CHUNK = 1 << 26          # bit patterns per GPU call (64 chunks cover all 2^32)
ORACLE_SAMPLE = 1 << 14  # patterns per chunk also checked against the oracle's encoder


def _lib():
    if not os.path.exists(LIB):   # normally built by __graft_entry__.build()
        import importlib.util
        spec = importlib.util.spec_from_file_location("moe_e4m3_sweep_build",
                                                      os.path.join(HERE, "hip", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build(LIB)
    lib = ctypes.CDLL(LIB)
    lib.e4m3_sweep.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p]
    lib.e4m3_sweep.restype = ctypes.c_int
    lib.e4m3_quotient_sweep.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p]
    lib.e4m3_quotient_sweep.restype = ctypes.c_int
    return lib


def test_fp8_quotient_every_bf16_pair():
    """The FP8 kernels form x / scale with e4m3_quotient (a reciprocal per
    scale and Markstein's fma corrections) instead of an IEEE division; its
    E4M3 code must be the IEEE quotient's for every input a block can hold:
    every positive finite bf16 amax (scale = amax / 448) against every bf16 x
    with |x| <= amax, and NaN x (2,139,029,504 pairs, about 1.76e9 of them on
    the fast path)."""
    lib = _lib()
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    counts = torch.zeros(3, dtype=torch.int32, device=dev)
    example = torch.zeros(1, dtype=torch.int32, device=dev)
    n_all, per_call = 0x7F7F, 4096
    t0 = time.time()
    for first in range(1, n_all + 1, per_call):
        n = min(per_call, n_all + 1 - first)
        rc = lib.e4m3_quotient_sweep(first, n, ctypes.c_void_p(counts.data_ptr()),
                                     ctypes.c_void_p(example.data_ptr()),
                                     ctypes.c_void_p(stream.cuda_stream))
        assert rc == 0, f"e4m3_quotient_sweep returned {rc} at amax 0x{first:04x}"
    torch.cuda.synchronize()
    c = counts.cpu().numpy().view(np.uint32)
    ex = int(example.cpu().numpy().view(np.uint32)[0])
    print(f"[quotient sweep] {time.time() - t0:.1f} s: {c[0]} in-domain and {c[1]} out-of-domain "
          f"disagreements, {c[2]} pairs on the fast path", flush=True)
    assert c[0] == 0, f"amax 0x{ex >> 16:04x}, x 0x{ex & 0xFFFF:04x}: codes differ"
    # the fast path covered every scale of 2^-90 or more (host count, IEEE fp32 division)
    amax = (np.arange(1, n_all + 1, dtype=np.uint32) << 16).view(np.float32)
    scale = amax / np.float32(448.0)
    assert int(c[2]) == int(np.count_nonzero(scale >= np.float32(2.0 ** -90))) * 65536


def test_e4m3_conversion_every_finite_fp32():
    lib = _lib()
    dev = torch.device("cuda", 0)
    stream = torch.cuda.current_stream(dev)
    buf = torch.empty(CHUNK, dtype=torch.uint8, device=dev)
    rng = np.random.default_rng(0)
    checked = 0
    t0 = time.time()
    for c in range((1 << 32) // CHUNK):
        first = c * CHUNK
        rc = lib.e4m3_sweep(first, CHUNK, ctypes.c_void_p(buf.data_ptr()),
                            ctypes.c_void_p(stream.cuda_stream))
        assert rc == 0, f"e4m3_sweep returned {rc} at chunk {c}"
        got = buf.cpu().numpy()
        bits = np.arange(first, first + CHUNK, dtype=np.uint64).astype(np.uint32)
        vals = bits.view(np.float32)
        finite = np.isfinite(vals)
        ref = (torch.from_numpy(vals).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
               .view(torch.uint8).numpy())
        bad = np.flatnonzero(finite & (got != ref))
        assert bad.size == 0, (
            f"{bad.size} mismatches in chunk {c}; first patterns "
            f"{[hex(int(bits[i])) for i in bad[:4]]}: gpu {[hex(int(got[i])) for i in bad[:4]]}, "
            f"reference {[hex(int(ref[i])) for i in bad[:4]]}")
        pick = rng.choice(np.flatnonzero(finite), size=min(ORACLE_SAMPLE, int(finite.sum())),
                          replace=False) if finite.any() else np.zeros(0, dtype=np.int64)
        assert np.array_equal(got[pick], e4m3_encode(vals[pick])), f"oracle sample, chunk {c}"
        checked += int(finite.sum())
    print(f"[e4m3 sweep] {checked} finite fp32 patterns, 0 mismatches, {time.time() - t0:.1f} s",
          flush=True)
    assert checked == (1 << 32) - (1 << 24)   # every pattern but the 2^24 infinities and NaNs
