"""Host-side checks of bench.py (CPU): the algorithmic byte counts its GB/s
figures divide by, the source-hash gate on the committed traffic record, the
rotation rule for cold inputs, and the refusal of more than one GPU.

The byte counts are pinned to values worked out by hand from the operations'
definitions (each input read once, each output written once, index arrays
counted): for dispatch x is 2TH bytes and every one of the S = T*k rows 2H
(bf16) or H codes plus 4H/128 scale bytes (FP8), plus a 4-byte position per
slot; combine reads S rows of 2H bytes and a position and weight per slot
and writes 2TH; the layout reads an id and writes a position and a row
source per slot.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


# (T, H, k): layout, bf16 dispatch, FP8 dispatch, combine bytes
SHAPES = {
    "deepseekv3": ((4096, 7168, 8), (393_216, 528_613_376, 301_072_384, 528_744_448)),
    "deepseek16b": ((4096, 2048, 6), (294_912, 117_538_816, 68_780_032, 117_637_120)),
    "qwen3_skewed": ((16384, 4096, 8), (1_572_864, 1_208_483_840, 688_390_144, 1_209_008_128)),
}


@pytest.mark.parametrize("name", sorted(SHAPES))
def test_op_bytes_match_the_definitions(name):
    (T, H, k), want = SHAPES[name]
    got = bench.op_bytes(T, H, k)
    assert (got["layout"], got["dispatch_bf16"], got["dispatch_fp8"], got["combine"]) == want


def test_mxfp8_bytes():
    # x once, S rows of H codes and H/32 E8M0 bytes, a position per slot
    assert bench.mxfp8_bytes(4096, 7168, 8) == 58_720_256 + 234_881_024 + 7_340_032 + 131_072


def test_copies_for_spans_the_cold_footprint():
    assert bench.copies_for(1) == bench.COLD_FOOTPRINT
    assert bench.copies_for(bench.COLD_FOOTPRINT) == 3
    assert bench.copies_for(bench.COLD_FOOTPRINT // 3 + 1) == 3
    n = bench.copies_for(58_720_256)
    assert n * 58_720_256 >= bench.COLD_FOOTPRINT and (n - 1) * 58_720_256 < bench.COLD_FOOTPRINT


def _record(sources, digest, traffic):
    return {"kernels": {bench.KERNEL_OF_OP["dispatch_bf16"]: {
        "sources": sources, "sources_sha256": digest, "traffic_bytes": traffic}}}


def test_traffic_record_is_gated_on_the_kernel_sources(tmp_path, monkeypatch):
    sources = ["combine_moe_dispatch_02_amd/csrc/dispatch.hip", "include/moe_ep.h"]
    good = bench.sources_sha256(sources)
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    path.write_text(json.dumps(_record(sources, good, 123_456)))
    assert bench.measured_traffic("dispatch_bf16") == 123_456
    path.write_text(json.dumps(_record(sources, "0" * 64, 123_456)))
    assert bench.measured_traffic("dispatch_bf16") is None        # a source changed
    path.write_text("{}")
    assert bench.measured_traffic("dispatch_bf16") is None        # no record for the kernel
    os.remove(path)
    assert bench.measured_traffic("dispatch_bf16") is None        # no file


def test_sources_hash_depends_on_content_and_order():
    a = "combine_moe_dispatch_02_amd/csrc/dispatch.hip"
    b = "combine_moe_dispatch_02_amd/csrc/combine.hip"
    assert bench.sources_sha256([a]) != bench.sources_sha256([b])
    assert bench.sources_sha256([a, b]) != bench.sources_sha256([b, a])
    assert bench.sources_sha256([a, b]) == bench.sources_sha256([a, b])


def test_committed_record_names_the_step_kernels():
    with open(bench.TRAFFIC_FILE) as f:
        kernels = json.load(f)["kernels"]
    for op, kernel in bench.KERNEL_OF_OP.items():
        assert kernel in kernels, op
        assert kernels[kernel]["sources"], op


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "--gpus 2 is not supported" in (r.stdout + r.stderr)
