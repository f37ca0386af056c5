"""Host-side accounting of the benchmark (no GPU): the dense and executed
Newton-Schulz flop counts and the multi-GPU refusal."""

import subprocess
import sys
import os

import pytest

HERE = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, HERE)
import bench  # noqa: E402


def test_dense_ns_flops_of_one_matrix():
    # per step: Gram 2 r^2 c, square 2 r^3, B X 2 r^2 c, with r = min side
    r, c = 1024, 4096
    want = 5 * (2 * r * r * c + 2 * r ** 3 + 2 * r * r * c)
    assert bench.ns_flops([(c, r)], 5) == want
    assert bench.ns_flops([(r, c)], 5) == want


def test_executed_ns_flops_counts_upper_tiles_and_padding():
    # 1024 x 4096: 4 x 4 tiles of 256, of which 10 are upper tiles
    up = 10 * 256 * 256
    want = 2 * up * 4096 + 2 * up * 1024 + 2 * 1024 * 1024 * 4096
    assert bench.ns_executed_flops([(1024, 4096)], 1, "bf16") == want
    # 64 x 256 under bf16 runs in one workgroup: every product in full on
    # its own sides (rounded up to 32); under fp32 it pads to one 256 x 256 tile
    assert bench.ns_executed_flops([(256, 64)], 1, "bf16") == 4 * 64 * 64 * 256 + 2 * 64 ** 3
    assert bench.ns_executed_flops([(256, 300)], 1, "bf16") == 4 * 256.0 ** 2 * 512 + 2 * 256.0 ** 3
    # one tile row: symmetric saving is nil, so executed == dense at r = 256
    assert bench.ns_executed_flops([(256, 1024)], 1, "bf16") == bench.ns_flops([(256, 1024)], 1)


def test_executed_ns_flops_of_small_fp32_tiles():
    # fp32 with no matrix above 256 rows: Gram and square over the 36 upper
    # 32 x 32 tiles of the padded 256 x 256 result, the X update in full
    up = 36 * 32 * 32
    want = 2 * up * 1024 + 2 * up * 256 + 2 * 256 * 256 * 1024
    assert bench.ns_executed_flops([(1024, 200)], 1, "fp32") == want
    # beside a larger fp32 matrix they keep the 256 x 256 tiles
    big = bench.ns_executed_flops([(512, 512)], 1, "fp32")
    assert bench.ns_executed_flops([(1024, 200), (512, 512)], 1, "fp32") == \
        bench.ns_flops([(1024, 256)], 1) + big
    # under bf16 only the thin matrices (fewer than 16 rows) run in fp32
    thin = 36 * 32 * 32
    assert bench.ns_executed_flops([(3, 300), (256, 256)], 1, "bf16") == \
        (2 * thin * 512 + 2 * thin * 256 + 2 * 256 * 256 * 512) + 3 * 2 * 256.0 ** 3
    # 33 x 65 under bf16: one workgroup on 64 x 96
    assert bench.ns_executed_flops([(65, 33)], 1, "bf16") == 4 * 64 * 64 * 96 + 2 * 64 ** 3


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(HERE, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode != 0
    assert "one GPU" in (p.stdout + p.stderr) or "1 GPU" in (p.stdout + p.stderr)
