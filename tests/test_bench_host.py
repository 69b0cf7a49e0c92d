"""Host-side checks of bench.py (no GPU): the algorithmic bytes and flops that
the roofline fractions divide by, against the per-step figures derived by hand
for each workload (360 B per packed C4R4 token, 232 B per C2R4 token, 1152 B per
protected token, 2180 B of query / output / lse per (sequence, head), 4 B per
page-table entry; 2 (576 + 512) flops per token and head), and the one-GPU
refusal."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_bytes_of_the_workloads():
    # tiny: 1024 tokens, 132 protected
    assert bench.algorithmic_bytes([1024], 16, 4) == 892 * 360 + 132 * 1152 + 16 * 4 + 16 * 2180
    assert bench.algorithmic_bytes([1024], 16, 4) == 508_128
    assert bench.algorithmic_bytes([32768] * 8, 16, 4) == 95_503_616
    assert bench.algorithmic_bytes([8192] * 32, 128, 4) == 106_662_912
    assert bench.algorithmic_bytes([131072] * 8, 16, 2) == 244_585_728
    # every token protected below 133 tokens; an empty sequence costs only its rows
    assert bench.algorithmic_bytes([100], 16, 4) == 100 * 1152 + 2 * 4 + 16 * 2180
    assert bench.algorithmic_bytes([0], 16, 4) == 16 * 2180


def test_algorithmic_flops_and_bf16_bytes():
    assert bench.algorithmic_flops([1024], 16) == 35_651_584
    assert bench.algorithmic_flops([32768] * 8, 16) == 9_126_805_504
    assert bench.bf16_algorithmic_bytes([32768] * 8, 16) == 8 * 32768 * 1152 + 8 * 512 * 4 + 128 * 2180


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2
    assert "one GPU" in r.stdout
