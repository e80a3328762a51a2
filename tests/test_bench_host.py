"""Host-side checks of bench.py that need no GPU: the one-GPU rule and the
algorithmic byte counts behind every reported roofline fraction."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes():
    # packed codes + fp16 scales and mins + fp16 activations (per call)
    assert bench.algorithmic_bytes(25088, 3072, 1) == 40_949_760
    assert bench.algorithmic_bytes(3072, 3072, 1) == 5_019_648
    assert bench.algorithmic_bytes(3072, 8192, 1) == 13_385_728
    assert bench.algorithmic_bytes(25088, 3072, 34) == 41_152_512
    assert bench.algorithmic_bytes(25088, 3072, 256) == 42_516_480


def test_quantize_and_head_bytes():
    n, k = 25088, 3072
    assert bench.quantize_bytes(n, k) == n * k * 4 + n * k // 2 + 4 * n * (k // 128)
    assert bench.quantize_bytes(n, k) == 349_224_960
    assert bench.head_bytes(16384, 3072) == 16384 * 3072 + 2 * 16384 + 2 * 3072
