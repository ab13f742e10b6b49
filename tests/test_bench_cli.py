"""CPU checks of bench.py's command line (no GPU needed): the one-GPU rule and the
algorithmic counts the roofline objects are built on."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_counts():
    import bench
    # canvas step: 4 * B * Hq * 256 * (L + 256) * D (QK^T and PV, two FLOP per MAC)
    assert bench.step_flops(1, 16, 8192, 128) == 4.0 * 16 * 256 * (8192 + 256) * 128
    # commit: block row i sees L cache rows and i+1 block rows
    assert bench.commit_flops(1, 1, 0, 1) == 4.0 * sum(i + 1 for i in range(256))
    # decode bytes: the cache K and V of the prefix dominate
    b = bench.decode_bytes(32, 8192, 1, 16, 8, 128)
    assert 2 * 32 * 8192 * 8 * 128 * 2 < b < 1.001 * 2 * 32 * 8192 * 8 * 128 * 2
