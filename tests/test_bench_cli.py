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


def test_counted_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    """A counter file is reported only while its hash matches the kernel source it
    was taken on; a missing file or another hash gives null traffic."""
    import bench
    tag = "canvas_attn_l128k"
    good = "\n".join(["# counters", f"kernel_source_hash: {bench.kernel_source_hash('long')}",
                      "traffic_bytes_per_launch: 547886180"]) + "\n"
    stale = good.replace(bench.kernel_source_hash("long"), "0000000000000000")
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("long") is None
    (prof / f"{tag}_traffic.txt").write_text(good)
    assert bench.measured_traffic("long") == 547886180
    (prof / f"{tag}_traffic.txt").write_text(stale)
    assert bench.measured_traffic("long") is None
