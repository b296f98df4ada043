"""bench.py's contract checks that need no GPU: it refuses more than one GPU with a
message, and its CPU baseline (the oracle timed on a bounded sample) reports the fields
the JSON line carries."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_cpu_baseline_fields():
    sys.path.insert(0, ROOT)
    import bench

    cb = bench.cpu_baseline(sample_tokens=256)
    for key in ("value", "unit", "cores", "kind", "sample", "affinity_cores"):
        assert key in cb, key
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s" and cb["value"] > 0
    assert cb["cores"] >= 1 and cb["affinity_cores"] >= 1
    assert "256 of 32768 tokens" in cb["sample"]


def test_traffic_digest_covers_the_prefill_kernel_sources():
    sys.path.insert(0, ROOT)
    import bench

    files = bench.KERNEL_SOURCES["swa_ring_kernel"]
    assert "prefill_mfma.hip" in files and "mfma_tile.h" in files
    assert len(bench.kernel_source_digest("swa_ring_kernel")) == 16
