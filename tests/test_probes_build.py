"""The committed probes behind the measured ceilings (HBM streaming in the decode's launch
shapes, LDS read bandwidth) still compile for gfx950 with the flags their summaries give."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.slow
@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
@pytest.mark.parametrize("probe", ["bench_stream_probe.hip", "bench_lds_probe.hip"])
def test_probe_compiles(probe):
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "probe")
        r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-O3", "-Xclang", "-target-feature", "-Xclang",
                            "-packed-fp32-ops", "-o", out, os.path.join(ROOT, probe)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        assert os.path.exists(out)
