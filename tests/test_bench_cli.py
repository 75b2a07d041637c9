"""bench.py measures one GPU: any other --gpus value is refused before a workload is built."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("extra", [[], ["--prefill", "64"], ["--copy-calibration"]])
def test_multi_gpu_refused(extra):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", *extra],
                       cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 2, r.stderr[-2000:]
    line = [l for l in r.stdout.splitlines() if l.startswith("{")][-1]
    assert "one GPU" in json.loads(line)["error"]
