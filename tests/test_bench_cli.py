"""The benchmark's command line on the CPU: it refuses more than one GPU and
bad step counts with a JSON error line and exit status 2, before touching a
device."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("args", [["--gpus", "2"], ["--gpus", "8"], ["--steps", "0"],
                                  ["--warmup", "-1"]])
def test_bench_refuses_unsupported_runs(args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2, r.stderr[-2000:]
    line = [l for l in r.stdout.splitlines() if l.startswith("{")][-1]
    assert "error" in json.loads(line)
