"""bench.py end to end at row counts whose acceptance stage differs from
the default four rows: above eight rows the window's finish stage spans
several workgroups and its workspace carries an arrival counter (a single
layer keeps each run short)."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("rows", [9, 24])
def test_bench_runs_above_eight_rows(rows):
    cmd = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--rows", str(rows), "--layers", "1",
           "--steps", "2", "--warmup", "1", "--no-sweep", "--no-cpu-baseline", "--no-sampling"]
    print("running", " ".join(cmd[2:]), flush=True)
    p = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert p.returncode == 0, p.stderr[-3000:]
    line = json.loads(p.stdout.strip().splitlines()[-1])
    assert line["config"]["rows"] == rows
    assert line["ms_acceptance"] > 0 and line["ms_acceptance_separate_calls"] > 0
