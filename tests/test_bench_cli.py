"""bench.py's command-line contract that holds without a GPU: more than one GPU
is refused with a message (the hot path has no cross-GPU step), before any GPU
work."""
from __future__ import annotations

import subprocess
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parent.parent


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""
