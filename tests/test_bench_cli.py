"""bench.py's command line on the CPU: the library runs on one GPU, so a
request for more exits at once with a message and status 2, before any GPU
or library work."""

import pathlib
import subprocess
import sys

ROOT = pathlib.Path(__file__).resolve().parent.parent


def test_bench_refuses_more_than_one_gpu():
    run = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert run.returncode == 2
    assert "one GPU only" in run.stderr
    assert run.stdout == ""
