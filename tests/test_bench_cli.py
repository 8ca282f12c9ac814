"""bench.py's command-line contract on the host (no GPU is touched): more than
one GPU is refused with a message and a non-zero status, and the options that
select workloads and sections parse."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr) and r.stdout.count("{") == 0


def test_help_lists_the_workload_options():
    r = _run("--help")
    assert r.returncode == 0
    for opt in ("--workload", "--bwd-workload", "--partial-shift", "--mask-alpha-ns",
                "--rope-base", "--block-lengths", "--sweep", "--steps", "--warmup",
                "--c4-steps", "--sweep-steps"):
        assert opt in r.stdout, opt
