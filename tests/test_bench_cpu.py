"""bench.py's command line, without a device: it measures one GPU only, and
the flags that pick one workload's shape are refused for the full run."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode == 2 and "one GPU only" in r.stderr and r.stdout == ""


def test_single_workload_flags_are_refused_for_the_full_run():
    r = _run("--M", "4")
    assert r.returncode == 2 and "one --workload" in r.stderr and r.stdout == ""
