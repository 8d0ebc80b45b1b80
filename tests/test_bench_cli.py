"""bench.py's command line: the cases it refuses before touching a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_unusable_step_counts_are_refused():
    for args in (("--steps", "0"), ("--warmup", "-1"), ("--ffn-events-every", "0")):
        r = run_bench(*args)
        assert r.returncode == 2, args
        assert r.stdout == "", args
