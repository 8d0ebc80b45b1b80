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


def test_unknown_workload_is_refused():
    r = run_bench("--workload", "no_such_workload")
    assert r.returncode == 2
    assert "unknown workload" in r.stderr
    assert r.stdout == ""


def test_first_timed_step_always_records_events():
    """Events go around the FFN of timed steps 0, N, 2N, ..., so any --steps
    and --warmup give at least one timing (no empty mean, no NaN)."""
    import ast
    src = open(os.path.join(ROOT, "bench.py")).read()
    tree = ast.parse(src)
    step = next(n for n in ast.walk(tree) if isinstance(n, ast.FunctionDef) and n.name == "step")
    text = ast.get_source_segment(src, step)
    assert "timed % args.ffn_events_every == 0" in text
    assert "step(args.warmup + i, i)" in src


def test_training_steps_of_the_normalised_block_are_refused():
    """The RMSNorm of the pre-norm block has no backward here, so training
    steps of that workload are refused before any GPU work."""
    r = run_bench("--workload", "small_block_4096x4", "--with-backward")
    assert r.returncode == 2
    assert "RMSNorm" in r.stderr
    assert r.stdout == ""
