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


def test_routed_stream_stages_match_the_layer_shapes():
    """The read+write probe is run at each routed stage's own mix: written over
    read bytes is T*k*H / (2*E*H*d) = T*k/(2*E*d) for SwiGLU (h against W1 and
    W3) and T*k/(E*H) for down (y_perm against W2) when every expert has rows;
    at the V3 prefill shape (4096 tokens, top-8, 256 experts, d 7168, H 2048)
    that is 1/112 and 1/16."""
    sys.path.insert(0, ROOT)
    import bench
    from sparse_mixture_experts_51_amd import workloads
    wl = workloads.WORKLOADS["v3_prefill_4096"]
    st = bench.routed_stream_stages(wl, wl.n_experts)
    (r_sw, w_sw, row_sw), (r_dn, w_dn, row_dn) = st["swiglu"], st["down"]
    assert w_sw / r_sw == 1 / 112 and w_dn / r_dn == 1 / 16
    assert (row_sw, row_dn) == (2 * 7168, 2 * 2048)
    # together the two stages read every routed weight once
    assert r_sw + r_dn == 2.0 * 3 * 2048 * 7168 * 256
    # fewer touched experts: reads shrink, writes (one row per routed token) do not
    half = bench.routed_stream_stages(wl, 128)
    assert half["swiglu"][0] == r_sw / 2 and half["swiglu"][1] == w_sw
