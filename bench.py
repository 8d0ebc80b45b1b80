"""Benchmark of the DeepSeekMoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch: for every layer of
the workload, moe_route -> moe_permute -> moe_grouped_ffn -> moe_combine
(the combine also adds the residual stream of stacked layers; pre-norm block
workloads run moe_rmsnorm first and route the normalised rows), then
moe_update_bias for every layer.  Inputs are seeded synthetic tensors already
resident in HBM before the timed region.  Prints ONE JSON line.

The default workload is the DeepSeek-V3-shaped prefill layer (4096 tokens,
d_model 7168, 256 routed experts top-8 plus one shared expert, expert hidden
2048); the mini-model and decode workloads are behind --workload.

value = tokens x layers / second (each token counted once per MoE layer
forward).  The roofline object covers the dominant kernel group -- the
grouped expert GEMMs of moe_grouped_ffn -- timed live with HIP events on the
stream they are launched on, around one layer's call in the first timed step
and every fifth one after it (layers in turn; an event record costs a few
microseconds of stream time).  moe_update_bias is timed the same way in those
steps and reported on its own.  By default 20 warm-up steps and 100 timed
steps: the clocks settle within the warm-up.

Workloads of one batch (the prefill and decode layers, which stand for
inference) route every step with the same, frozen bias, so each step does
the same work; the bias update still runs every step, into a training copy
of the bias that routing does not read.  Multi-step training workloads (the
stacked mini layers) route with the live bias.

cpu_baseline times the CPU oracle on a bounded token sample of the same
workload, on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd tokens/sec (1 MI355X); % bf16 MFMA peak / % HBM peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target wall time of the CPU oracle sample")
    ap.add_argument("--ffn-events-every", type=int, default=5,
                    help="time one layer's moe_grouped_ffn with HIP events in every N-th timed step")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain device copy of 1 GiB (counter calibration)")
    ap.add_argument("--with-backward", action="store_true",
                    help="also time training steps (forward, backward of every layer, bias "
                         "updates) and report them as a 'train' object")
    return ap.parse_args()


def time_training(args, wl, shape, params, xs, stream):
    """Training steps: every layer's forward (x_perm gathered), then the
    backward of every layer from the last to the first with a seeded upstream
    gradient (stacked layers pass the residual's gradient on), then the bias
    updates.  HIP events around one layer's moe_grouped_ffn_backward per
    N-th step give the backward expert GEMMs' rate."""
    import numpy as np
    import torch

    from sparse_mixture_experts_51_amd import moe, workloads

    L = wl.layers
    dev = "cuda:0"
    stacked = L > 1
    bufs = [moe.alloc_buffers(shape, dev, x_perm=True) for _ in range(L)]
    grads = [moe.alloc_backward(shape, dev) for _ in range(L)]
    dtop = workloads.normal((wl.tokens, wl.d_model), 1.0, 99991, dev, torch.bfloat16)
    ev = []
    n_x = len(xs)

    def step(i, timed):
        x = xs[i % n_x]
        inputs = []
        for l in range(L):
            inputs.append(x)
            moe.layer_forward(shape, x, params[l], bufs[l], residual=x if stacked else None,
                              use_x_perm=True, stream=stream)
            x = bufs[l]["out"]
        dout = dtop
        for l in reversed(range(L)):
            b, g, p = bufs[l], grads[l], params[l]
            ws = g["workspace"]
            moe.moe_combine_backward(shape, dout, b["y_perm"], b["topk_gate"], b["pos"],
                                     g["dy_perm"], g["dgate"], stream)
            timed_l = timed is not None and timed % args.ffn_events_every == 0 and \
                l == (timed // args.ffn_events_every) % L
            if timed_l:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            moe.moe_grouped_ffn_backward(shape, inputs[l], b["x_perm"], b["offsets"], p["w1"],
                                         p["w3"], p["w2"], p.get("ws1"), p.get("ws3"), p.get("ws2"),
                                         g["dy_perm"], dout if shape.shared_hidden else None,
                                         g["dx_perm"], g["dx_shared"], g["dw1"], g["dw3"],
                                         g["dw2"], g["dws1"], g["dws3"], g["dws2"], ws, stream)
            if timed_l:
                e1.record(stream)
                ev.append((e0, e1))
            moe.moe_route_backward(shape, inputs[l], p["w_router"], b["topk_idx"], b["topk_gate"],
                                   g["dgate"], 1e-4, g["dx_perm"], g["dx_shared"], b["pos"],
                                   dout if stacked else None, g["dx"], g["dw_router"], ws, stream)
            dout = g["dx"]
        for l in range(L):
            moe.moe_update_bias(shape, bufs[l]["counts"], params[l]["bias"], 1e-3, stream)

    for i in range(args.warmup):
        step(i, None)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i, i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    bwd_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    d, H, Hs, T, k = wl.d_model, wl.hidden, wl.shared_hidden, wl.tokens, wl.top_k
    rows_h = T * k * H + T * Hs
    algo = 12.0 * d * rows_h    # dgrad 6 d H + wgrad 6 d H per row
    executed = 16.0 * d * rows_h  # plus the recompute of x W1^T, x W3^T
    return {"ms_per_step": ms, "tokens_per_s": T * L / (ms * 1e-3),
            "value_counts": "tokens x layers per second of forward + backward + bias update",
            "backward_ffn_ms_per_launch": bwd_ms,
            "backward_ffn_algorithmic_flop": algo, "backward_ffn_executed_flop": executed,
            "backward_ffn_tflops": algo / (bwd_ms * 1e-3) / 1e12,
            "backward_ffn_frac": algo / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "backward_ffn_executed_frac": executed / (bwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "kernel": "moe_grouped_ffn_backward = the five grouped GEMMs of the routed experts "
                      "and of the shared expert"}


def hbm_read_probe():
    """Achievable HBM read rate over 8 GiB, best of four passes, GB/s, for each
    probe of libmoe_probe.so: moe_probe_hbm_read (LDS DMA, the streamed
    weights' pattern) and moe_probe_hbm_read_nt (non-temporal register loads,
    the register path's pattern)."""
    import ctypes

    import torch

    from sparse_mixture_experts_51_amd import build as _build

    if not os.path.exists(_build.PROBE_LIB):
        raise SystemExit(f"{_build.PROBE_LIB} is missing: run the build first")
    P = ctypes.CDLL(_build.PROBE_LIB)
    nbytes = 8 << 30
    buf = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda:0")
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    out = {}
    for key, name in (("dma", "moe_probe_hbm_read"), ("nt", "moe_probe_hbm_read_nt")):
        fn = getattr(P, name)
        fn.restype = ctypes.c_int
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
        best = 0.0
        for _ in range(4):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if fn(buf.data_ptr(), nbytes, sink.data_ptr(), stream.cuda_stream) != 0:
                raise RuntimeError(f"{name} failed")
            e1.record(stream)
            torch.cuda.synchronize()
            best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        out[key] = best
    del buf, sink
    return out


def hbm_stream_probe(stages):
    """Achievable HBM read rate (GB/s) of a weight stream whose units write
    output as they go: moe_probe_hbm_read_write over about 8 GiB, best of four
    passes, once per entry of `stages`, name -> (bytes written per byte read,
    weight row bytes).  Returns name -> (written per read as run, GB/s)."""
    import ctypes

    import torch

    from sparse_mixture_experts_51_amd import build as _build

    P = ctypes.CDLL(_build.PROBE_LIB)
    fn = P.moe_probe_hbm_read_write
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                   ctypes.c_void_p, ctypes.c_void_p]
    cap = 8 << 30
    buf = torch.ones(cap // 2, dtype=torch.bfloat16, device="cuda:0")
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    rates = {}
    for key, (ratio, row) in stages.items():
        piece = 256 * row
        nbytes = cap // piece * piece
        per = min(piece, max(16, int(round(ratio * piece / 16)) * 16))
        out = torch.empty(nbytes // piece * per // 4, dtype=torch.int32, device="cuda:0")
        best = 0.0
        for _ in range(4):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if fn(buf.data_ptr(), nbytes, row, out.data_ptr(), per, sink.data_ptr(), stream.cuda_stream) != 0:
                raise RuntimeError("moe_probe_hbm_read_write failed")
            e1.record(stream)
            torch.cuda.synchronize()
            best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        rates[key] = (per / piece, best)
        del out
    del buf, sink
    return rates


def routed_stream_stages(wl, touched):
    """Per routed stage of moe_grouped_ffn: (weight bytes read, output bytes
    written, weight row bytes).  SwiGLU reads W1 and W3 of the touched
    experts (rows of d) and writes h (T*k rows of H); down reads W2 (rows of
    H) and writes y_perm (T*k rows of d); bf16 throughout."""
    d, H, T, k = wl.d_model, wl.hidden, wl.tokens, wl.top_k
    return {"swiglu": (4.0 * H * d * touched, 2.0 * T * k * H, 2 * d),
            "down": (2.0 * H * d * touched, 2.0 * T * k * d, 2 * H)}


def ffn_algorithmic(wl, counts_per_layer):
    """Algorithmic FLOPs and HBM bytes of one moe_grouped_ffn call per layer:
    FLOPs = 6*d*H per routed row + 6*d*Hs per shared row; bytes = weights of
    the experts that received rows + shared weights + x read once + y_perm and
    y_shared written once (bf16)."""
    d, H, Hs, T, k = wl.d_model, wl.hidden, wl.shared_hidden, wl.tokens, wl.top_k
    flops = 6.0 * d * H * T * k + 6.0 * d * Hs * T
    out = []
    for counts in counts_per_layer:
        touched = int((counts > 0).sum())
        byts = 2.0 * (3 * H * d * touched + 3 * Hs * d + T * d + T * k * d + (T * d if Hs else 0))
        out.append((flops, byts))
    return out


def cpu_model() -> str:
    """The host CPU's model name (first "model name" line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, target_s: float, params_dev=None, x_dev=None):
    """The CPU oracle, as it stands, on a bounded sample of the workload.

    Mini shapes: whole layer passes over all tokens (layer i % L of step
    i // L) until the timed oracle work reaches target_s.  V3 shapes (22.5 GB
    of experts): the first n tokens are routed on the host, only the experts
    they chose are copied to the host (from the device copies the GPU path
    uses: the same seeded draws), and the oracle's expert FFN and combine run
    for them.  Copies and weight draws are outside the timed part.  Threads:
    the CPUs this process may use, capped at 16 (one GPU's share of a GPU
    host)."""
    import numpy as np
    import torch

    import oracle
    from sparse_mixture_experts_51_amd import workloads

    threads = oracle.default_threads()
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count() or 1
    host = {"cores": threads, "cpu_model": cpu_model(), "cpus_available": affinity}
    if wl.n_experts * wl.hidden * wl.d_model * 6 <= (1 << 31):
        hp = {}
        done, dt = 0, 0.0
        while dt < target_s and done < wl.layers * wl.steps:
            l, st = done % wl.layers, done // wl.layers
            if l not in hp:
                p = workloads.layer_params(wl, l, "cpu")
                hp[l] = {k: (oracle.as_bf16_bits(v) if v.dtype == torch.bfloat16 else v.numpy())
                         for k, v in p.items()}
            xb = oracle.as_bf16_bits(workloads.tokens(wl, st, "cpu"))
            t0 = time.perf_counter()
            if wl.norm:
                oracle.block(xb, hp[l], wl.top_k, seq_len=wl.seq_len, nthreads=threads)
            else:
                oracle.layer(xb, hp[l], wl.top_k, seq_len=wl.seq_len, nthreads=threads)
            dt += time.perf_counter() - t0
            done += 1
        return {"value": done * wl.tokens / dt, "unit": "tokens/s", **host,
                "kind": "oracle",
                "sample": f"{done} layer passes over all {wl.tokens} tokens of {wl.name} ("
                          f"{'RMSNorm, ' if wl.norm else ''}route, balance statistic, permute, "
                          f"grouped FFN, combine), fp64 oracle, "
                          f"{dt:.1f} s on {threads} threads; counts tokens x layers per second"}

    import concurrent.futures as cf
    if params_dev is None:
        params_dev = workloads.layer_params(wl, 0, "cpu")
    xb = oracle.as_bf16_bits(workloads.tokens(wl, 0, "cpu") if x_dev is None else x_dev)
    w_r = params_dev["w_router"].cpu().numpy()
    b = params_dev["bias"].cpu().numpy()
    sh = {k: oracle.as_bf16_bits(params_dev[k]) for k in ("ws1", "ws3", "ws2") if k in params_dev}
    cache = {}

    def one_pass(n):
        r = oracle.route(xb[:n], w_r, b, wl.top_k, threads)
        jobs = [(t, j) for t in range(n) for j in range(wl.top_k)]
        with cf.ThreadPoolExecutor(threads) as ex:
            ys = list(ex.map(lambda tj: oracle.expert_ffn(xb[tj[0]], *cache[r["idx"][tj]]), jobs))
            ysh = list(ex.map(lambda t: oracle.expert_ffn(xb[t], sh["ws1"], sh["ws3"], sh["ws2"]),
                              range(n)))
        pos = np.arange(n * wl.top_k, dtype=np.int32).reshape(n, wl.top_k)
        oracle.combine(np.stack(ys), np.stack(ysh), r["gate"], r["idx"], pos)

    # double the token count until one pass takes half the target; with all
    # tokens in the sample, repeat whole passes until then
    n, passes, dt = 4, 1, 0.0
    while True:
        r = oracle.route(xb[:n], w_r, b, wl.top_k, threads)
        for e in np.unique(r["idx"]):
            if e not in cache:
                cache[e] = tuple(oracle.as_bf16_bits(params_dev[k][int(e)]) for k in ("w1", "w3", "w2"))
        t0 = time.perf_counter()
        one_pass(n)
        dt = time.perf_counter() - t0
        if dt >= target_s / 2:
            break
        if n >= wl.tokens:
            while dt < target_s / 2:
                t0 = time.perf_counter()
                one_pass(n)
                dt += time.perf_counter() - t0
                passes += 1
            break
        n = min(wl.tokens, n * 2)
    what = f"first {n} of {wl.tokens} tokens" if n < wl.tokens else f"all {n} tokens, {passes} passes,"
    return {"value": n * passes / dt, "unit": "tokens/s", **host, "kind": "oracle",
            "sample": f"{what} of {wl.name}: routed on the host, then expert FFN of their "
                      f"{wl.top_k} chosen experts plus the shared expert and the combine, fp64 "
                      f"oracle, {dt:.1f} s on {threads} threads"}


MLA_METRIC = "MLA attention tokens/sec (1 MI355X); % bf16 MFMA peak / % HBM peak"


def mla_algorithmic(wl):
    """FLOPs and HBM bytes of one MLA call by the definitions: the three
    projections and the decompression (prefill) as matrix products, the
    attention's scores and weighted sums; bytes = activations in and out,
    weights, cache entries written and (decode) the cached rows read."""
    d, H, dc, dn, dr, dv = wl.d_model, wl.n_heads, wl.d_latent, wl.d_nope, wl.d_rope, wl.d_v
    qw = dn + dr
    T = wl.tokens
    proj = 2.0 * T * d * (H * qw + dc + dr)
    outp = 2.0 * T * H * dv * d
    wbytes = 2.0 * (H * qw * d + (dc + dr) * d + H * (dn + dv) * dc + d * H * dv)
    if wl.decode:
        n = wl.seq_len + 1  # keys per new token
        attn = 2.0 * wl.batch * H * (dn * dc + n * (dc + dr) + n * dc + dv * dc)
        flops = proj + attn + outp
        byts = 2.0 * wl.batch * (2 * d + (dc + dr) * (n + 1)) + wbytes
    else:
        pairs = wl.batch * wl.seq_len * (wl.seq_len + 1) / 2.0  # causal (query, key) pairs
        attn = 2.0 * H * pairs * (qw + dv)
        flops = proj + 2.0 * T * dc * H * (dn + dv) + attn + outp
        byts = 2.0 * T * (2 * d + dc + dr) + wbytes
    return flops, byts


def mla_cpu_baseline(wl, target_s, x, params):
    """The MLA oracle on whole sequences of the workload (prefill) or on
    sequences' decode steps (with their cache), until about target_s."""
    import numpy as np

    import oracle
    threads = oracle.default_threads()
    hp = {k: oracle.as_bf16_bits(v) for k, v in params.items()}
    xb = oracle.as_bf16_bits(x)
    done, dt = 0, 0.0
    if wl.decode:
        ckv = np.zeros((threads, wl.max_len, wl.d_latent))
        ckr = np.zeros((threads, wl.max_len, wl.d_rope))
        while dt < target_s and done < 64 * wl.batch:
            t0 = time.perf_counter()
            oracle.mla_decode(xb[:threads], hp, wl.n_heads, np.full(threads, wl.seq_len), ckv, ckr,
                              nthreads=threads)
            dt += time.perf_counter() - t0
            done += threads
        what = (f"{done} decode steps at position {wl.seq_len} ({threads} sequences per call, "
                f"zero caches: the same arithmetic)")
    else:
        S = wl.seq_len
        while dt < target_s and done < wl.batch:
            n = min(threads, wl.batch - done)
            t0 = time.perf_counter()
            oracle.mla_prefill(xb[done * S:(done + n) * S], hp, wl.n_heads, n, S, wl.max_len,
                               nthreads=threads)
            dt += time.perf_counter() - t0
            done += n
        done *= S
        what = f"{done // S} whole sequences of {S} tokens"
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count() or 1
    return {"value": done / dt, "unit": "tokens/s", "cores": threads, "cpu_model": cpu_model(),
            "cpus_available": affinity, "kind": "oracle",
            "sample": f"{what} of {wl.name}, fp64 oracle with explicit decompression, "
                      f"{dt:.1f} s on {threads} threads"}


def run_mla(args, name):
    """MLA attention workloads: a step is one mla_prefill (all sequences of
    the batch) or one mla_decode step of every sequence (the same position
    each step, so every step does the same work); each call timed with HIP
    events on its stream."""
    import numpy as np
    import torch

    from sparse_mixture_experts_51_amd import moe, workloads

    wl = workloads.MLA_WORKLOADS[name]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    moe.load()
    params = workloads.mla_params(wl, 0, dev)
    shape = moe.MlaShape(wl.batch, 0 if wl.decode else wl.seq_len, wl.max_len, wl.d_model,
                         wl.n_heads, wl.d_latent, wl.d_nope, wl.d_rope, wl.d_v)
    buf = moe.alloc_mla(shape, dev, decode=wl.decode)
    stream = torch.cuda.current_stream()
    if wl.decode:
        # the caches hold seq_len tokens of every sequence
        pshape = moe.MlaShape(wl.batch, wl.seq_len, wl.max_len, wl.d_model, wl.n_heads,
                              wl.d_latent, wl.d_nope, wl.d_rope, wl.d_v)
        pbuf = moe.alloc_mla(pshape, dev)
        px = workloads.mla_tokens(wl, wl.batch * wl.seq_len, 0, dev)
        moe.mla_prefill(pshape, px, params, buf["cache_kv"], buf["cache_kr"], pbuf["out"],
                        workspace=pbuf["workspace"])
        del pbuf
        x = workloads.mla_tokens(wl, wl.batch, 1, dev)
        pos = torch.full((wl.batch,), wl.seq_len, dtype=torch.int32, device=dev)

        def call():
            moe.mla_decode(shape, x, pos, params, buf["cache_kv"], buf["cache_kr"], buf["out"],
                           residual=x, workspace=buf["workspace"], stream=stream)
    else:
        x = workloads.mla_tokens(wl, wl.tokens, 0, dev)

        def call():
            moe.mla_prefill(shape, x, params, buf["cache_kv"], buf["cache_kr"], buf["out"],
                            residual=x, workspace=buf["workspace"], stream=stream)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    launch = "eager"
    if wl.decode:
        # a decode step is five small launches: replay them as one captured
        # HIP graph, as a serving loop would (the graph's replays match the
        # eager call bit for bit, tests/test_gpu_mla.py)
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            call()
        torch.cuda.current_stream().wait_stream(stream)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            call()
        eager_call = call

        def call():  # noqa: F811
            graph.replay()  # on the current stream, where the events go
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        launch = "hip graph replay of one mla_decode call"
        del eager_call
        stream = torch.cuda.current_stream()
    ev = []
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(args.steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        ev.append((e0, e1))
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    per = [a.elapsed_time(b) for a, b in ev]
    med = float(np.median(per))
    flops, byts = mla_algorithmic(wl)
    tflops = flops / (med * 1e-3) / 1e12
    gbs = byts / (med * 1e-3) / 1e9
    line = {
        "metric": MLA_METRIC, "value": wl.tokens / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": name, "batch": wl.batch, "seq_len": wl.seq_len,
                   "max_len": wl.max_len, "d_model": wl.d_model, "n_heads": wl.n_heads,
                   "d_latent": wl.d_latent, "d_nope": wl.d_nope, "d_rope": wl.d_rope,
                   "d_v": wl.d_v, "decode": wl.decode, "launch": launch},
        "roofline": {"bound": "hbm" if wl.decode else "mfma",
                     "achieved": gbs if wl.decode else tflops,
                     "peak": PEAK_HBM_GBS if wl.decode else PEAK_BF16_TFLOPS,
                     "unit": "GB/s" if wl.decode else "TFLOP/s",
                     "frac": gbs / PEAK_HBM_GBS if wl.decode else tflops / PEAK_BF16_TFLOPS,
                     "traffic": None, "kernel": "the whole mla_decode / mla_prefill call",
                     "algorithmic_flop": flops, "algorithmic_bytes": byts,
                     "ms_per_call_median": med, "tflops": tflops, "gbs": gbs},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = mla_cpu_baseline(wl, args.cpu_seconds, x, params)
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.steps < 1 or args.warmup < 0 or args.ffn_events_every < 1:
        print("bench.py needs --steps >= 1, --warmup >= 0 and --ffn-events-every >= 1", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_mixture_experts_51_amd import moe, profiling, workloads

    name = args.workload or workloads.DEFAULT_BENCH_WORKLOAD
    if name in workloads.MLA_WORKLOADS:
        if args.with_backward or args.calibrate_copy:
            print("--with-backward and --calibrate-copy apply to the MoE workloads", file=sys.stderr)
            sys.exit(2)
        run_mla(args, name)
        return
    if name not in workloads.WORKLOADS:
        print(f"unknown workload {name!r}; one of "
              f"{sorted(workloads.WORKLOADS) + sorted(workloads.MLA_WORKLOADS)}", file=sys.stderr)
        sys.exit(2)

    if args.with_backward and workloads.WORKLOADS[name].norm:
        print("--with-backward: the backward of the pre-norm block's RMSNorm is not built",
              file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        # a plain device-to-device copy of profiling.COPY_BYTES bytes, three times
        src = torch.empty(profiling.COPY_BYTES, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    wl = workloads.WORKLOADS[name]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    moe.load()
    # achievable HBM read rate first, outside the timed region
    probes = hbm_read_probe()
    shape = moe.Shape.of(wl)
    L = wl.layers
    params = [workloads.layer_params(wl, l, dev) for l in range(L)]
    n_x = 2 if wl.steps > 1 else 1
    xs = [workloads.tokens(wl, s, dev) for s in range(n_x)]
    bufs = [moe.alloc_buffers(shape, dev) for _ in range(L)]
    stream = torch.cuda.current_stream()
    stacked = L > 1
    # one batch (inference-shaped): route with a frozen bias, update a training copy
    frozen = wl.steps == 1
    train_bias = [params[l]["bias"].clone() if frozen else params[l]["bias"] for l in range(L)]
    ev = []   # (start, end) events around one moe_grouped_ffn per timed step (layers in turn)
    evb = []  # (start, end) events around the bias updates of the same steps

    def step(i, timed, counts_out=None):
        """Step i; timed = index among the timed steps, or None."""
        x = xs[i % n_x]
        events = timed is not None and timed % args.ffn_events_every == 0
        for l in range(L):
            b, p = bufs[l], params[l]
            ws = b["workspace"]
            xin = x
            if wl.norm:  # pre-norm block: the MoE sees RMSNorm(x), the residual is x
                moe.moe_rmsnorm(shape, x, p["norm"], 1e-6, b["xn"], stream)
                xin = b["xn"]
            moe.moe_route(shape, xin, p["w_router"], p["bias"], b["topk_idx"], b["topk_gate"],
                          b["margin"], b["seq_balance"], 1e-4, ws, stream)
            moe.moe_permute(shape, b["topk_idx"], b["counts"], b["offsets"], b["perm_src"],
                            b["pos"], None, None, ws, stream)
            if counts_out is not None:
                counts_out.append(b["counts"].cpu().numpy())
            # one layer's FFN in every N-th timed step is timed with events
            # (layers in turn): each event record costs a few microseconds of
            # stream time, so timing every layer would inflate the step it measures
            ffn_timed = events and l == (timed // args.ffn_events_every) % L
            if ffn_timed:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            moe.moe_grouped_ffn(shape, xin, None, b["perm_src"], b["offsets"], p["w1"], p["w3"],
                                p["w2"], p.get("ws1"), p.get("ws3"), p.get("ws2"), b["y_perm"],
                                b["y_shared"], ws, stream)
            if ffn_timed:
                e1.record(stream)
                ev.append((e0, e1))
            moe.moe_combine(shape, b["y_perm"], b["y_shared"], b["topk_gate"], b["pos"],
                            x if stacked or wl.norm else None, b["out"], stream)
            x = b["out"]
        if events:
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        for l in range(L):
            moe.moe_update_bias(shape, bufs[l]["counts"], train_bias[l], 1e-3, stream)
        if events:
            e1.record(stream)
            evb.append((e0, e1))

    for i in range(args.warmup):
        step(i, None)
    torch.cuda.synchronize()
    # the live bias moves every step, and with it the set of experts that
    # receive rows; keep the starting biases to replay the timed steps afterwards
    bias0 = [params[l]["bias"].clone() for l in range(L)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i, i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / args.steps
    tokens_per_s = wl.tokens * L / (ms * 1e-3)

    ffn_times = [a.elapsed_time(b) for a, b in ev]
    ffn_ms = float(np.mean(ffn_times))
    bias_ms = float(np.mean([a.elapsed_time(b) for a, b in evb]))
    # Algorithmic bytes per moe_grouped_ffn launch, averaged over the same
    # launches the events timed: replay the timed steps (untimed, from the
    # same biases) and read every layer's counts.
    for l in range(L):
        params[l]["bias"].copy_(bias0[l])
    counts = []
    for i in range(args.steps):
        step(args.warmup + i, None, counts)
    torch.cuda.synchronize()
    algo = ffn_algorithmic(wl, counts)
    touched = float(np.mean([int((c > 0).sum()) for c in counts]))
    flops = float(np.mean([f for f, _ in algo]))
    byts = float(np.mean([b for _, b in algo]))
    t_s = ffn_ms * 1e-3
    ai = flops / byts
    ridge = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    if ai >= ridge:
        roof = {"bound": "mfma", "achieved": flops / t_s / 1e12, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": byts / t_s / 1e9, "peak": PEAK_HBM_GBS,
                "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    recorded = profiling.load_traffic(os.path.join(ROOT, "profiles"), wl.name)
    roof["traffic"] = recorded["hbm_bytes_per_launch"] if recorded else None
    if recorded:
        # counter traffic also holds the h round trip, which the algorithmic
        # bytes leave out
        roof["traffic_over_algorithmic"] = roof["traffic"] / byts
        roof["h_round_trip_bytes"] = 2.0 * 2 * (wl.tokens * wl.top_k * wl.hidden
                                                + wl.tokens * wl.shared_hidden)
    roof["kernel"] = ("moe_grouped_ffn = every grouped_gemm_kernel launch of one call "
                      "(SwiGLU and down stages; with streaming tiles the shared expert has its own)")
    roof["ms_per_launch"] = ffn_ms
    roof["ms_per_launch_median"] = float(np.median(ffn_times))
    roof["launches_timed"] = len(ffn_times)
    roof["algorithmic_flop"] = flops
    roof["algorithmic_bytes"] = byts
    roof["touched_experts"] = touched  # mean over the timed launches
    roof["mfma_frac"] = flops / t_s / 1e12 / PEAK_BF16_TFLOPS
    roof["hbm_frac"] = byts / t_s / 1e9 / PEAK_HBM_GBS
    # time at the spec roofline (the slower of MFMA and HBM) over measured time
    roof["attainable_frac"] = max(flops / (PEAK_BF16_TFLOPS * 1e12), byts / (PEAK_HBM_GBS * 1e9)) / t_s
    probe = max(probes.values())
    roof["hbm_read_probe_gbs"] = probe
    roof["hbm_read_probe_dma_gbs"] = probes["dma"]
    roof["hbm_read_probe_nt_gbs"] = probes["nt"]
    roof["hbm_read_probe"] = ("the faster of two reads of 8 GiB, best of four passes each: "
                              "moe_probe_hbm_read (LDS DMA, 32 KiB steps, one block per CU) and "
                              "moe_probe_hbm_read_nt (non-temporal 16-byte register loads)")
    roof["hbm_frac_of_probe"] = byts / t_s / 1e9 / probe
    if roof["bound"] == "hbm":
        # The two routed stages stream the touched experts' weights and write
        # h (SwiGLU) and y_perm (down) as their units finish: the same stream
        # with writes in the same ratio, on the probe, gives their time at the
        # achievable rate.
        stages = routed_stream_stages(wl, touched)
        rates = hbm_stream_probe({key: (w / r, row) for key, (r, w, row) in stages.items()})
        r_sw, r_dn = stages["swiglu"][0], stages["down"][0]
        routed_ms = (r_sw / (rates["swiglu"][1] * 1e9) + r_dn / (rates["down"][1] * 1e9)) * 1e3
        roof["stream_probe"] = {
            "kind": "moe_probe_hbm_read_write over about 8 GiB, best of four passes: the read rate of "
                    "an LDS-DMA stream of 256-row weight tiles with the stage's row length, 128 bytes of "
                    "each row per step, that writes after each tile what the routed stage writes per "
                    "tile of weights",
            "swiglu_written_per_read": rates["swiglu"][0], "swiglu_read_gbs": rates["swiglu"][1],
            "down_written_per_read": rates["down"][0], "down_read_gbs": rates["down"][1],
            "routed_weight_bytes": r_sw + r_dn,
            "routed_streams_ms_at_probe": routed_ms,
        }

    line = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": wl.tokens, "layers": L,
                   "seq_len": wl.seq_len, "d_model": wl.d_model, "n_experts": wl.n_experts,
                   "top_k": wl.top_k, "hidden": wl.hidden, "shared_hidden": wl.shared_hidden,
                   "value_counts": "tokens x layers per second",
                   "routing_bias": "frozen (inference); the update runs into a training copy"
                                   if frozen else "live (updated every step)",
                   "parallelism": "none (1 GPU)"},
        "update_bias_ms_per_step": bias_ms,
        "roofline": roof,
    }
    if args.with_backward:
        for l in range(L):
            params[l]["bias"].copy_(bias0[l])
        line["train"] = time_training(args, wl, shape, params, xs, stream)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds, params[0], xs[0])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
