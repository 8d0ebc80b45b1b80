"""Benchmark of the DeepSeekMoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the whole hot path over one batch: for every layer of
the workload, moe_route -> moe_permute -> moe_grouped_ffn -> moe_combine
(the combine also adds the residual stream of stacked layers), then
moe_update_bias for every layer.  Inputs are seeded synthetic tensors already
resident in HBM before the timed region.  Prints ONE JSON line.

value = tokens x layers / second (each token counted once per MoE layer
forward).  The roofline object covers the dominant kernel pair -- the grouped
expert GEMMs of moe_grouped_ffn -- timed live with HIP events on the stream
they are launched on, around one layer's call in every fifth timed step
(layers in turn; an event record costs a few microseconds of stream time).
By default 20 warm-up steps and 100 timed steps: the clocks settle within
the warm-up.  cpu_baseline times the CPU oracle on a bounded token sample of
the same workload.
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
    return ap.parse_args()


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


def cpu_baseline(wl, target_s: float):
    """The CPU oracle, as it stands, on a bounded sample of the workload.

    Mini shapes: whole layer passes over all tokens (layer i % L of step
    i // L) until the timed oracle work reaches target_s.  V3 shapes (22.5 GB
    of experts): the first n tokens are routed on the host, only the experts
    they chose are drawn, and the oracle's expert FFN and combine run for
    them.  Weight generation is outside the timed part."""
    import numpy as np
    import torch

    import oracle
    from sparse_mixture_experts_51_amd import workloads

    threads = oracle.default_threads()
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
            oracle.layer(xb, hp[l], wl.top_k, seq_len=wl.seq_len, nthreads=threads)
            dt += time.perf_counter() - t0
            done += 1
        return {"value": done * wl.tokens / dt, "unit": "tokens/s", "cores": threads,
                "kind": "oracle",
                "sample": f"{done} layer passes over all {wl.tokens} tokens of {wl.name} (route, "
                          f"balance statistic, permute, grouped FFN, combine), fp64 oracle, "
                          f"{dt:.1f} s on {threads} threads; counts tokens x layers per second"}

    import concurrent.futures as cf
    xb = oracle.as_bf16_bits(workloads.tokens(wl, 0, "cpu"))
    w_r = workloads.router(wl, 0, "cpu").numpy()
    b = workloads.bias(wl, 0, "cpu").numpy()
    sh = {k: oracle.as_bf16_bits(v) for k, v in workloads.shared_weights(wl, 0, "cpu").items()}
    cache = {}
    n = 4
    while True:
        r = oracle.route(xb[:n], w_r, b, wl.top_k, threads)
        for e in np.unique(r["idx"]):
            if e not in cache:
                ew = workloads.one_expert(wl, int(e), 0, "cpu")
                cache[e] = tuple(oracle.as_bf16_bits(ew[k]) for k in ("w1", "w3", "w2"))
        t0 = time.perf_counter()
        r = oracle.route(xb[:n], w_r, b, wl.top_k, threads)
        jobs = [(t, j) for t in range(n) for j in range(wl.top_k)]
        with cf.ThreadPoolExecutor(threads) as ex:
            ys = list(ex.map(lambda tj: oracle.expert_ffn(xb[tj[0]], *cache[r["idx"][tj]]), jobs))
            ysh = list(ex.map(lambda t: oracle.expert_ffn(xb[t], sh["ws1"], sh["ws3"], sh["ws2"]),
                              range(n)))
        pos = np.arange(n * wl.top_k, dtype=np.int32).reshape(n, wl.top_k)
        oracle.combine(np.stack(ys), np.stack(ysh), r["gate"], r["idx"], pos)
        dt = time.perf_counter() - t0
        if dt >= target_s / 2 or n >= min(64, wl.tokens):
            break
        n = min(64, wl.tokens, n * 2)
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {wl.tokens} tokens of {wl.name}: routed on the host, then "
                      f"expert FFN of their {wl.top_k} chosen experts plus the shared expert and "
                      f"the combine, fp64 oracle, {dt:.1f} s on {threads} threads"}


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

    if args.calibrate_copy:
        # a plain device-to-device copy of profiling.COPY_BYTES bytes, three times
        src = torch.empty(profiling.COPY_BYTES, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    name = args.workload or workloads.DEFAULT_BENCH_WORKLOAD
    wl = workloads.WORKLOADS[name]
    dev = "cuda:0"
    torch.cuda.set_device(0)
    moe.load()
    shape = moe.Shape.of(wl)
    L = wl.layers
    params = [workloads.layer_params(wl, l, dev) for l in range(L)]
    n_x = 2 if wl.steps > 1 else 1
    xs = [workloads.tokens(wl, s, dev) for s in range(n_x)]
    bufs = [moe.alloc_buffers(shape, dev) for _ in range(L)]
    stream = torch.cuda.current_stream()
    stacked = L > 1
    ev = []  # (start, end) events around one moe_grouped_ffn per timed step (layers in turn)

    def step(i, timed, counts_out=None):
        x = xs[i % n_x]
        for l in range(L):
            b, p = bufs[l], params[l]
            ws = b["workspace"]
            moe.moe_route(shape, x, p["w_router"], p["bias"], b["topk_idx"], b["topk_gate"],
                          b["margin"], b["seq_balance"], 1e-4, ws, stream)
            moe.moe_permute(shape, b["topk_idx"], b["counts"], b["offsets"], b["perm_src"],
                            b["pos"], None, None, ws, stream)
            if counts_out is not None:
                counts_out.append(b["counts"].cpu().numpy())
            # one layer's FFN in every N-th step is timed with events (layers
            # in turn): each event record costs a few microseconds of stream
            # time, so timing every layer would inflate the step it measures
            ffn_timed = timed and i % args.ffn_events_every == 0 and l == (i // args.ffn_events_every) % L
            if ffn_timed:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            moe.moe_grouped_ffn(shape, x, None, b["perm_src"], b["offsets"], p["w1"], p["w3"],
                                p["w2"], p.get("ws1"), p.get("ws3"), p.get("ws2"), b["y_perm"],
                                b["y_shared"], ws, stream)
            if ffn_timed:
                e1.record(stream)
                ev.append((e0, e1))
            moe.moe_combine(shape, b["y_perm"], b["y_shared"], b["topk_gate"], b["pos"],
                            x if stacked else None, b["out"], stream)
            x = b["out"]
        for l in range(L):
            moe.moe_update_bias(shape, bufs[l]["counts"], params[l]["bias"], 1e-3, stream)

    for i in range(args.warmup):
        step(i, False)
    torch.cuda.synchronize()
    # the bias moves every step, and with it the set of experts that receive
    # rows; keep the starting biases to replay the timed steps afterwards
    bias0 = [params[l]["bias"].clone() for l in range(L)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i, True)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / args.steps
    tokens_per_s = wl.tokens * L / (ms * 1e-3)

    ffn_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    # Algorithmic bytes per moe_grouped_ffn launch, averaged over the same
    # launches the events timed: replay the timed steps (untimed, from the
    # same biases) and read every layer's counts.
    for l in range(L):
        params[l]["bias"].copy_(bias0[l])
    counts = []
    for i in range(args.steps):
        step(args.warmup + i, False, counts)
    torch.cuda.synchronize()
    algo = ffn_algorithmic(wl, counts)
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
        roof["traffic_over_algorithmic"] = roof["traffic"] / byts
    roof["kernel"] = ("moe_grouped_ffn = every grouped_gemm_kernel launch of one call "
                      "(SwiGLU and down stages; with streaming tiles the shared expert has its own)")
    roof["ms_per_launch"] = ffn_ms
    roof["algorithmic_flop"] = flops
    roof["algorithmic_bytes"] = byts
    roof["mfma_frac"] = flops / t_s / 1e12 / PEAK_BF16_TFLOPS
    roof["hbm_frac"] = byts / t_s / 1e9 / PEAK_HBM_GBS
    # time at the spec roofline (the slower of MFMA and HBM) over measured time
    roof["attainable_frac"] = max(flops / (PEAK_BF16_TFLOPS * 1e12), byts / (PEAK_HBM_GBS * 1e9)) / t_s
    probes = hbm_read_probe()
    probe = max(probes.values())
    roof["hbm_read_probe_gbs"] = probe
    roof["hbm_read_probe_dma_gbs"] = probes["dma"]
    roof["hbm_read_probe_nt_gbs"] = probes["nt"]
    roof["hbm_read_probe"] = ("the faster of two reads of 8 GiB, best of four passes each: "
                              "moe_probe_hbm_read (LDS DMA, 32 KiB steps, one block per CU) and "
                              "moe_probe_hbm_read_nt (non-temporal 16-byte register loads)")
    roof["hbm_frac_of_probe"] = byts / t_s / 1e9 / probe

    line = {
        "metric": METRIC, "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": wl.tokens, "layers": L,
                   "seq_len": wl.seq_len, "d_model": wl.d_model, "n_experts": wl.n_experts,
                   "top_k": wl.top_k, "hidden": wl.hidden, "shared_hidden": wl.shared_hidden,
                   "value_counts": "tokens x layers per second",
                   "parallelism": "none (1 GPU)"},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
