"""Summaries of rocprofv3 output for the committed profiles.

    python -m sparse_mixture_experts_51_amd.profiling stats  <kernel_stats.csv> <out.md> <command>
    python -m sparse_mixture_experts_51_amd.profiling traffic <fetch_dir> <write_dir> <workload> \\
           <out.md> <command-fetch> <command-write>

    python -m sparse_mixture_experts_51_amd.profiling kernels <fetch_dir> <write_dir> \
           <kernel_stats.csv> <bench.json> <out.md> <command-fetch> <command-write> <command-stats>
    python -m sparse_mixture_experts_51_amd.profiling mfma <pmc_dir> <kernel_stats.csv> \
           <bench.json> <out.md> <command-pmc> <command-stats>

`stats` turns a --kernel-trace --stats summary into a markdown table.
`traffic` reads two --pmc runs (FETCH_SIZE, then WRITE_SIZE) of
`bench.py --calibrate-copy`, whose first kernel is a plain device copy of
known size: each counter is scaled by bytes_copied / counter_on_the_copy, and
the per-launch HBM bytes of the grouped FFN (both GEMM kernels of one
moe_grouped_ffn call) are written with the sha256 of the GEMM source, so that
bench.py only reports them while that kernel is unchanged.
`kernels` puts every kernel of the step in one table: HBM bytes per dispatch
from the same two counter runs (scaled the same way), its average duration
from a --kernel-trace --stats run, and the rates against 8 TB/s, beside the
algorithmic bytes of the kernel (what the method must move).
`mfma` compares, per kernel, the matrix-core work the counters saw
(SQ_INSTS_VALU_MFMA_MOPS_BF16 / _F32, in units of 512 operations) with the
algorithmic FLOPs, and gives the matrix-core busy fraction
SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs).
The bench JSON line of the profiled command supplies the workload's shape
and the experts that received rows.
"""
from __future__ import annotations

import collections
import csv
import glob
import hashlib
import json
import os
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
GEMM_SRC = os.path.join(PKG, "csrc", "grouped_gemm.hip")
COPY_BYTES = 1 << 30  # bench.py --calibrate-copy copies this many bytes per launch
COPY_KERNEL = "copyBuffer"
TRAFFIC_TAG = "traffic-json: "


def gemm_source_sha() -> str:
    with open(GEMM_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _csv(path_or_dir: str, suffix: str):
    if os.path.isdir(path_or_dir):
        files = glob.glob(os.path.join(path_or_dir, "**", f"*{suffix}"), recursive=True)
        if not files:
            raise FileNotFoundError(f"no *{suffix} under {path_or_dir}")
        path_or_dir = files[0]
    with open(path_or_dir) as f:
        return list(csv.DictReader(f))


def stats_markdown(stats_csv: str, command: str, title: str) -> str:
    rows = _csv(stats_csv, "kernel_stats.csv")
    out = [f"# {title}", "", "Command:", "", "```", command, "```", "",
           "| kernel | calls | avg (us) | min (us) | max (us) | share |",
           "|---|---:|---:|---:|---:|---:|"]
    for r in rows:
        name = r["Name"].replace("|", "/")
        if "grouped_gemm_kernel<" in name:
            name = short_name(name)  # the template flags would be cut off below
        if len(name) > 90:
            name = name[:87] + "..."
        out.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{float(r['Percentage']):.2f}% |")
    return "\n".join(out) + "\n"


def _per_dispatch(rows, counter):
    """kernel name -> list of (dispatch id, value) for one counter."""
    d = collections.defaultdict(list)
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        d[r["Kernel_Name"]].append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    return d


def traffic(fetch_dir: str, write_dir: str) -> dict:
    res = {}
    for counter, path in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        d = _per_dispatch(_csv(path, "counter_collection.csv"), counter)
        copy = [v for k, lst in d.items() if COPY_KERNEL in k for _, v in lst]
        if not copy:
            raise RuntimeError(f"no {COPY_KERNEL} dispatch in the {counter} run")
        # the calibration copies are the large ones; other copies are small uploads
        copy = [v for v in copy if v >= 0.5 * max(copy)]
        factor = COPY_BYTES / (sum(copy) / len(copy) * 1024.0)
        # one FFN call runs each grouped_gemm instance once (the SwiGLU and down
        # stages, each possibly split into a routed and a shared-expert launch):
        # per call, the mean dispatch of every instance, summed
        gemm = {k: [v for _, v in lst] for k, lst in d.items() if _forward_gemm(k)}
        if not any(gemm_flags(k)[0] for k in gemm) or not any(not gemm_flags(k)[0] for k in gemm):
            raise RuntimeError(f"no grouped_gemm dispatches in the {counter} run")
        kib = sum(sum(v) / len(v) for v in gemm.values())
        res[counter] = {"kib_per_launch": kib, "factor": factor, "bytes_per_launch": kib * 1024 * factor,
                        "copy_kib": sum(copy) / len(copy)}
    return res


def traffic_markdown(fetch_dir, write_dir, workload, cmd_fetch, cmd_write) -> str:
    t = traffic(fetch_dir, write_dir)
    total = t["FETCH_SIZE"]["bytes_per_launch"] + t["WRITE_SIZE"]["bytes_per_launch"]
    payload = {"workload": workload, "kernel": "moe_grouped_ffn (grouped_gemm_kernel SwiGLU + down)",
               "gemm_source_sha256": gemm_source_sha(), "hbm_bytes_per_launch": total,
               "fetch_bytes_per_launch": t["FETCH_SIZE"]["bytes_per_launch"],
               "write_bytes_per_launch": t["WRITE_SIZE"]["bytes_per_launch"],
               "fetch_factor": t["FETCH_SIZE"]["factor"], "write_factor": t["WRITE_SIZE"]["factor"]}
    lines = [f"# HBM traffic of moe_grouped_ffn, {workload}", "",
             "Two counter runs of the same command (FETCH_SIZE, then WRITE_SIZE, KiB per",
             f"dispatch).  The command first copies {COPY_BYTES} bytes with a plain device",
             "copy; each counter is scaled by bytes_copied / (counter on that copy).", "",
             "```", cmd_fetch, cmd_write, "```", "",
             "| counter | copy reads (KiB) | factor | FFN launch (KiB) | FFN launch (bytes, scaled) |",
             "|---|---:|---:|---:|---:|"]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        v = t[c]
        lines.append(f"| {c} | {v['copy_kib']:.0f} | {v['factor']:.4f} | {v['kib_per_launch']:.0f} | "
                     f"{v['bytes_per_launch']:.4g} |")
    lines += ["", f"HBM bytes per launch: {total:.4g}", "", TRAFFIC_TAG + json.dumps(payload), ""]
    return "\n".join(lines)


def load_traffic(profiles_dir: str, workload: str):
    """Per-launch HBM bytes recorded for `workload`, or None when absent or
    taken on a different version of the GEMM kernel."""
    path = os.path.join(profiles_dir, f"grouped_ffn_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if line.startswith(TRAFFIC_TAG):
                payload = json.loads(line[len(TRAFFIC_TAG):])
                if payload.get("gemm_source_sha256") != gemm_source_sha():
                    return None
                return payload
    return None


PEAK_HBM = 8e12
PEAK_BF16 = 2.5e15
PEAK_F32_MFMA = 157.3e12
SIMDS = 1024  # 256 compute units x 4 SIMDs
XCDS = 8      # GRBM_GUI_ACTIVE per dispatch comes summed over the 8 XCDs


def _stats_by_kernel(stats_csv: str) -> dict:
    """kernel name -> (calls, average duration in seconds)."""
    rows = _csv(stats_csv, "kernel_stats.csv")
    return {r["Name"]: (int(r["Calls"]), float(r["AverageNs"]) * 1e-9) for r in rows}


def gemm_flags(name: str) -> tuple:
    """(SwiGLU stage?, backward epilogue?, K-major weights?) of a
    `grouped_gemm_kernel<TileCfg<...>, bool, bool, bool>` instance name."""
    base = name.split("(")[0]
    rest = base[base.index("TileCfg<"):]
    rest = rest[rest.index(">") + 1:]
    flags = [f.strip() == "true" for f in rest.replace(">", "").split(",") if f.strip()]
    flags += [False] * (3 - len(flags))
    return flags[0], flags[1], flags[2]


def _forward_gemm(name: str) -> bool:
    return "grouped_gemm" in name and not any(gemm_flags(name)[1:])


def _mean_per_kernel(rows, counter) -> dict:
    d = _per_dispatch(rows, counter)
    return {k: sum(v for _, v in lst) / len(lst) for k, lst in d.items()}


def short_name(name: str) -> str:
    """`void moe::grouped_gemm_kernel<moe::TileCfg<192, 256, ...>, true, false, false>(...)`
    -> `grouped_gemm_kernel<192x256, SwiGLU>` (the backward's instances: SwiGLU-bwd,
    dgrad); other kernels keep their bare name."""
    base = name.split("(")[0].replace("void ", "").replace("moe::", "")
    if base.startswith("grouped_gemm_kernel"):
        cfg = base[base.index("TileCfg<") + 8:].split(">")[0].split(",")
        swiglu, bwd, wkm = gemm_flags(base)
        stage = ("SwiGLU-bwd" if bwd else "SwiGLU") if swiglu else ("dgrad" if wkm else "down")
        loaders = int(cfg[8]) if len(cfg) > 8 else 0
        tile = f"{cfg[0].strip()}x{cfg[1].strip()}" + (f"+{loaders}ldr" if loaders else "")
        return f"grouped_gemm_kernel<{tile}, {stage}>"
    return base.split("<")[0]


def _gemm_parts(name: str, names) -> tuple:
    """(stage, routed?, shared?) of a grouped-GEMM instance.  When a streaming
    (192x256) instance is present, the routed experts run in it and the shared
    expert in the other instance of the same stage; otherwise one instance
    per stage runs both."""
    stage = "swiglu" if short_name(name).endswith("SwiGLU>") else "down"
    streaming = any("TileCfg<192, 256" in n for n in names)
    if not streaming:
        return stage, True, True
    if "TileCfg<192, 256" in name:
        return stage, True, False
    return stage, False, True


def algorithmic(name: str, names, b: dict) -> tuple:
    """(FLOPs, bytes) that the method must do in one dispatch of kernel
    `name`, for the bench line `b` (its config and roofline), or (None, None)
    for kernels outside the layer (torch fills, copies, probes)."""
    c = b["config"]
    T, d, E, k, H, Hs = (c["tokens"], c["d_model"], c["n_experts"], c["top_k"], c["hidden"],
                         c["shared_hidden"])
    S = c["seq_len"]
    touched = b["roofline"].get("touched_experts", E)
    stacked = c["layers"] > 1
    n = short_name(name)
    if n.startswith("grouped_gemm_kernel"):
        stage, routed, shared = _gemm_parts(name, names)
        fl = by = 0.0
        if stage == "swiglu":
            if routed:
                fl += 4.0 * d * H * T * k
                by += 2.0 * (2 * H * d * touched + T * d + T * k * H)
            if shared:
                fl += 4.0 * d * Hs * T
                by += 2.0 * (2 * Hs * d + T * d + T * Hs)
        else:
            if routed:
                fl += 2.0 * d * H * T * k
                by += 2.0 * (H * d * touched + T * k * H + T * k * d)
            if shared:
                fl += 2.0 * d * Hs * T
                by += 2.0 * (Hs * d + T * Hs + T * d)
        return fl, by
    if n in ("router_scores_kernel", "router_scores_mfma_kernel"):
        return 2.0 * T * d * E, 2.0 * T * d + 4.0 * d * E + 4.0 * T * E
    if n == "router_fused_kernel":
        return 2.0 * T * d * E, 2.0 * T * d + 4.0 * d * E + 4.0 * E + 8.0 * T * k + 4.0 * T
    if n == "select_kernel":
        return None, 4.0 * T * E + 4.0 * E + 8.0 * T * k + 4.0 * T + (8.0 * T if S else 0.0)
    if n == "seq_partial_kernel":
        return None, 4.0 * T * E + 8.0 * T + 4.0 * T * k
    if n == "seq_final_kernel":
        return None, 4.0 * (T // S if S else 0)
    if n == "perm_count_kernel":
        return None, 4.0 * T * k
    if n == "perm_scatter_kernel":
        return None, 4.0 * T * k + 8.0 * T * k + 8.0 * E
    if n == "perm_scan_kernel":
        return None, 8.0 * E
    if n == "perm_gather_kernel":
        return None, 4.0 * T * k * d
    if n == "combine_kernel":
        return None, 2.0 * T * k * d + 2.0 * T * d * (2 + (1 if stacked else 0)) + 8.0 * T * k
    if n == "update_bias_kernel":
        return None, 8.0 * E
    return None, None


def _is_layer_kernel(name: str) -> bool:
    return "moe::" in name


def kernels_markdown(fetch_dir, write_dir, stats_csv, bench_json, cmd_fetch, cmd_write,
                     cmd_stats) -> str:
    with open(bench_json) as f:
        b = json.loads(f.read().strip().splitlines()[-1])
    stats = _stats_by_kernel(stats_csv)
    scaled = {}
    factors = {}
    for counter, path in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _csv(path, "counter_collection.csv")
        means = _mean_per_kernel(rows, counter)
        copy = [v for kk, lst in _per_dispatch(rows, counter).items() if COPY_KERNEL in kk
                for _, v in lst]
        copy = [v for v in copy if v >= 0.5 * max(copy)]
        factors[counter] = COPY_BYTES / (sum(copy) / len(copy) * 1024.0)
        scaled[counter] = {kk: v * 1024.0 * factors[counter] for kk, v in means.items()}
    names = [n for n in stats if _is_layer_kernel(n)]
    names.sort(key=lambda n: -stats[n][0] * stats[n][1])
    c = b["config"]
    lines = [f"# Every kernel of the step: HBM bytes and rates, {c['workload']}", "",
             "Durations: average per dispatch of a --kernel-trace --stats run.  Bytes: FETCH_SIZE",
             "and WRITE_SIZE per dispatch from two --pmc runs, each scaled by bytes_copied /",
             f"(counter on a plain copy of {COPY_BYTES} bytes) -- factors "
             f"{factors['FETCH_SIZE']:.4f} (fetch) and {factors['WRITE_SIZE']:.4f} (write).",
             "Algorithmic bytes: what the method must move in that dispatch (inputs read once,",
             "outputs written once, weights of the experts that received rows).  Rates are",
             "against the 8 TB/s HBM peak.", "", "```", cmd_stats, cmd_fetch, cmd_write, "```", "",
             "| kernel | calls | avg (us) | counter bytes | counter GB/s | algorithmic bytes | "
             "algorithmic GB/s | % of 8 TB/s | counter / algorithmic |",
             "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for n in names:
        calls, t = stats[n]
        cb = scaled["FETCH_SIZE"].get(n, float("nan")) + scaled["WRITE_SIZE"].get(n, float("nan"))
        _, ab = algorithmic(n, names, b)
        ab_s = f"{ab:.4g}" if ab is not None else "-"
        ag = f"{ab / t / 1e9:.0f}" if ab is not None else "-"
        pct = f"{100 * ab / t / PEAK_HBM:.1f}%" if ab is not None else "-"
        ratio = f"{cb / ab:.2f}" if ab else "-"
        lines.append(f"| `{short_name(n)}` | {calls} | {t * 1e6:.1f} | {cb:.4g} | {cb / t / 1e9:.0f} | "
                     f"{ab_s} | {ag} | {pct} | {ratio} |")
    return "\n".join(lines) + "\n"


def mfma_markdown(pmc_dir, stats_csv, bench_json, cmd_pmc, cmd_stats) -> str:
    with open(bench_json) as f:
        b = json.loads(f.read().strip().splitlines()[-1])
    stats = _stats_by_kernel(stats_csv)
    rows = _csv(pmc_dir, "counter_collection.csv")
    bf16 = _mean_per_kernel(rows, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    f32 = _mean_per_kernel(rows, "SQ_INSTS_VALU_MFMA_MOPS_F32")
    busy = _mean_per_kernel(rows, "SQ_VALU_MFMA_BUSY_CYCLES")
    gui = _mean_per_kernel(rows, "GRBM_GUI_ACTIVE")
    names = [n for n in stats if _is_layer_kernel(n) and (bf16.get(n, 0) > 0 or f32.get(n, 0) > 0)]
    names.sort(key=lambda n: -stats[n][0] * stats[n][1])
    c = b["config"]
    lines = [f"# Matrix-core work and utilisation per kernel, {c['workload']}", "",
             "Counter FLOPs = (SQ_INSTS_VALU_MFMA_MOPS_BF16 + SQ_INSTS_VALU_MFMA_MOPS_F32) x 512",
             "per dispatch; algorithmic FLOPs = what the method must compute in that dispatch",
             "(2 per multiply-add; the grouped GEMMs' counter FLOPs exceed it by the padding",
             "rows of partly filled 32-row tiles).  GRBM_GUI_ACTIVE per dispatch comes summed",
             f"over the {XCDS} XCDs (it reads {XCDS} x clock x duration), so the clock is",
             f"GRBM_GUI_ACTIVE / {XCDS} / duration and MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES /",
             f"(GRBM_GUI_ACTIVE / {XCDS} x {SIMDS} SIMDs).  Achieved = algorithmic FLOPs / average",
             "duration (--kernel-trace --stats run) against the dense peak of the kernel's",
             "type (bf16 2.5 PFLOP/s, fp32 matrix 157.3 TFLOP/s, both at 2.4 GHz); the last",
             "column rescales that peak to the clock the kernel actually ran at (given for",
             "kernels of 200 us or more: on shorter ones the counter run's dispatch overhead",
             "inflates the active cycles).", "", "```",
             cmd_stats, cmd_pmc, "```", "",
             "| kernel | avg (us) | counter FLOPs | algorithmic FLOPs | counter / algorithmic | "
             "achieved TFLOP/s | % of peak | MFMA busy | clock (GHz) | % of peak at that clock |",
             "|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for n in names:
        _, t = stats[n]
        is_bf16 = bf16.get(n, 0) > 0
        cf = (bf16.get(n, 0) + f32.get(n, 0)) * 512.0
        af, _ = algorithmic(n, names, b)
        peak = PEAK_BF16 if is_bf16 else PEAK_F32_MFMA
        g = gui.get(n, 0.0) / XCDS
        util = busy.get(n, 0.0) / (g * SIMDS) if g else float("nan")
        # short kernels: the counter run's own dispatch overhead inflates the
        # active cycles against the traced duration, so no clock is derived
        clock = g / t / 1e9 if g and t >= 200e-6 else None
        af_s = f"{af:.4g}" if af else "-"
        ratio = f"{cf / af:.3f}" if af else "-"
        ach = f"{af / t / 1e12:.0f}" if af else "-"
        pct = f"{100 * af / t / peak:.1f}%" if af else "-"
        pct_clk = f"{100 * af / t / (peak * clock / 2.4):.1f}%" if af and clock else "-"
        clk = f"{clock:.2f}" if clock else "-"
        lines.append(f"| `{short_name(n)}` | {t * 1e6:.1f} | {cf:.4g} | {af_s} | {ratio} | {ach} | "
                     f"{pct} | {100 * util:.1f}% | {clk} | {pct_clk} |")
    return "\n".join(lines) + "\n"


def main(argv):
    if argv[1] == "stats":
        _, _, src, out, cmd = argv[:5]
        title = argv[5] if len(argv) > 5 else "rocprofv3 kernel statistics"
        with open(out, "w") as f:
            f.write(stats_markdown(src, cmd, title))
    elif argv[1] == "traffic":
        _, _, fdir, wdir, workload, out, cf, cw = argv[:8]
        with open(out, "w") as f:
            f.write(traffic_markdown(fdir, wdir, workload, cf, cw))
    elif argv[1] == "kernels":
        _, _, fdir, wdir, st, bj, out, cf, cw, cs = argv[:10]
        with open(out, "w") as f:
            f.write(kernels_markdown(fdir, wdir, st, bj, cf, cw, cs))
    elif argv[1] == "mfma":
        _, _, pdir, st, bj, out, cp, cs = argv[:8]
        with open(out, "w") as f:
            f.write(mfma_markdown(pdir, st, bj, cp, cs))
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv)
