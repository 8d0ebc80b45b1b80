"""Summaries of rocprofv3 output for the committed profiles.

    python -m sparse_mixture_experts_51_amd.profiling stats  <kernel_stats.csv> <out.md> <command>
    python -m sparse_mixture_experts_51_amd.profiling traffic <fetch_dir> <write_dir> <workload> \\
           <out.md> <command-fetch> <command-write>

`stats` turns a --kernel-trace --stats summary into a markdown table.
`traffic` reads two --pmc runs (FETCH_SIZE, then WRITE_SIZE) of
`bench.py --calibrate-copy`, whose first kernel is a plain device copy of
known size: each counter is scaled by bytes_copied / counter_on_the_copy, and
the per-launch HBM bytes of the grouped FFN (both GEMM kernels of one
moe_grouped_ffn call) are written with the sha256 of the GEMM source, so that
bench.py only reports them while that kernel is unchanged.
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
        gemm = {k: [v for _, v in lst] for k, lst in d.items() if "grouped_gemm" in k}
        if not any("true>(" in k for k in gemm) or not any("false>(" in k for k in gemm):
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
    else:
        raise SystemExit(__doc__)


if __name__ == "__main__":
    main(sys.argv)
