"""Host-side checks of the rocprofv3 summary helpers (synthetic CSV input)."""
import csv
import json
import os

import pytest

from sparse_mixture_experts_51_amd import profiling

SWIG = "void moe::grouped_gemm_kernel<moe::TileCfg<128, 128, 2, 2, 2, true>, true>(moe::GroupedGemmArgs)"
DOWN = "void moe::grouped_gemm_kernel<moe::TileCfg<128, 128, 2, 2, 2, true>, false>(moe::GroupedGemmArgs)"


def _write(dirpath, counter, rows):
    os.makedirs(dirpath, exist_ok=True)
    with open(os.path.join(dirpath, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": v})


def test_traffic_scales_by_the_calibration_copy(tmp_path):
    kib = profiling.COPY_BYTES / 1024
    # the counter reads 2x the true bytes on the copy, so the factor is 0.5;
    # a small upload copy must not enter the calibration
    _write(tmp_path / "f", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 4.0),
                                          ("__amd_rocclr_copyBuffer", 2 * kib),
                                          ("__amd_rocclr_copyBuffer", 2 * kib),
                                          (SWIG, 1000.0), (SWIG, 3000.0), (DOWN, 500.0)])
    _write(tmp_path / "w", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", kib),
                                          (SWIG, 100.0), (DOWN, 300.0)])
    t = profiling.traffic(str(tmp_path / "f"), str(tmp_path / "w"))
    assert t["FETCH_SIZE"]["factor"] == pytest.approx(0.5)
    assert t["FETCH_SIZE"]["bytes_per_launch"] == pytest.approx((2000.0 + 500.0) * 1024 * 0.5)
    assert t["WRITE_SIZE"]["bytes_per_launch"] == pytest.approx(400.0 * 1024)


def test_traffic_sums_the_instances_of_one_call(tmp_path):
    # a call that splits each stage into two kernel instances: per call, the
    # mean of each instance, summed over the instances
    big_s = SWIG.replace("128, 128, 2, 2, 2", "256, 128, 4, 2, 1")
    big_d = DOWN.replace("128, 128, 2, 2, 2", "256, 128, 4, 2, 1")
    kib = profiling.COPY_BYTES / 1024
    rows = [("__amd_rocclr_copyBuffer", kib)]
    for _ in range(3):
        rows += [(SWIG, 1000.0), (big_s, 100.0), (DOWN, 500.0), (big_d, 50.0)]
    _write(tmp_path / "f", "FETCH_SIZE", rows)
    _write(tmp_path / "w", "WRITE_SIZE", rows)
    t = profiling.traffic(str(tmp_path / "f"), str(tmp_path / "w"))
    assert t["FETCH_SIZE"]["bytes_per_launch"] == pytest.approx(1650.0 * 1024)


def test_traffic_record_is_tied_to_the_gemm_source(tmp_path):
    kib = profiling.COPY_BYTES / 1024
    _write(tmp_path / "f", "FETCH_SIZE", [("__amd_rocclr_copyBuffer", kib), (SWIG, 10.0), (DOWN, 10.0)])
    _write(tmp_path / "w", "WRITE_SIZE", [("__amd_rocclr_copyBuffer", kib), (SWIG, 1.0), (DOWN, 1.0)])
    md = profiling.traffic_markdown(str(tmp_path / "f"), str(tmp_path / "w"), "wl", "cmd-f", "cmd-w")
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "grouped_ffn_traffic_wl.md").write_text(md)
    rec = profiling.load_traffic(str(prof), "wl")
    assert rec["hbm_bytes_per_launch"] == pytest.approx(22.0 * 1024)
    stale = md.replace(profiling.gemm_source_sha(), "0" * 64)
    (prof / "grouped_ffn_traffic_wl.md").write_text(stale)
    assert profiling.load_traffic(str(prof), "wl") is None
    assert profiling.load_traffic(str(prof), "other") is None


def test_stats_markdown(tmp_path):
    p = tmp_path / "k_kernel_stats.csv"
    p.write_text('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
                 f'"{SWIG}",2,2000,1000.0,50.0,900,1100,1.0\n')
    md = profiling.stats_markdown(str(p), "rocprofv3 ...", "t")
    assert "| 2 | 1.0 | 0.9 | 1.1 | 50.00% |" in md


def _write_multi(dirpath, rows):
    """rows: (kernel, counter, value) for one dispatch each (ids in order)."""
    os.makedirs(dirpath, exist_ok=True)
    with open(os.path.join(dirpath, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (name, counter, v) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": v})


STREAM_S = "void moe::grouped_gemm_kernel<moe::TileCfg<192, 256, 2, 4, 1, true, false, 2, 4>, true>(moe::GroupedGemmArgs)"
SHARED_S = "void moe::grouped_gemm_kernel<moe::TileCfg<256, 128, 4, 2, 1, true, true, 3, 4>, true>(moe::GroupedGemmArgs)"
COMBINE = "void moe::combine_kernel<int>(unsigned short const*, unsigned short const*)"
BENCH = {"config": {"workload": "wl", "tokens": 64, "d_model": 128, "n_experts": 8, "top_k": 2,
                    "hidden": 64, "shared_hidden": 64, "seq_len": 0, "layers": 1},
         "roofline": {"touched_experts": 5.0}}


def test_algorithmic_work_of_the_gemm_instances():
    names = [STREAM_S, SHARED_S]
    T, d, k, H, Hs = 64, 128, 2, 64, 64
    f, b = profiling.algorithmic(STREAM_S, names, BENCH)
    assert f == 4.0 * d * H * T * k  # routed rows only: the shared expert has its own launch
    assert b == 2.0 * (2 * H * d * 5 + T * d + T * k * H)
    f, b = profiling.algorithmic(SHARED_S, names, BENCH)
    assert f == 4.0 * d * Hs * T
    # without a streaming instance one launch per stage runs both
    f, _ = profiling.algorithmic(SWIG, [SWIG, DOWN], BENCH)
    assert f == 4.0 * d * (H * T * k + Hs * T)
    f, _ = profiling.algorithmic(DOWN, [SWIG, DOWN], BENCH)
    assert f == 2.0 * d * (H * T * k + Hs * T)
    assert profiling.algorithmic("__amd_rocclr_copyBuffer", names, BENCH) == (None, None)
    assert profiling.short_name(SHARED_S) == "grouped_gemm_kernel<256x128+4ldr, SwiGLU>"


def test_kernels_and_mfma_tables(tmp_path):
    kib = profiling.COPY_BYTES / 1024
    _write_multi(tmp_path / "f", [("__amd_rocclr_copyBuffer", "FETCH_SIZE", 2 * kib),
                                  (COMBINE, "FETCH_SIZE", 100.0), (COMBINE, "FETCH_SIZE", 300.0)])
    _write_multi(tmp_path / "w", [("__amd_rocclr_copyBuffer", "WRITE_SIZE", kib),
                                  (COMBINE, "WRITE_SIZE", 50.0)])
    st = tmp_path / "k_kernel_stats.csv"
    st.write_text('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
                  f'"{COMBINE}",2,2000,1000.0,50.0,900,1100,1.0\n'
                  f'"{SWIG}",2,4000,2000.0,50.0,900,1100,1.0\n')
    bj = tmp_path / "b.json"
    bj.write_text("noise\n" + json.dumps(BENCH) + "\n")
    md = profiling.kernels_markdown(str(tmp_path / "f"), str(tmp_path / "w"), str(st), str(bj),
                                    "cf", "cw", "cs")
    # combine: (200 KiB fetched x 0.5 + 50 KiB written) in 1 us
    row = next(l for l in md.splitlines() if l.startswith("| `combine_kernel`"))
    assert "| 2 | 1.0 | 1.536e+05 | 154 |" in row
    _write_multi(tmp_path / "p", [(SWIG, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1000.0),
                                  (SWIG, "SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0),
                                  (SWIG, "SQ_VALU_MFMA_BUSY_CYCLES", 512.0 * 1024),
                                  (SWIG, "GRBM_GUI_ACTIVE", 8 * 2048.0),
                                  (COMBINE, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)])
    md = profiling.mfma_markdown(str(tmp_path / "p"), str(st), str(bj), "cp", "cs")
    row = next(l for l in md.splitlines() if "SwiGLU" in l)
    # a quarter of the SIMD cycles busy; no clock for a 2 us kernel
    assert "| 5.12e+05 |" in row and "| 25.0% | - | - |" in row
    assert "combine_kernel" not in md  # no matrix-core work
