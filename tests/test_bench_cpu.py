"""Host logic of bench.py on the CPU: the rocprofv3 counter and trace digests.

Synthetic counter files stand in for two --pmc runs: a copy probe of known
size fixes each counter's scale, and the digest must report, for the largest
dispatch of each kernel family, the scaled bytes per launch; a kernel-trace
digest must group dispatches by launch shape; the MFMA counter digest must
relate the GEMM's MFMA busy cycles to those of the MFMA loop probe.
"""

import csv

import pytest

import bench

COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
        "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
        "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
        "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write_counters(d, name, rows):
    d.mkdir(parents=True)
    with open(d / "bench_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        for i, (kernel, grid, values) in enumerate(rows):
            for v in values:  # one row per counter instance, summed by the digest
                w.writerow({c: 0 for c in COLS} | {
                    "Dispatch_Id": i + 1, "Kernel_Name": kernel, "Grid_Size": grid,
                    "Counter_Name": name, "Counter_Value": v})


def test_summarize_pmc_scales_by_copy_probe(tmp_path, monkeypatch):
    probe_kib = bench.COPY_PROBE_BYTES / 1024
    fam = {k: (tmp_path / f"{k}.txt", sub, what) for k, (_, sub, what) in bench.COUNTERS.items()}
    monkeypatch.setattr(bench, "COUNTERS", fam)
    neg = "at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda"
    gemv = "ternary::(anonymous namespace)::gemv_f4_kernel<false, 0, 1>(ternary::(anonymous namespace)::F4Batch)"
    gemm = "ternary::dma::gemm_dma_kernel<false, false, Cfg<256, 128, 4, 1, 4, 2> >(BigBatch)"
    # FETCH_SIZE reads half the bytes (scale 2), WRITE_SIZE all of them (scale 1)
    _write_counters(tmp_path / "F", "FETCH_SIZE", [
        (neg, 1 << 20, [probe_kib / 4, probe_kib / 4]),
        (gemv, 16384, [10.0]),                 # a smaller launch: ignored
        (gemv, 1015808, [30000.0, 3000.0]),    # the fused launch, two instances
        (gemm, 819200, [400000.0]),
        (gemm, 65536, [9.0])])
    _write_counters(tmp_path / "W", "WRITE_SIZE", [
        (neg, 1 << 20, [probe_kib]),
        (gemv, 1015808, [100.0]),
        (gemm, 819200, [200000.0])])
    bench.summarize_pmc(str(tmp_path / "F"), str(tmp_path / "W"))
    kv = {}
    for ln in (tmp_path / "decode.txt").read_text().splitlines():
        if ln and not ln.startswith("#"):
            k, v = ln.split(None, 1)
            kv[k] = v
    assert float(kv["fetch_scale"]) == pytest.approx(2.0)
    assert float(kv["write_scale"]) == pytest.approx(1.0)
    assert int(kv["grid_threads"]) == 1015808
    assert float(kv["traffic_bytes_per_launch"]) == pytest.approx(33000 * 1024 * 2 + 100 * 1024)
    assert kv["source_hash"] == bench.kernel_source_hash()
    assert bench.stored_traffic("decode") == pytest.approx(33000 * 1024 * 2 + 100 * 1024)
    assert bench.stored_traffic("prefill") == pytest.approx(400000 * 1024 * 2 + 200000 * 1024)


def test_stored_traffic_is_null_for_other_sources(tmp_path, monkeypatch):
    p = tmp_path / "c.txt"
    p.write_text("source_hash 0000000000000000\ntraffic_bytes_per_launch 1.0\n")
    monkeypatch.setattr(bench, "COUNTERS", {"decode": (p, "gemv", "x")})
    assert bench.stored_traffic("decode") is None


def test_summarize_trace_groups_by_shape(tmp_path, monkeypatch):
    d = tmp_path / "T"
    d.mkdir()
    with open(d / "bench_kernel_stats.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                    "MaxNs", "StdDev"])
        w.writerow(["ternary::gemv_stream_kernel<false, false, 1, false>(x)", 3, 60000, 20000,
                    100, 19000, 21000, 0])
    with open(d / "bench_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Grid_Size_X", "Grid_Size_Y", "Workgroup_Size_X",
                    "Start_Timestamp", "End_Timestamp"])
        for t0, dt in ((0, 19000), (50000, 21000), (90000, 20000)):
            w.writerow(["ternary::gemv_stream_kernel<false, false, 1, false>(x)", 1015808, 1,
                        1024, t0, t0 + dt])
    out = tmp_path / "trace.txt"
    monkeypatch.setattr(bench, "TRACE_FILE", out)
    bench.summarize_trace(str(d))
    text = out.read_text()
    assert "grid=1015808 wg=1024" in text
    line = [ln for ln in text.splitlines() if "grid=1015808" in ln][0]
    calls, median, mean = line.split()[:3]
    assert int(calls) == 3 and float(median) == pytest.approx(20.0) and float(mean) == pytest.approx(20.0)


def test_summarize_mfma_relates_gemm_to_probe(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "MFMA_FILE", tmp_path / "mfma.txt")
    gemm = "ternary::dma::gemm_dma_kernel<false, false, Cfg<256, 128, 4, 1, 4, 2> >(BigBatch)"
    probe = "(anonymous namespace)::probe_mfma_kernel(int, float*)"
    wg = 2048
    iters = bench.PROBE_ITERS[wg]
    flops = wg * 4 * 4 * 16384 * iters
    d1, d2 = tmp_path / "A", tmp_path / "B"
    d1.mkdir()
    d2.mkdir()
    with open(d1 / "bench_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        rows = [(1, gemm, 819200, {"SQ_VALU_MFMA_BUSY_CYCLES": [300.0, 300.0],
                                   "GRBM_GUI_ACTIVE": [1000.0],
                                   "SQ_INSTS_VALU_MFMA_MOPS_BF16": [2.0e9]}),
                (2, gemm, 4096, {"SQ_VALU_MFMA_BUSY_CYCLES": [1.0], "GRBM_GUI_ACTIVE": [1.0]}),
                (3, probe, wg * 256, {"SQ_VALU_MFMA_BUSY_CYCLES": [800.0],
                                      "GRBM_GUI_ACTIVE": [1000.0],
                                      "SQ_INSTS_VALU_MFMA_MOPS_BF16": [flops / 512]})]
        for did, k, grid, cs in rows:
            for c, vs in cs.items():
                for v in vs:
                    w.writerow({c2: 0 for c2 in COLS} | {
                        "Dispatch_Id": did, "Kernel_Name": k, "Grid_Size": grid,
                        "Counter_Name": c, "Counter_Value": v})
    with open(d2 / "bench_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        for c, v in (("SQ_LDS_BANK_CONFLICT", 10.0), ("SQ_LDS_IDX_ACTIVE", 400.0)):
            w.writerow({c2: 0 for c2 in COLS} | {"Dispatch_Id": 1, "Kernel_Name": gemm,
                                                 "Grid_Size": 819200, "Counter_Name": c,
                                                 "Counter_Value": v})
        w.writerow({c2: 0 for c2 in COLS} | {"Dispatch_Id": 3, "Kernel_Name": probe,
                                             "Grid_Size": wg * 256,
                                             "Counter_Name": "SQ_LDS_IDX_ACTIVE",
                                             "Counter_Value": 0.0})
    bench.summarize_mfma(str(d1), str(d2))
    kv = {}
    for ln in (tmp_path / "mfma.txt").read_text().splitlines():
        if ln and not ln.startswith("#"):
            k, v = ln.split(None, 1)
            kv[k] = v
    assert float(kv["gemm_mfma_busy_per_gui"]) == pytest.approx(0.6)
    assert float(kv["probe_mfma_busy_per_gui"]) == pytest.approx(0.8)
    assert float(kv["gemm_mfma_busy_vs_probe"]) == pytest.approx(0.75)
    assert float(kv["probe_mfma_flops"]) == pytest.approx(flops)
    assert float(kv["probe_flops_issued"]) == pytest.approx(flops)
    assert float(kv["gemm_mfma_flops"]) == pytest.approx(1.024e12)
    assert float(kv["gemm_lds_bank_conflict_per_active"]) == pytest.approx(0.025)
    assert bench.stored_mfma() == pytest.approx(0.75)


def test_summarize_valu_takes_the_fused_launch(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "VALU_FILE", tmp_path / "valu.txt")
    gemv = "ternary::(anonymous namespace)::gemv_f4_kernel<false, 0, 1>(ternary::(anonymous namespace)::F4Batch)"
    d = tmp_path / "V"
    d.mkdir()
    with open(d / "bench_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=COLS)
        w.writeheader()
        for i, (grid, busy, wait, life) in enumerate([(884736, 40.0, 30.0, 60.0),
                                                      (884736, 36.0, 26.0, 56.0),
                                                      (65536, 5.0, 1.0, 100.0)]):
            for name, v in (("VALUBusy", busy), ("SQ_WAIT_INST_ANY", wait),
                            ("SQ_WAVE_CYCLES", life), ("SQ_ACTIVE_INST_ANY", life / 4)):
                w.writerow({c: 0 for c in COLS} | {"Dispatch_Id": i + 1, "Kernel_Name": gemv,
                                                   "Grid_Size": grid, "Counter_Name": name,
                                                   "Counter_Value": v})
    bench.summarize_valu(str(d))
    kv = {}
    for ln in (tmp_path / "valu.txt").read_text().splitlines():
        if ln and not ln.startswith("#"):
            k, v = ln.split(None, 1)
            kv[k] = v.split()[0]
    assert int(kv["grid_threads"]) == 884736           # the larger launch only
    assert float(kv["VALUBusy"]) == pytest.approx(38.0)
    assert float(kv["wait_share"]) == pytest.approx(28.0 / 58.0, rel=1e-3)
    assert float(kv["issue_share"]) == pytest.approx(0.25, rel=1e-3)


def test_summarize_workload_labels_projections(tmp_path, monkeypatch):
    # dispatches run projection by projection (WORKLOAD_REPS + 1 each); a
    # split-K reduce belongs to the GEMM before it; pack/tile kernels are left out
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    cols = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    n = bench.WORKLOAD_REPS + 1
    gemm = "void ternary::dma::gemm_dma_kernel<false, 128, ternary::dma::Cfg<128, 16> >(ternary::dma::BigBatch)"
    red = "void ternary::dma::gemm_split_reduce<false, true, X>(float4 const*)"
    for counter, scale in (("FETCH_SIZE", 1), ("WRITE_SIZE", 2)):
        d = tmp_path / counter
        d.mkdir()
        with open(d / "bench_counter_collection.csv", "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=cols)
            w.writeheader()
            i = 1
            rows = [("ternary::tile_kernel(x)", 5, 999.0),
                    ("at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>", 7,
                     (bench.COPY_PROBE_BYTES / 1024) / (2 if counter == "FETCH_SIZE" else 1))]
            for shape, grid in (("up", 100), ("down", 70)):
                for _ in range(n):
                    rows.append((gemm, grid, 1000.0 * scale))
                    rows.append((red, 3, 10.0))
            for k, g, v in rows:
                w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Grid_Size": g,
                            "Counter_Name": counter, "Counter_Value": v})
                i += 1
    bench.summarize_workload("27b_m64", [tmp_path / "FETCH_SIZE", tmp_path / "WRITE_SIZE"])
    text = (tmp_path / "profiles" / "gemm_dma_27b_m64_counters.txt").read_text()
    lines = [ln for ln in text.splitlines() if ln.startswith("[")]
    assert len(lines) == 4, lines
    assert lines[0].startswith("[up] dma::gemm_dma_kernel") and f"n={n}" in lines[0]
    assert lines[1].startswith("[up] dma::gemm_split_reduce")
    assert lines[2].startswith("[down] dma::gemm_dma_kernel") and "grid=70" in lines[2]
    assert lines[3].startswith("[down] dma::gemm_split_reduce")
    assert "tile_kernel" not in text
    # 1000 KiB fetched (scale 2) + 2000 KiB written (scale 1) per dispatch
    assert f"traffic_bytes {4000 * 1024}" in lines[0]


def test_summarize_workload_few_token_fused(tmp_path, monkeypatch):
    # the 16-token fused step: few-token GEMM launches and their K-slice
    # reduce, named after the kernel family that runs it
    monkeypatch.setattr(bench, "ROOT", tmp_path)
    cols = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    n = bench.WORKLOAD_REPS + 1
    few = "void ternary::(anonymous namespace)::few_kernel<false, 0, 16, 1, 1>(ternary::(anonymous namespace)::FewBatch)"
    red = "void ternary::(anonymous namespace)::few_reduce<false, true>(ternary::(anonymous namespace)::FewReduceBatch)"
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        d = tmp_path / counter
        d.mkdir()
        with open(d / "bench_counter_collection.csv", "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=cols)
            w.writeheader()
            rows = [("at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>", 7,
                     (bench.COPY_PROBE_BYTES / 1024) / (2 if counter == "FETCH_SIZE" else 1))]
            for _ in range(n):
                rows += [(few, 270336, 100.0), (red, 16384, 5.0)]
            for i, (k, g, v) in enumerate(rows, 1):
                w.writerow({"Dispatch_Id": i, "Kernel_Name": k, "Grid_Size": g,
                            "Counter_Name": counter, "Counter_Value": v})
    bench.summarize_workload("7b_fused_m16", [tmp_path / "FETCH_SIZE", tmp_path / "WRITE_SIZE"])
    text = (tmp_path / "profiles" / "gemm_few_7b_fused_m16_counters.txt").read_text()
    lines = [ln for ln in text.splitlines() if ln.startswith("[")]
    assert len(lines) == 2, lines
    assert lines[0].startswith("[fused step] few_kernel") and f"n={n}" in lines[0]
    assert lines[1].startswith("[fused step] few_reduce")
    assert "alg_bytes_per_step" in text
