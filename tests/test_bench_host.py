"""Host-side logic of bench.py that needs no GPU: the roofline bound of the
prompt calls, the source hashes the counter summaries are tied to, and the
counter summarizer on a synthetic rocprofv3 CSV."""
import csv
import types

import bench


def test_call_roofline_picks_the_slower_resource():
    # 200 MB at 8 TB/s = 25 us against 10 GFLOP at 2.5 PFLOP/s = 4 us: HBM
    r = bench.call_roofline(200e6, 10e9, 100e-6, "x")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["frac"] - 0.25) < 1e-9 and abs(r["achieved"] - 2000.0) < 1e-6
    assert abs(r["mfma_frac"] - 0.04) < 1e-9
    # 1 MB (0.125 us) against 100 GFLOP (40 us): the matrix cores
    r = bench.call_roofline(1e6, 100e9, 80e-6, "x")
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert abs(r["frac"] - 0.5) < 1e-9 and abs(r["hbm_frac"] - 0.125e-6 / 80e-6) < 1e-4


def test_call_roofline_alu_bound():
    # 1 MB (0.125 us) and 1 GFLOP (0.4 us) against 3.93e9 lane-ops (100 us at 39.3 T/s)
    ops = bench.PEAK_VALU_TOPS * 1e12 * 100e-6
    r = bench.call_roofline(1e6, 1e9, 200e-6, "x", alu_ops=ops)
    assert r["bound"] == "alu" and r["unit"] == "T lane-ops/s" and abs(r["peak"] - 39.32) < 0.01
    assert abs(r["frac"] - 0.5) < 1e-9 and "hbm_frac" in r and "mfma_frac" in r
    assert abs(bench.PEAK_VALU_TOPS * 2 * 2 - 157.3) < 0.1  # the fp32 vector peak: FMA x packed


def test_source_hashes_cover_their_own_kernels():
    assert set(bench.STEP_SRCS) & set(bench.PROMPT_SRCS) == {"h2o_internal.h", "h2o_device.h"}
    assert "h2o_prefill.hip" not in bench.STEP_SRCS and "h2o_prefill.hip" in bench.PROMPT_SRCS
    assert bench.kernel_hash() != bench.kernel_hash(prompt=True)


def test_summarize_pmc_means_over_the_timed_window(tmp_path, capsys):
    f = tmp_path / "c.csv"
    with open(f, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        for i in range(10):  # launches 0..9; the timed window is the last steps x layers = 4
            w.writerow(["h2o::step_kernel<...>", "SQ_WAVE_CYCLES", 100 + i])
            w.writerow(["h2o::step_kernel<...>", "SQ_WAIT_ANY", 50])
            w.writerow(["other_kernel", "SQ_WAVE_CYCLES", 1e9])
    args = types.SimpleNamespace(steps=2, layers=2, summarize_kernel="step_kernel", summarize_trace=None,
                                 summarize_counters=None, summarize_pmc=str(f), summarize_bench_line=None)
    bench.summarize(args)
    out = capsys.readouterr().out
    assert f"kernel_source_sha256_16: {bench.kernel_hash()}" in out
    assert "SQ_WAVE_CYCLES: timed-window mean 107.5 per launch (10 launches)" in out
    assert "SQ_WAIT_ANY / SQ_WAVE_CYCLES: 0.465" in out


def test_bench_refuses_more_than_one_gpu():
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], cwd=root,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_default_window_is_the_paged_workload_after_its_bulk_step():
    """With no flags the bench measures the paged mixed-length workload (the
    largest single-GPU one); its window starts after the bulk first step and the
    warm-up, whatever --steps / --warmup say."""
    from kv_cache_eviction_h2o_amd import workloads as WL
    args = bench_args([])
    assert args.workload == WL.PAGED_MIXED.name
    w = WL.PAGED_MIXED
    assert bench.bench_window(w) == (60, 4, 5)
    assert bench.bench_window(w, 20, 5) == (20, 5, 6)
    assert bench.bench_window(WL.OPT_LAYER, 20, 5) == (20, 5, 512)
    # contiguous traces keep the window inside them
    assert bench.bench_window(WL.OPT_LAYER, 600, 16) == (600, 16, 424)
    # every workload bench.py accepts has a default window
    for wl in WL.ALL + WL.VARIANTS:
        K, W, s0 = bench.bench_window(wl)
        assert K >= 1 and s0 >= W


def bench_args(argv):
    import sys
    saved = sys.argv
    try:
        sys.argv = ["bench.py", *argv]
        return bench.parse()
    finally:
        sys.argv = saved


def test_summary_records_window_and_traffic_scales_to_the_line(tmp_path, capsys, monkeypatch):
    """The counter summary keeps the profiled window's algorithmic bytes; a bench
    line on another window reports the same measured/algorithmic ratio applied
    to its own algorithmic bytes."""
    import json
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    for path, name, val in ((fetch, "FETCH_SIZE", 500.0), (write, "WRITE_SIZE", 100.0)):
        with open(path, "w", newline="") as fh:
            cw = csv.writer(fh)
            cw.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
            cw.writerow(["copyBuffer", name, 524288.0 if name == "FETCH_SIZE" else 1048576.0])
            for _ in range(3):
                cw.writerow(["h2o::step_kernel<...>", name, val])
    line = tmp_path / "line.json"
    line.write_text("noise\n" + json.dumps({"steps": 3, "config": {"workload": "paged_mixed_4k-64k_20pct",
                                                                    "layers": 1, "window_steps": [6, 9]},
                                            "algorithmic_bytes_per_launch": 1000 * 1024}) + "\n")
    args = types.SimpleNamespace(steps=None, layers=0, summarize_kernel="step_kernel", summarize_trace=None,
                                 summarize_counters=[str(fetch), str(write)], summarize_pmc=None,
                                 summarize_bench_line=str(line))
    bench.summarize(args)
    out = capsys.readouterr().out
    # FETCH_SIZE counts half the bytes read (x2), WRITE_SIZE all of them: 1100 KiB per launch
    assert "hbm_bytes_per_launch: 1.126400e+06" in out
    assert "window_steps: [6, 9]" in out and "measured / algorithmic: 1.1000" in out
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "h2o_step_kernel_paged_mixed_4k-64k_20pct_counters.md").write_text(out)
    monkeypatch.setattr(bench, "PROFILES", str(prof))
    from kv_cache_eviction_h2o_amd import workloads as WL
    tr = bench.traffic_from_profiles(WL.PAGED_MIXED, 2000.0)
    assert abs(tr["ratio"] - 1.1) < 1e-9 and abs(tr["bytes"] - 2200.0) < 1e-6 and tr["window"] == [6, 9]


def test_snapkv_traffic_only_for_the_current_prompt_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.snapkv_traffic("w") is None  # no summary
    f = tmp_path / "h2o_snapkv_kernels_w_counters.md"
    f.write_text(f"kernel_source_sha256_16: {bench.kernel_hash(prompt=True)}\nhbm_bytes_per_call: 8.5e+07\n")
    assert bench.snapkv_traffic("w") == 8.5e7
    f.write_text(f"kernel_source_sha256_16: {bench.kernel_hash()}\nhbm_bytes_per_call: 8.5e+07\n")
    assert bench.snapkv_traffic("w") is None  # taken on other sources
