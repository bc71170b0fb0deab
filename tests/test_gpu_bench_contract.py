"""bench.py's output line on a short run of the default workload: one JSON
line with the fields its readers depend on, the roofline object for the step
kernel and the oracle's CPU baseline."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu


def test_default_bench_line_has_every_field():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--steps", "8", "--warmup", "2",
                        "--cpu-seconds", "1"], cwd=root, capture_output=True, text=True, timeout=170)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [x for x in r.stdout.splitlines() if x.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 8 and d["warmup"] == 2 and d["value"] > 0
    assert d["higher_is_better"] is True and d["data"] == "synthetic"
    # the default is the largest single-GPU workload, timed after its bulk first step and the warm-up
    assert d["config"]["workload"] == "paged_mixed_4k-64k_20pct"
    assert d["config"]["window_steps"] == [3, 11]
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0 < rf["frac"] < 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert "traffic" in rf
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
    assert cb["one_core"]["cores"] == 1 and cb["one_core"]["value"] > 0


@pytest.mark.parametrize("mode", ["--prefill", "--snapkv"])
def test_prompt_call_bench_lines(mode):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), mode, "--steps", "8", "--warmup", "2",
                        "--cpu-seconds", "1"], cwd=root, capture_output=True, text=True, timeout=170)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [x for x in r.stdout.splitlines() if x.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])
    assert d["n_gpus"] == 1 and d["steps"] == 8 and d["value"] > 0
    assert d["config"]["entry_point"] == ("h2o_prefill_scores" if mode == "--prefill" else "h2o_snapkv_select")
    rf = d["roofline"]
    if mode == "--prefill":
        # every causal score costs two exponentials and ~12 ALU operations over the two passes:
        # the vector ALU binds, above HBM (q and K read once) and the matrix cores
        assert rf["bound"] == "alu" and rf["unit"] == "T lane-ops/s" and 0 < rf["frac"] < 1
        assert 0 < rf["hbm_frac"] < rf["frac"] and 0 < rf["mfma_frac"] < rf["frac"]
    else:
        # SnapKV scores only its window rows: reading K once takes longer than their ALU work
        assert rf["bound"] == "hbm" and rf["peak"] == 8000.0 and 0 < rf["frac"] < 1
        assert 0 < rf["alu_frac"] < rf["frac"] and 0 < rf["mfma_frac"] < rf["frac"]
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert d["cpu_baseline"]["kind"] == "oracle" and d["cpu_baseline"]["value"] > 0
