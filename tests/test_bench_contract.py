"""bench.py's output contract: one JSON line with the fields the benchmark
line is read by, a roofline entry and the oracle's CPU baseline; a request
for more than one GPU is refused with a message (this build measures one)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_default_workload_is_the_largest_config_with_the_table():
    """With no flags the headline is the batched varlen B=64 config (the
    largest that fits one GPU) and every named config is timed beside it."""
    sys.path.insert(0, ROOT)
    import bench
    import workloads

    old = sys.argv
    sys.argv = ["bench.py"]
    try:
        args = bench.parse()
    finally:
        sys.argv = old
    assert workloads.CONFIGS[args.config].name == "gqa_b64_h32x8_d128_varlen16k"
    assert args.table and args.gpus == 1 and args.splits == 0 and args.out_dtype == "f32"
    assert bench.fused_merge(64, 8, 5, 256) == "two kernels"
    assert bench.fused_merge(1, 8, 24, 256) == "fused"
    assert bench.fused_merge(1, 8, 1, 256) == "none (one split)"


@pytest.mark.gpu
def test_bench_prints_one_json_line_with_the_contract_fields():
    r = subprocess.run([sys.executable, BENCH, "--config", "0", "--steps", "5", "--warmup", "2",
                        "--cpu-seconds", "0.5", "--no-table"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["unit"] == "GB/s" and d["value"] > 0 and d["higher_is_better"] is True
    assert d["config"]["workload"] == "mha_b1_h8_d64_l1024"
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
