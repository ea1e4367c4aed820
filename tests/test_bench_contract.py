"""The bench script's contract: one JSON line with the required fields (GPU), and a
clear refusal of more than one GPU (CPU, before anything touches a GPU)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""


def test_cpu_baseline_legs_time_the_oracle():
    """The bench's host baselines run the oracle on the CPU: on a bounded slot sample in
    this process, and over contiguous slot ranges in fresh worker processes; both count
    the real elements of the slots they cover (rank 1 of the tiny set holds the whole
    [200, 300] param: 60,000 real elements in 6 slots)."""
    import bench
    import synth
    w = synth.get("tiny")
    rate, valid, dt = bench.cpu_baseline(w, 1, 6, steps=1)
    assert valid == 200 * 300 and dt > 0 and rate == pytest.approx(valid / dt)
    rate_p, valid_p, dt_p, used = bench.cpu_baseline_parallel(w, 1, 6, 2, steps=1)
    assert used == 2 and valid_p == 200 * 300 and rate_p == pytest.approx(valid_p / dt_p)
    # a sample starting mid-shard: slots 3..5 of rank 1 (block row 1 of [200, 300]: 72 rows)
    _, valid_tail, _ = bench.cpu_baseline(w, 1, 3, steps=1, first=3)
    assert valid_tail == 72 * 300


@pytest.mark.gpu
def test_bench_line_has_the_contract_fields():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "dense", "--steps", "3",
                        "--warmup", "1", "--no-cpu-baseline"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
                "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1 and d["value"] > 0
    assert d["config"]["workload"] == "dense_layer_set"
    rl = d["roofline"]
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in rl, key
    assert rl["bound"] == "hbm" and rl["peak"] == 8000.0 and rl["unit"] == "GB/s"
    assert abs(rl["frac"] - rl["achieved"] / rl["peak"]) < 1e-12
    c = d["ceiling"]  # the same-run copy ceiling, the second denominator
    assert c["copy_gbs"] > 0 and abs(c["update_vs_copy"] - rl["achieved"] / c["copy_gbs"]) < 1e-9
