"""bench.py on the GPU, on the tiny workload: one JSON line with every field
of the benchmark contract (the step throughput, the roofline of the dominant
kernel, the copy ceiling and both oracle baselines)."""

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line():
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "5", "--warmup", "2",
           "--cpu-seconds", "0.6"]
    print("\n[bench tiny]", " ".join(cmd[1:]), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [line for line in r.stdout.splitlines() if line.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["unit"] == "params/s" and d["dtype"] == "f32" and d["vs_baseline"] is None
    assert d["config"]["workload"].startswith("tiny") and "model" not in d["config"]
    assert d["value"] == pytest.approx(d["config"]["shard_params"] / (d["ms_per_step"] * 1e-3), rel=1e-9)
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert roof["achieved"] > 0 and roof["frac"] == pytest.approx(roof["achieved"] / roof["peak"], abs=1e-4)
    S = d["config"]["shard_params"]
    fused = d["config"]["unpack"] == "fused into AdamW"
    assert fused                                   # the default path
    assert roof["algorithmic_bytes_per_launch"] == 28 * S + 2 * S    # the tiny shard has no padding
    assert roof["timed_launches"] >= 1 and "note" not in roof        # one launch per update call
    parallel = len(os.sched_getaffinity(0)) > 1
    for base in ("cpu_baseline", "cpu_baseline_parallel") if parallel else ("cpu_baseline",):
        b = d[base]
        assert b["kind"] == "oracle" and b["unit"] == "params/s" and b["value"] > 0 and b["cores"] >= 1
        assert b["host_cpus"] >= b["affinity_cpus"] >= b["cores"]
        assert b["sample"]
    assert d["cpu_baseline"]["cores"] == 1
    assert d["copy_ceiling"]["copied_correctly"] is True and d["copy_ceiling"]["GBps"] > 0
    print(f"[bench tiny] {d['ms_per_step']:.4f} ms per step", flush=True)


@pytest.mark.parametrize("mode,kernels,update_bytes", [
    ("--state-arrays", {"pack_sqnorm", "adamw", "unpack"}, 28),
    ("--separate-unpack", {"pack_sqnorm", "adamw", "unpack"}, 28),
    ("--flat", {"sqnorm", "adamw"}, 28),
])
def test_bench_modes(mode, kernels, update_bytes):
    """The other step forms of the benchmark on the tiny workload: the line's
    phases and the update's bytes per element."""
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "tiny", "--steps", "3", "--warmup", "1",
           "--no-cpu-baseline", "--no-copy-ceiling", mode]
    print(f"\n[bench tiny {mode}]", flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    assert set(d["kernels"]) == kernels
    S = d["config"]["shard_params"]
    assert d["roofline"]["algorithmic_bytes_per_launch"] == update_bytes * S
    if mode == "--state-arrays":
        assert d["config"]["state"] == "three arrays" and d["config"]["unpack"] == "separate"
