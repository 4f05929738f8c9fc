"""bench.py's JSON line on a small workload, eager and graph-replayed (needs an MI355X).

Each run is a child process (one GPU process at a time), short enough for a
test: the one-matrix workload with a few steps and no CPU baseline."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*extra):
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "single_256x512", "--steps", "20",
           "--warmup", "3", "--no-cpu-baseline", *extra]
    print("running:", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    return json.loads(r.stdout.strip().splitlines()[-1])


@pytest.mark.parametrize("graph", [False, True])
def test_bench_line(graph):
    line = run_bench(*(["--graph"] if graph else []))
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
                "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert key in line, key
    assert line["n_gpus"] == 1 and line["steps"] == 20 and line["warmup"] == 3
    assert line["unit"] == "matrices/s" and line["value"] > 0
    assert abs(line["value"] - 1.0 / (line["ms_per_step"] * 1e-3)) <= 1e-3 * line["value"]
    assert line["config"]["workload"] == "single_256x512" and line["config"]["graph"] is graph
    roof = line["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and 0 < roof["frac"] < 1
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert line["device"]["cus"] > 0 and line["device"]["peak_clock_mhz"] > 0
    print(f"graph={graph}: {line['ms_per_step']} ms per step on {line['device']}", flush=True)


def test_bench_adamw_route_line():
    """The adamw route's line on the 65 RMSNorm vectors: elements per second,
    an HBM roofline whose fraction is achieved / 8 TB/s."""
    cmd = [sys.executable, os.path.join(ROOT, "bench.py"), "--route", "adamw", "--workload", "adamw_llama_norms",
           "--steps", "20", "--warmup", "3", "--no-cpu-baseline"]
    print("running:", " ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["unit"] == "elements/s" and line["value"] > 0 and line["n_gpus"] == 1
    assert line["config"]["workload"] == "adamw_llama_norms"
    roof = line["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
