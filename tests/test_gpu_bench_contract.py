"""bench.py end to end on the GPU with a small workload: one JSON line whose
fields and types follow the benchmark contract (metric, value, roofline with
the kernel's measured bandwidth, CPU oracle baseline, ceiling)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


def test_bench_line_follows_the_contract():
    d = run_bench("--workload", "tiny_gpt_d32", "--steps", "5", "--warmup", "2", "--cpu-seconds", "0.4")
    for key, typ in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                     ("dtype", str), ("data", str), ("config", dict), ("roofline", dict), ("cpu_baseline", dict)):
        assert isinstance(d[key], typ), key
    assert d["vs_baseline"] is None
    assert d["n_gpus"] == 1 and d["steps"] == 5 and d["warmup"] == 2
    assert d["unit"] == "Gparams/s" and d["higher_is_better"] is True and d["data"] == "synthetic"
    assert d["config"]["workload"] == "tiny_gpt_d32" and d["config"]["launch"] == "stream"
    assert d["config"]["placement"] == "spread" and d["config"]["arena_bytes"] > 0
    assert abs(d["value"] - d["config"]["shard_elems"] / (d["ms_per_step"] * 1e-3) / 1e9) <= 1e-3 * d["value"] + 1e-3
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["achieved"] > 0 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert "traffic" in rf
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["unit"] == "Gparams/s" and cb["value"] > 0 and cb["cores"] >= 1
    assert isinstance(cb["sample"], str) and cb["sample"]
    assert d["ceiling"]["achieved"] > 0 and d["rebuild"]["achieved"] > 0
    # the read-only settle passes ran before the warm-up steps, for about the default two seconds
    assert d["settle"]["passes"] > 0 and 1.9 <= d["settle"]["seconds"] <= 10.0


def test_bench_graph_mode_line():
    # --graph times replays of the recorded step; the line keeps the contract
    # and names the launch mode and the scheduled kernel.
    d = run_bench("--workload", "tiny_gpt_d32", "--steps", "20", "--warmup", "3", "--no-cpu-baseline", "--graph")
    assert d["config"]["launch"] == "graph"
    assert d["roofline"]["kernel"].endswith(",scheduled>") and d["roofline"]["traffic"] is None
    assert d["value"] > 0 and d["ms_per_step"] > 0 and "cpu_baseline" not in d


def test_bench_packed_placement_line():
    d = run_bench("--workload", "tiny_gpt_d32", "--steps", "10", "--warmup", "2", "--no-cpu-baseline",
                  "--placement", "packed")
    assert d["config"]["placement"] == "packed" and d["config"]["arena_bytes"] == 0
    assert d["roofline"]["traffic"] is None and d["value"] > 0


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "8"], capture_output=True,
                       text=True, timeout=60, cwd=ROOT)
    assert r.returncode == 2 and r.stdout == ""
