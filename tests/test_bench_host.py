"""Host-side checks of bench.py (no GPU): the one-GPU guard, the CPU oracle
baseline leg and the rule that counter traffic is reported only for the
kernel source it was measured on."""
import glob
import json
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from bf16_numerics_amd import workloads as W  # noqa: E402


def test_workload_choices_match_the_generators():
    assert set(bench.WORKLOAD_NAMES) == set(W.WORKLOADS)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("master,sr", [(True, True), (False, False)])
def test_cpu_baseline_runs_the_oracle_on_one_and_k_threads(master, sr):
    w = W.tiny()
    n = w.n
    rs = np.random.default_rng(0)
    P = torch.from_numpy(rs.normal(0, 0.02, n).astype(np.float32)).to(torch.bfloat16)
    st = {"P": P, "G": torch.from_numpy(rs.normal(0, 1e-3, n).astype(np.float32)).to(torch.bfloat16),
          "M": P.float() if master else None, "m": torch.zeros(n), "v": torch.zeros(n)}
    out = bench.cpu_baseline(torch, w, st, 0, 0.2, rounding_sr=sr)
    assert out["kind"] == "oracle" and out["unit"] == "Gparams/s"
    assert out["cores"] == bench.cpu_threads() >= 1
    assert out["value"] > 0 and out["single_thread_value"] > 0
    assert ("no master" in out["sample"]) == (not master)
    assert ("RNE" in out["sample"]) == (not sr)


def test_counter_traffic_is_reported_only_for_the_measured_source(tmp_path, monkeypatch):
    digest = bench.kernel_source_digest()
    assert len(digest) == 16
    rec = {"kernel_source_sha256_16": digest, "bytes_per_launch": 123}
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "adamw_update_wl_traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: digest)
    assert bench.measured_traffic("wl") == 123
    rec["kernel_source_sha256_16"] = "0" * 16
    (prof / "adamw_update_wl_traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("wl") is None
    assert bench.measured_traffic("missing") is None


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(ROOT, "profiles", "*_traffic.json"))))
def test_committed_counter_records_are_consistent(path):
    """Each stored counter record adds up: read + write bytes, 28 B per shard
    element for the update, counter bytes within 1% above the algorithmic
    ones, and the copy calibration it was scaled by."""
    rec = json.load(open(path))
    w = W.WORKLOADS[rec["workload"]]()
    begin, end = w.shard()
    assert rec["shard_elems"] == end - begin
    assert rec["algorithmic_bytes_per_launch"] == 28 * rec["shard_elems"]
    assert rec["bytes_per_launch"] == pytest.approx(rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"],
                                                    abs=2)
    ratio = rec["bytes_per_launch"] / rec["algorithmic_bytes_per_launch"]
    assert rec["traffic_over_algorithmic"] == pytest.approx(ratio, abs=1e-5)
    assert 1.0 <= ratio < 1.01
    cal = rec["copy_reference"]
    assert rec["fetch_scale"] == pytest.approx(cal["read_KiB"] / np.mean(cal["FETCH_SIZE_KiB"]), rel=1e-5)
    assert rec["write_scale"] == pytest.approx(cal["write_KiB"] / np.mean(cal["WRITE_SIZE_KiB"]), rel=1e-5)
    assert rec["read_bytes_per_launch"] == pytest.approx(
        np.mean(rec["update_FETCH_SIZE_KiB"]) * 1024 * rec["fetch_scale"], rel=1e-6)
    assert rec["write_bytes_per_launch"] == pytest.approx(
        np.mean(rec["update_WRITE_SIZE_KiB"]) * 1024 * rec["write_scale"], rel=1e-6)
    # the rebuild (6 B per element) and the three no-math probes (28, 14, 14 B)
    for part, per in [(rec["rebuild"], 6)] + [(rec["stream_mix"][k], b) for k, b in
                                              (("both", 28), ("reads_only", 14), ("writes_only", 14))]:
        assert part["algorithmic_bytes_per_launch"] == per * rec["shard_elems"]
        assert part["bytes_per_launch"] == pytest.approx(part["read_bytes_per_launch"] + part["write_bytes_per_launch"],
                                                         abs=2)
        assert part["over_algorithmic"] == pytest.approx(part["bytes_per_launch"] / part["algorithmic_bytes_per_launch"],
                                                         abs=1e-5)
        assert 0.999 <= part["over_algorithmic"] < 1.03
