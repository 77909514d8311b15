"""Host logic of bench.py (no GPU): the one-GPU guard, the counter-based traffic (scaling by the calibration copy,
the source-hash check) and the per-step algorithmic bytes at the benchmark workload's shapes."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from fixtures import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stdout


def _write_counters(dirname, counter, rows):
    os.makedirs(dirname, exist_ok=True)
    with open(os.path.join(dirname, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_scaled_by_the_calibration_copy(tmp_path, monkeypatch):
    """FETCH_SIZE reads half of a copy's bytes on this part, WRITE_SIZE all of them: each counter is scaled by
    known / counted for the copy, per dispatch of the kernel, and the summary is refused once the source changes."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    copy_kib = bench.COPY_PROBE_BYTES / 1024.0
    kernel = "void mtpd::(anonymous namespace)::k_team<10, 1>(mtpd::TeamArgs)"
    copy = "void rocclr::copyBuffer(...)"
    _write_counters(str(tmp_path / "f"), "FETCH_SIZE", [(kernel, 1000.0), (kernel, 3000.0), (copy, copy_kib / 2)] * 1)
    _write_counters(str(tmp_path / "w"), "WRITE_SIZE", [(kernel, 500.0), (kernel, 500.0), (copy, copy_kib)])

    class A:
        summarize_pmc = (str(tmp_path / "f"), str(tmp_path / "w"))
        kernel = "k_team"
        workload = "wl"
        cmd = "test"

    bench.summarize_pmc(A)
    t = bench.load_traffic("k_team", "wl")
    assert t is not None
    # fetch: mean 2000 KiB per dispatch, doubled by the copy's factor; write: 500 KiB, factor 1
    assert t["fetch_bytes_per_launch"] == pytest.approx(2000 * 1024 * 2.0)
    assert t["write_bytes_per_launch"] == pytest.approx(500 * 1024 * 1.0)
    assert t["hbm_bytes_per_launch"] == pytest.approx(2000 * 1024 * 2.0 + 500 * 1024)
    # a summary taken on another source is not used
    p = bench.traffic_file("k_team", "wl")
    text = open(p).read().replace(t["source_sha256_16"], "0" * 16)
    open(p, "w").write(text)
    assert bench.load_traffic("k_team", "wl") is None


def test_committed_traffic_summaries_parse():
    """Every committed traffic summary carries its JSON record with the kernel, workload and byte counts."""
    import glob
    files = glob.glob(os.path.join(ROOT, "profiles", "*.traffic.md"))
    assert files
    for p in files:
        text = open(p).read()
        start = text.index("<!-- traffic-json: ") + len("<!-- traffic-json: ")
        t = json.loads(text[start:text.index(" -->", start)])
        kernel, workload = os.path.basename(p)[: -len(".traffic.md")].split("__")
        assert t["kernel"] == kernel and t["workload"] == workload
        assert t["hbm_bytes_per_launch"] == pytest.approx(t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"])
        assert "Command" in text and "rocprofv3" in text


def test_step_bytes_at_the_benchmark_workload():
    """E4B, 16 rows of 8192 keys, one kv head: the cache bytes are K once per key of the full layer plus the 512-key
    sliding window (K = V, 256 dims of bf16), the logits row is 262144 fp32 per row, and the head rows are 128
    tokens x 256 dims of bf16 per distinct cluster."""
    shape = synth.E4B
    total, parts = bench.step_bytes(shape, 16, [8192] * 16, 460)
    assert parts["kv"] == 16 * 256 * 2 * (8192 + 512)
    assert parts["logits"] == 16 * 262144 * 4
    assert parts["head"] == 460 * 128 * 256 * 2
    assert parts["ids"] == 16 * 32 * 128 * 4
    # weights: 4 layers of q, o (1024 x 256), gate, up, down (1024 x 256) and norms, pre_projection (256 x 5120),
    # post_projection (2560 x 256), the centroids (2048 x 256) and output_norm, in bf16
    per_layer = (1024 * 256 * 2 + 1024 * 256 * 3) * 2 + (256 + 4 * 256) * 2
    assert parts["weights"] == 4 * per_layer + (256 * 5120 + 2560 * 256 + 2048 * 256 + 256) * 2
    assert total == sum(parts.values())
    # with two kv heads the cache bytes double and nothing else changes
    _, p2 = bench.step_bytes(synth.WORKLOADS["e4b_nkv2_b16_ctx8192_block4"].shape, 16, [8192] * 16, 460)
    assert p2["kv"] == 2 * parts["kv"] and p2["weights"] == parts["weights"]
