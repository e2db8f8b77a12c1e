"""bench.py's contract on the CPU: it refuses more than one GPU with a
message, its CPU baseline is the oracle timed on a bounded sample with the
fields the result line carries, and the committed traffic record is read
only while the sources hash to the value recorded with it."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_baseline_fields_on_the_tiny_workload():
    import bench
    from tact_inputs import WORKLOADS
    wl = WORKLOADS["tiny"]
    cb = bench.cpu_baseline(wl, 1, 2)
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s"
    assert cb["value"] > 0 and cb["cores"] >= 1
    assert "2 units" in cb["sample"] and wl.name in cb["sample"]
    assert cb["extrapolated_full_config_s"] >= 0
    json.dumps(cb)                      # the result line is one JSON object


def test_traffic_record_is_used_only_for_matching_sources(tmp_path, monkeypatch):
    import bench
    rec = bench.measured_traffic("ct32b")
    if rec is None:
        pytest.skip("the committed counter record was taken on other sources")
    assert rec["compress_bytes"] > 0 and rec["decompress_bytes"] > 0
    # a record whose hash differs from the sources is not used
    prof = tmp_path / "profiles"
    prof.mkdir()
    bad = dict(rec, source_sha256="0" * 64)
    (prof / "codec_ct32b_hbm_traffic.md").write_text("traffic-record: " + json.dumps(bad) + "\n")
    csrc = tmp_path / "kv_cache_compression_tact_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in os.listdir(os.path.join(ROOT, "kv_cache_compression_tact_amd", "csrc")):
        if f.endswith((".hip", ".cpp", ".h")):
            src = os.path.join(ROOT, "kv_cache_compression_tact_amd", "csrc", f)
            (csrc / f).write_bytes(open(src, "rb").read())
    monkeypatch.setattr(bench, "__file__", str(tmp_path / "bench.py"))
    assert bench.measured_traffic("ct32b") is None
