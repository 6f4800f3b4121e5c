"""Host-side checks of the benchmark's contract (no GPU): the single-GPU guard,
and the reading of the committed HBM-traffic summary that fills
roofline.traffic (present only while the attention source is the one the
counters were taken with)."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402  (imports nothing from torch or the library at module level)


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def _tree(tmp_path, source: bytes, sha: str, traffic="8110119657"):
    (tmp_path / "profiles").mkdir()
    csrc = tmp_path / "compressed_kv_cache_kvc_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "attend.hip").write_bytes(source)
    (tmp_path / "profiles" / "traffic_attend_kernel_demo.md").write_text(
        "# demo\n\n- read bytes per launch: 1\n"
        f"- traffic bytes per launch: {traffic}\n- attend.hip sha256: `{sha}`\n")


def test_traffic_summary_parsed_only_for_the_matching_source(tmp_path, monkeypatch):
    src = b"// some kernel source\n"
    _tree(tmp_path, src, hashlib.sha256(src).hexdigest())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("demo") == 8110119657
    assert bench.measured_traffic("other") is None             # no summary for that workload
    (tmp_path / "compressed_kv_cache_kvc_amd" / "csrc" / "attend.hip").write_bytes(src + b"// edited\n")
    assert bench.measured_traffic("demo") is None              # counters no longer describe the source


def test_committed_streaming_summary_matches_the_attention_source():
    value = bench.measured_traffic("streaming")
    if value is None:
        pytest.fail("profiles/traffic_attend_kernel_streaming.md is missing or was taken with another attend.hip")
    # at least the algorithmic bytes of a mean streaming launch (queries, codes,
    # metadata, ids, centre tables, outputs): about 6.12 GB
    assert value >= 6.0e9
