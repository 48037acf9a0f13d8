"""Host-side behaviour of bench.py: the one-GPU guard and the validity
check of the stored rocprofv3 counter figures."""
import hashlib
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_message():
    """--gpus N > 1 stops before any device work, with status 2 and a message."""
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def test_profile_entry_follows_source_hash(tmp_path, monkeypatch):
    """A counter entry counts only while its sources hash to the stored
    value: a changed source turns the figures into None."""
    src = tmp_path / "k.hip"
    src.write_bytes(b"kernel v1\n")
    (tmp_path / "profiles").mkdir()
    ent = {"sources": ["k.hip"], "sha256": hashlib.sha256(b"kernel v1\n").hexdigest(),
           "fetch_bytes": 100, "write_bytes": 20, "mfma": {"util_pct": {"k": 1.0}}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps({"k": ent}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic("k") == 120
    assert bench.measured_mfma("k") == {"util_pct": {"k": 1.0}}
    assert bench.measured_traffic("absent") is None
    src.write_bytes(b"kernel v2\n")
    assert bench.measured_traffic("k") is None
    assert bench.measured_mfma("k") is None
