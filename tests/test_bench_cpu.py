"""Host-side logic of bench.py that needs no GPU: the measured-traffic lookup
(counters count only for the kernel source and build flags they were taken
on) and the one-GPU contract."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from bit_quantized_attention_amd.csrc import build  # noqa: E402


def _entries():
    with open(bench.TRAFFIC_FILE) as f:
        return json.load(f)


def test_every_traffic_entry_matches_the_current_kernel():
    """Committed counter figures were taken on the sources and flags in the
    tree: each resolves to its bytes (a stale one would print null)."""
    for key, e in _entries().items():
        assert bench._traffic_for(key) == e["bytes_per_launch"], key
        assert os.path.exists(os.path.join(ROOT, e["summary"] if os.sep in e["summary"] else
                                           os.path.join("profiles", e["summary"]))), key


def test_traffic_goes_stale_with_the_build_flags(monkeypatch):
    key, e = next(iter(_entries().items()))
    src = os.path.basename(e["source"])
    monkeypatch.setitem(build.EXTRA, src, build.EXTRA.get(src, []) + ["-O2"])
    assert bench._traffic_for(key) is None


def test_traffic_goes_stale_with_the_source(tmp_path, monkeypatch):
    d = _entries()
    key = next(iter(d))
    d[key]["source_sha256"] = "0" * 64
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(d))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench._traffic_for(key) is None
    assert bench._traffic_for("no_such_kernel") is None


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
