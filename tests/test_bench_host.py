"""Host-side checks of bench.py (no GPU): the one-GPU contract and the
measured-traffic lookup."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_digest_ignores_comments_and_layout(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    src.write_text("int f(int x) {\n  return x + 1;  // one\n}\n/* block\n comment */\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setitem(bench.KERNEL_SOURCES, "probe", ["k.hip"])
    d0 = bench.sources_digest("probe")
    src.write_text("int f(int x) {   return x + 1; // another comment\n}\n")
    assert bench.sources_digest("probe") == d0
    src.write_text("int f(int x) { return x + 2; }\n")
    assert bench.sources_digest("probe") != d0

